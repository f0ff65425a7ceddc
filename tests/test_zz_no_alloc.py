"""The NVFP4 quantizer entry point that allocates nothing (its dynamic-mode
partial maxima live in the library's static device scratch) against the
workspace entry point, through the C ABI: codes, block scales and the global
scale bit-identical, on two calls in a row -- the second on a smaller tensor
with a smaller maximum, so that anything left over in the shared scratch from
the first call would show up as a wrong global scale.
"""
import numpy as np
import pytest

import oracle
from microscaling_quantized_dit_amd import inputs

pytestmark = pytest.mark.gpu


def _run_both(mxq, x, layout):
    import torch
    R, C = x.shape
    q_ref, s_ref, g_ref = mxq.quantize_nvfp4(x, scale_layout=layout)
    out = (torch.full((R, C // 2), 0x5A, dtype=torch.uint8, device=x.device),
           torch.full((R, C // 16), 0x5A, dtype=torch.uint8, device=x.device),
           torch.full((1,), -1.0, dtype=torch.float32, device=x.device))
    q, s, g = mxq.quantize_nvfp4_noalloc(x, out, scale_layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(q, q_ref) and torch.equal(s, s_ref) and torch.equal(g, g_ref)
    return q, s, g


@pytest.mark.parametrize("layout", ["row", "tiled"])
def test_noalloc_matches_workspace_entry_point(mxq, layout):
    import torch
    big = inputs.flux_activation(4608, 3072, seed=5, stream="noalloc/big")     # 0.1% outliers x50
    small = inputs.tiny_activation(128, 256)                                  # amax far below big's
    for bits in (big, small):
        x = inputs.to_torch(bits, "cuda")
        q, s, g = _run_both(mxq, x, layout)
        # the global scale is the oracle's (over the whole tensor) in both calls
        assert float(g.item()) == float(oracle.nvfp4_global_scale(bits))
    # the smaller call's codes and scales equal the oracle's too (row-major order)
    if layout == "row":
        rq, rs, rg = oracle.quantize_nvfp4(small)
        assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(s.cpu().numpy(), rs)
        assert float(g.item()) == float(rg)



def test_noalloc_static_scale(mxq):
    """Static mode needs no scratch and gives the workspace entry point's bits."""
    import torch
    bits = inputs.flux_activation(256, 512, seed=6, stream="noalloc/static")
    x = inputs.to_torch(bits, "cuda")
    gs = torch.tensor([0.0625], dtype=torch.float32, device="cuda")
    q_ref, s_ref, g_ref = mxq.quantize_nvfp4(x, global_scale=gs)
    out = (torch.empty_like(q_ref), torch.empty_like(s_ref), torch.empty_like(g_ref))
    q, s, g = mxq.quantize_nvfp4_noalloc(x, out, global_scale=gs)
    torch.cuda.synchronize()
    assert torch.equal(q, q_ref) and torch.equal(s, s_ref) and torch.equal(g, g_ref)
