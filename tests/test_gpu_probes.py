"""The measurement probes compute what they claim: the MXFP8 GEMM with every A
stage DMA'd twice (the fusion lower-bound probe) returns the library GEMM's bits,
and the streaming copy copies."""
import pytest

from microscaling_quantized_dit_amd import inputs

pytestmark = pytest.mark.gpu


def test_gemm_a_twice_equals_the_gemm(mxq):
    import torch
    from microscaling_quantized_dit_amd import probes
    M, N, K = 1024, 768, 1536
    x = inputs.to_torch(inputs.flux_activation(M, K, seed=4, stream="probe/x"), "cuda")
    w = inputs.to_torch(inputs.weight(N, K, seed=4, stream="probe/w"), "cuda")
    aq, as_ = mxq.quantize_mxfp8(x, scale_layout="tiled")
    wq, ws = mxq.quantize_mxfp8(w, scale_layout="tiled")
    c = mxq.gemm_mxfp8(aq, as_, wq, ws, scale_layout="tiled")
    c2 = probes.gemm_mxfp8_a_twice(aq, as_, wq, ws, torch.empty_like(c))
    torch.cuda.synchronize()
    assert torch.equal(c, c2)


def test_copy_copies():
    import torch
    from microscaling_quantized_dit_amd import probes
    lib = probes.load()
    n = (1 << 20) + 4096 + 48                       # slabs and a remainder
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    assert lib.probe_copy(probes._ptr(src), probes._ptr(dst), n, 64, probes._stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
