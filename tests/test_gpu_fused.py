"""The MXFP8 GEMM with the activation quantizer in its prologue (mxq_gemm_mxfp8_fused).

Its result is defined as the separate chain's: the activation quantized by
mxq_quantize_mxfp8, then mxq_gemm_mxfp8 with the same element format for both
operands (page "NVIDIA Blackwell平台FP4量化技术解析与图像生成优化", section 3.1:
the bf16 activation is quantized at run time and handed to the low-precision
GEMM).  So:
  * every case requires the fused output bit-identical to that chain on the GPU
    (both entry points are parity-tested against the oracle elsewhere);
  * a small case and sampled rows of the long-sequence shape are also compared
    with the oracle directly: the oracle quantizes the activation and forms the
    fp64 product of its codes, within the GEMM tolerance (max error relative to
    max(|r|, rms(r)) <= 1e-2, relative Frobenius error <= 3e-3).
Shapes: one tile, ragged 256-tiles, more tiles than compute units (persistent,
prefetch across tile boundaries), the FLUX double-stream linears and the
long-sequence shape; blocks that are all zero, subnormal or beyond the largest
code; both weight-scale orders and all three epilogues."""
import numpy as np
import pytest

import oracle
from microscaling_quantized_dit_amd import inputs

pytestmark = pytest.mark.gpu

MAX_REL, FRO_REL = 1e-2, 3e-3
EPIS = {"none": oracle.EPI_NONE, "bias": oracle.EPI_BIAS, "bias_gelu": oracle.EPI_BIAS_GELU_TANH}


def _bf16(t):
    import torch
    return inputs.bf16_to_f64(t.cpu().view(torch.int16).numpy())


def _chain_and_fused(mxq, x, w, kind, layout, bias=None, epi="none"):
    """(fused output, chain output) on device tensors x [M, K] bf16, w [N, K] bf16."""
    wq, ws = mxq.quantize_mxfp8(w, kind, scale_layout=layout)
    aq, as_ = mxq.quantize_mxfp8(x, kind, scale_layout=layout)
    chain = mxq.gemm_mxfp8(aq, as_, wq, ws, bias=bias, epi=epi, a_kind=kind, w_kind=kind, scale_layout=layout)
    fused = mxq.gemm_mxfp8_fused(x, wq, ws, kind=kind, bias=bias, epi=epi, scale_layout=layout)
    return fused, chain


def _assert_same(fused, chain, what):
    import torch
    same = torch.eq(fused.view(torch.int16), chain.view(torch.int16))
    assert bool(same.all().item()), (what, int((~same).sum().item()))


@pytest.mark.parametrize("kind", ["e4m3", "e5m2"])
@pytest.mark.parametrize("layout", ["row", "tiled"])
@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (384, 640, 256), (640, 384, 1152), (2432, 7808, 512)])
def test_fused_equals_chain_shapes(mxq, kind, layout, M, N, K):
    x = inputs.to_torch(inputs.flux_activation(M, K, seed=M + K, stream="fused/A"), "cuda")
    w = inputs.to_torch(inputs.weight(N, K, seed=N + K, stream="fused/W"), "cuda")
    b = inputs.to_torch(inputs.bias(N, K, seed=N, stream="fused/b"), "cuda")
    for epi in ("none", "bias", "bias_gelu"):
        fused, chain = _chain_and_fused(mxq, x, w, kind, layout, bias=None if epi == "none" else b, epi=epi)
        _assert_same(fused, chain, (M, N, K, kind, layout, epi))


def test_fused_special_blocks(mxq):
    """All-zero blocks (scale 2^-127), blocks of bf16 subnormals only, blocks with
    values near the largest bf16 (codes saturate, scales at the top of the range),
    and single nonzero values, spread over one 512 x 512 operand."""
    import torch
    M = N = K = 512
    a = inputs.flux_activation(M, K, seed=7, stream="fused/special").copy()
    a[0:7, :] = 0                                   # zero rows
    a[7:64, 0:32] = 0                               # zero blocks
    a[64:96, :] = (np.arange(32 * K) % 127 + 1).reshape(32, K).astype(np.uint16)   # subnormals only
    big = np.uint16(0x7F00)                          # 2^127
    a[96:128, :] = big
    a[96:128, ::3] = np.uint16(0x7F7F)               # largest finite bf16
    a[128:160, :] = 0
    a[128:160, 5::64] = np.uint16(0x3F80)            # one 1.0 per 64 values
    x = inputs.to_torch(a, "cuda")
    w = inputs.to_torch(inputs.weight(N, K, seed=8, stream="fused/specialW"), "cuda")
    for kind in ("e4m3", "e5m2"):
        fused, chain = _chain_and_fused(mxq, x, w, kind, "tiled")
        _assert_same(fused, chain, ("special", kind))
    assert torch.isfinite(fused[128:160].float()).all().item()


@pytest.mark.parametrize("kind", ["e4m3", "e5m2"])
def test_fused_every_bf16_pattern(mxq, kind):
    """Every finite bf16 pattern as an activation value, once in pattern order
    (blocks of neighbouring magnitudes) and once in a seeded permutation (mixed
    blocks), against the identity weight: C is then the dequantized activation
    itself, so every code and block scale the fused kernel forms is compared with
    the separate quantizer's (bit for bit) and with the oracle's (within the
    GEMM tolerance; values below bf16's range underflow alike)."""
    import torch
    pats = np.arange(65536, dtype=np.uint32)
    vals = pats[((pats >> 7) & 0xFF) != 0xFF].astype(np.uint16)          # 65280 finite patterns
    rng = np.random.RandomState(5)
    K = N = 512
    a = np.concatenate([vals, vals[rng.permutation(vals.size)], np.zeros(K, np.uint16)]).reshape(-1, K)
    eye = np.zeros((N, K), np.uint16)
    eye[np.arange(N), np.arange(N)] = 0x3F80                              # 1.0
    x, w = inputs.to_torch(a, "cuda"), inputs.to_torch(eye, "cuda")
    for layout in ("row", "tiled"):
        fused, chain = _chain_and_fused(mxq, x, w, kind, layout)
        _assert_same(fused, chain, ("every pattern", kind, layout))
    fmt = oracle.E4M3 if kind == "e4m3" else oracle.E5M2
    aq, as_ = oracle.quantize_mxfp8(a, fmt)
    wq, ws = oracle.quantize_mxfp8(eye, fmt)
    r = oracle.gemm_mxfp8(aq, as_, wq, ws, fmt, fmt)
    e = oracle.compare(_bf16(fused), r)
    assert e["max_rel"] <= MAX_REL and e["fro_rel"] <= FRO_REL, (kind, e)


@pytest.mark.parametrize("name,N,K,epi", [("qkv", 9216, 3072, "none"), ("out_proj", 3072, 3072, "none"),
                                          ("mlp_up", 12288, 3072, "bias_gelu"), ("mlp_down", 3072, 12288, "none")])
def test_fused_flux_shapes(mxq, name, N, K, epi):
    M = 4608
    x = inputs.to_torch(inputs.flux_activation(M, K, seed=K, stream="fused/flux/A"), "cuda")
    w = inputs.to_torch(inputs.weight(N, K, seed=N, stream="fused/flux/W"), "cuda")
    b = inputs.to_torch(inputs.bias(N, K, seed=N, stream="fused/flux/b"), "cuda") if epi != "none" else None
    fused, chain = _chain_and_fused(mxq, x, w, "e4m3", "tiled", bias=b, epi=epi)
    _assert_same(fused, chain, name)


def test_fused_against_oracle_small(mxq):
    """The fused entry point against the oracle directly (its own quantization of
    the activation and of the weight, fp64 product), bias + GELU."""
    M, N, K = 384, 640, 1152
    a = inputs.flux_activation(M, K, seed=3, stream="fused/or/A")
    wb = inputs.weight(N, K, seed=4, stream="fused/or/W")
    bias = inputs.bias(N, K, seed=5, stream="fused/or/b")
    for fmt, kind in ((oracle.E4M3, "e4m3"), (oracle.E5M2, "e5m2")):
        aq, as_ = oracle.quantize_mxfp8(a, fmt)
        wq, ws = oracle.quantize_mxfp8(wb, fmt)
        import torch
        c = mxq.gemm_mxfp8_fused(inputs.to_torch(a, "cuda"), torch.from_numpy(wq).cuda(), torch.from_numpy(ws).cuda(),
                                 kind=kind, bias=inputs.to_torch(bias, "cuda"), epi="bias_gelu")
        r = oracle.gemm_mxfp8(aq, as_, wq, ws, fmt, fmt, bias=bias, epi=oracle.EPI_BIAS_GELU_TANH)
        e = oracle.compare(_bf16(c), r)
        assert e["max_rel"] <= MAX_REL and e["fro_rel"] <= FRO_REL, (kind, e)


@pytest.mark.parametrize("kind", ["e4m3", "e5m2"])
def test_fused_long_sequence(mxq, kind):
    """M = 32768, K = 4096, N = 4096 with bias: bit-identical to the chain, and
    two sampled rows of every 256-row tile against the oracle."""
    M, N, K = 32768, 4096, 4096
    fmt = oracle.E4M3 if kind == "e4m3" else oracle.E5M2
    a = inputs.long_sequence_activation(M, K, seed=0, stream="fused/cfg5/A")
    wb = inputs.weight(N, K, seed=1, stream="fused/cfg5/W")
    bias = inputs.bias(N, K, seed=2, stream="fused/cfg5/b")
    x, w, b = inputs.to_torch(a, "cuda"), inputs.to_torch(wb, "cuda"), inputs.to_torch(bias, "cuda")
    fused, chain = _chain_and_fused(mxq, x, w, kind, "tiled", bias=b, epi="bias")
    _assert_same(fused, chain, ("cfg5", kind))
    rng = np.random.RandomState(11)
    rows = np.array(sorted({0, M - 1} | {t0 + h * 128 + int(rng.randint(0, 128)) for t0 in range(0, M, 256)
                                          for h in (0, 1)}))
    aq, as_ = oracle.quantize_mxfp8(a[rows], fmt)
    wq, ws = oracle.quantize_mxfp8(wb, fmt)
    r = oracle.gemm_mxfp8(aq, as_, wq, ws, fmt, fmt, bias=bias, epi=oracle.EPI_BIAS)
    e = oracle.compare(_bf16(fused)[rows], r)
    assert e["max_rel"] <= MAX_REL and e["fro_rel"] <= FRO_REL, (kind, e)
