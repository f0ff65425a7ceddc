"""The matrix-core accumulation behaviour the error bounds of the tests rest on,
measured with single instructions on crafted and random operands
(libmxq_probes.so; no expected value comes from the GPU: every reference is an
exact fp64 sum of exactly representable products).

  * v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3, unit scales -- the MXFP8 GEMM's and the
    attention's instruction) does NOT accumulate like IEEE fp32: a product sum that
    fp32 represents exactly comes back with small products dropped.  Its error
    stays within the bound the attention test uses: products in groups of 8
    consecutive K positions, each group's largest product exact and every other
    one losing at most min(|p|, 2^-12 x the group's largest), plus 2^-22 sum |p|.
  * v_mfma_f32_32x32x16_{f16,bf16} (the NVFP4 and weight-only FP8 GEMMs'
    instructions) stay within 2^-21 sum |p| of the exact sum.
  * v_exp_f32 (the attention kernel's exponential) is within 2^-21 relative of
    2^x, the allowance the attention bound takes for it."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

E43 = np.array([oracle.code_value(oracle.E4M3, c) if (c & 0x7F) != 0x7F else np.nan for c in range(256)])
FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])


@pytest.fixture(scope="module")
def probes():
    from microscaling_quantized_dit_amd import probes as p
    p.load()
    return p


def _code(v):
    c = [c for c in FINITE if E43[c] == v]
    assert c, v
    return c[0]


def test_fp8_accumulation_is_not_ieee_fp32(probes):
    """One product 2^16 and 63 products 2^-7: the exact sum 65536 + 63 * 2^-7 is an
    fp32 value, yet the seven small products sharing the large one's group of 8 are
    dropped (the group keeps 13 bits below its largest product)."""
    a = np.zeros((32, 64), np.uint8)
    b = np.zeros((32, 64), np.uint8)
    a[0, 0], b[0, 0] = _code(256.0), _code(256.0)
    a[0, 1:], b[0, 1:] = _code(2.0 ** -4), _code(2.0 ** -3)
    d = probes.mfma_once_fp8(a, b)
    exact = 65536.0 + 63 * 2.0 ** -7
    assert np.float32(exact) == exact
    assert d[0, 0] == 65536.0 + 56 * 2.0 ** -7


def _truncation_bound(p):
    """The bound of the tests for sums of products p [..., K] (K % 8 == 0)."""
    g = np.abs(p).reshape(p.shape[:-1] + (p.shape[-1] // 8, 8))
    mx = g.max(axis=-1, keepdims=True)
    lost = np.minimum(g, 2.0 ** -12 * mx).sum(axis=-1) - np.minimum(mx[..., 0], 2.0 ** -12 * mx[..., 0])
    return lost.sum(axis=-1) + 2.0 ** -22 * np.abs(p).sum(axis=-1)


@pytest.mark.parametrize("spread", ["wide", "flux_like"])
def test_fp8_accumulation_within_the_bound(probes, spread):
    """1024 dot products of 64 random E4M3 pairs per launch, over 20 launches: every
    result within the bound of its exact sum (computed in fp64, exact)."""
    rng = np.random.RandomState(31 if spread == "wide" else 32)
    worst = 0.0
    for _ in range(20):
        if spread == "wide":
            a = rng.choice(FINITE, size=(32, 64)).astype(np.uint8)
            b = rng.choice(FINITE, size=(32, 64)).astype(np.uint8)
        else:   # codes of N(0, 1) data at a per-block scale: a narrower exponent range
            a = np.array([oracle.round_quotient(oracle.E4M3, abs(x), 1.0 / 64) | (0x80 if x < 0 else 0)
                          for x in rng.randn(32 * 64)], np.uint8).reshape(32, 64)
            b = np.array([oracle.round_quotient(oracle.E4M3, abs(x), 1.0 / 64) | (0x80 if x < 0 else 0)
                          for x in rng.randn(32 * 64)], np.uint8).reshape(32, 64)
        d = probes.mfma_once_fp8(a, b)
        p = E43[a][:, None, :] * E43[b][None, :, :]          # [32, 32, 64], exact
        exact = p.sum(axis=-1)
        bound = _truncation_bound(p)
        err = np.abs(d - exact)
        assert np.all(err <= bound), float((err / bound).max())
        worst = max(worst, float((err / np.maximum(bound, 1e-300)).max()))
    assert worst > 0.0        # the instruction really is inexact on these operands


@pytest.mark.parametrize("kind", ["fp16", "bf16"])
def test_16bit_accumulation_close_to_fp32(probes, kind):
    rng = np.random.RandomState(41)
    for _ in range(10):
        if kind == "fp16":
            a = (rng.randn(32, 16) * 2.0 ** rng.randint(-8, 8, (32, 16))).astype(np.float16)
            b = (rng.randn(32, 16) * 2.0 ** rng.randint(-8, 8, (32, 16))).astype(np.float16)
            av, bv = a.astype(np.float64), b.astype(np.float64)
            ab, bb = a.view(np.uint16), b.view(np.uint16)
        else:
            a32 = (rng.randn(32, 16) * 2.0 ** rng.randint(-20, 20, (32, 16))).astype(np.float32)
            b32 = (rng.randn(32, 16) * 2.0 ** rng.randint(-20, 20, (32, 16))).astype(np.float32)
            ab = (a32.view(np.uint32) >> 16).astype(np.uint16)
            bb = (b32.view(np.uint32) >> 16).astype(np.uint16)
            av = (ab.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            bv = (bb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        d = probes.mfma_once_16(ab, bb, kind)
        p = av[:, None, :] * bv[None, :, :]
        err = np.abs(d - p.sum(axis=-1))
        assert np.all(err <= 2.0 ** -21 * np.abs(p).sum(axis=-1)), kind


def test_exp2_accuracy(probes):
    """v_exp_f32 against 2^x in fp64 (exact to far below fp32's precision) on every
    argument the attention kernel can feed it: [-126, 9) (256 P <= 2^8 before the
    scaling margin; below 2^-126 the code underflows anyway), 2^20 seeded values
    plus every integer and half-integer of the range."""
    import torch
    rng = np.random.RandomState(5)
    x = np.concatenate([rng.uniform(-126.0, 9.0, size=1 << 20), np.arange(-126.0, 9.0, 0.5)]).astype(np.float32)
    y = probes.exp2(torch.from_numpy(x).cuda()).cpu().numpy().astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(y - ref) / ref
    assert rel.max() <= 2.0 ** -21, (rel.max(), x[np.argmax(rel)])
