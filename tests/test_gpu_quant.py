"""GPU quantizers against the CPU oracle: codes, scales and the global scale must
be bit-identical (the quantizers have exactly one correct result).

Inputs are seeded (microscaling_quantized_dit_amd.inputs) or crafted bit
patterns; every expected value is computed by the oracle on the CPU from the
same input bytes.
"""
import numpy as np
import pytest

import oracle
from microscaling_quantized_dit_amd import inputs
from tests.scale_order import tile_scales, untile_scales

pytestmark = pytest.mark.gpu

KINDS = [("e4m3", oracle.E4M3), ("e5m2", oracle.E5M2)]


def _dev(bits):
    return inputs.to_torch(bits, "cuda")


def _np(t):
    return t.cpu().numpy()


def _check_mx(mxq, bits, kind, fmt, rows=None):
    q, s = mxq.quantize_mxfp8(_dev(bits), kind)
    q, s = _np(q), _np(s)
    if rows is None:
        rq, rs = oracle.quantize_mxfp8(bits, fmt)
        np.testing.assert_array_equal(s, rs)
        np.testing.assert_array_equal(q, rq)
    else:
        rq, rs = oracle.quantize_mxfp8(bits[rows], fmt)
        np.testing.assert_array_equal(s[rows], rs)
        np.testing.assert_array_equal(q[rows], rq)


def _check_nv(mxq, bits, rows=None, static=None):
    import torch
    gin = None if static is None else torch.tensor([static], dtype=torch.float32, device="cuda")
    q, s, g = mxq.quantize_nvfp4(_dev(bits), global_scale=gin)
    q, s, g = _np(q), _np(s), float(_np(g)[0])
    if static is None:
        rg = oracle.nvfp4_global_scale(bits)
    else:
        rg = np.float32(static)
    assert np.float32(g).tobytes() == np.float32(rg).tobytes()
    sub = bits if rows is None else bits[rows]
    rq, rs, _ = oracle.quantize_nvfp4(sub, global_scale=rg)
    np.testing.assert_array_equal(s if rows is None else s[rows], rs)
    np.testing.assert_array_equal(q if rows is None else q[rows], rq)


# ------------------------------------------------------------- tiny config

@pytest.mark.parametrize("kind,fmt", KINDS)
def test_mxfp8_tiny(mxq, kind, fmt):
    _check_mx(mxq, inputs.tiny_activation(), kind, fmt)
    _check_mx(mxq, inputs.weight(256, 256, std=0.02, stream="tiny/W"), kind, fmt)


def test_nvfp4_tiny_dynamic_and_static(mxq):
    a = inputs.tiny_activation()
    _check_nv(mxq, a)
    _check_nv(mxq, inputs.weight(256, 256, std=0.02, stream="tiny/W"))
    for sg in [1.0, 0.0625, 0.013671875, 3.3e-3]:
        _check_nv(mxq, a, static=sg)


# ------------------------------------------------------ exhaustive bf16 sweep

def _sweep(block: int, amax_bits):
    """Every finite bf16 pattern, (block - 1) per block, each block completed by
    one 'controller' value that fixes the block maximum."""
    pats = np.array([p for p in range(65536) if (p & 0x7F80) != 0x7F80], np.uint16)
    out = []
    for a in amax_bits:
        per = block - 1
        n = (pats.size + per - 1) // per
        body = np.resize(pats, n * per).reshape(n, per)
        ctrl = np.full((n, 1), a, np.uint16)
        out.append(np.concatenate([ctrl, body], axis=1).reshape(-1))
    flat = np.concatenate(out)
    cols = 32 * 64
    pad = (-flat.size) % cols
    return np.concatenate([flat, np.zeros(pad, np.uint16)]).reshape(-1, cols)


@pytest.mark.parametrize("kind,fmt", KINDS)
def test_mxfp8_exhaustive_bf16(mxq, kind, fmt):
    # controllers: the block max ranges over small, typical and huge magnitudes
    x = _sweep(32, [0x0000, 0x3F80, 0x4B00, 0x7F7F, 0x0001, 0x2000])
    _check_mx(mxq, x, kind, fmt)


def test_nvfp4_exhaustive_bf16(mxq):
    x = _sweep(16, [0x3F80, 0x4B00, 0x0080])
    _check_nv(mxq, x)                         # dynamic: s_g from 0x7F7F's neighbours
    _check_nv(mxq, x, static=1.0)
    _check_nv(mxq, x, static=2.0 ** -20)


# --------------------------------------------------------- crafted edge cases

def test_edge_cases(mxq):
    z = np.zeros((2, 64), np.uint16)
    z[0, 3] = 0x8000                                     # -0
    z[1, 5] = 0x0001                                     # smallest subnormal
    for kind, fmt in KINDS:
        _check_mx(mxq, z, kind, fmt)
    _check_nv(mxq, np.zeros((1, 16), np.uint16))         # all-zero tensor: s_g = 1
    _check_nv(mxq, z)
    # exact ties: amax/2688 a power of two, block maxima on E4M3 midpoints, elements on E2M1 midpoints
    vals = np.array([2688.0 * 4, 6 * 17.0 * 4, 0.25 * 4, 0.75 * 4, 1.25 * 4, 2.5 * 4, 5 * 4, 3.5 * 4,
                     -1.75 * 4, 448.0 * 6 * 4, 1e-30, -1e-30, 3.0, 6.5 * 4, -5.0 * 4, 0.0], np.float64)
    row = inputs.bf16_bits(vals)
    t = np.tile(row, (4, 4))
    _check_nv(mxq, t)
    _check_nv(mxq, t, static=4.0)
    _check_nv(mxq, t, static=1.0)
    for kind, fmt in KINDS:
        _check_mx(mxq, t.reshape(-1, 32), kind, fmt)


@pytest.mark.parametrize("shape", [(1, 32), (3, 96), (5, 160), (7, 4128)])
def test_ragged_shapes(mxq, shape):
    x = inputs.flux_activation(*shape, seed=5, stream="ragged")
    for kind, fmt in KINDS:
        _check_mx(mxq, x, kind, fmt)
    _check_nv(mxq, x)


def test_nvfp4_extreme_tensor_scales(mxq):
    """Tensors whose amax makes s_g an fp32 subnormal, or 6 s_g's reciprocal leave
    fp32's normal range, or that span the whole bf16 range."""
    tiny = np.array([[0x0001, 0x8003, 0x0040, 0x007F, 0x0010, 0x8000, 0x0002, 0x0005] * 4], np.uint16)
    _check_nv(mxq, tiny)                              # amax ~ 2^-127: s_g subnormal
    wide = np.array([[0x7F7F, 0x0001, 0x3F80, 0xBF80, 0x0080, 0x4000, 0x8001, 0x7F00] * 4], np.uint16)
    _check_nv(mxq, wide)
    _check_nv(mxq, wide, static=2.0 ** -125)
    _check_nv(mxq, tiny, static=2.0 ** 100)


# -------------------------------------------------- full-size (config 2 shapes)

@pytest.mark.parametrize("cols", [3072, 12288])
def test_flux_activation_full_size(mxq, cols):
    """The 4608-token FLUX activations at their real shapes: MXFP8 checked in
    full, NVFP4 on every 7th row plus the exact global scale."""
    x = inputs.flux_activation(4608, cols, seed=0, stream="cfg2/x%d" % cols)
    _check_mx(mxq, x, "e4m3", oracle.E4M3)
    rows = np.arange(0, 4608, 7)
    _check_mx(mxq, x, "e5m2", oracle.E5M2, rows=rows)
    _check_nv(mxq, x, rows=rows)


@pytest.mark.parametrize("cols", [3072, 15360])
def test_flux_single_stream_activation_nvfp4(mxq, cols):
    """The single-stream linears' activations (18432 tokens; 15360 = linear2's
    input, 566 MB) quantized as the bench step does it: dynamic scale, tiled
    scales.  The global scale over the whole tensor is bit-exact; codes and scales
    of 32 rows (first and last included) match the oracle's."""
    import torch
    R = 18432
    x = inputs.flux_activation(R, cols, seed=0, stream="cfg4/x%d" % cols)
    q, s, g = mxq.quantize_nvfp4(_dev(x), scale_layout="tiled")
    rg = oracle.nvfp4_global_scale(x)
    assert np.float32(_np(g)[0]).tobytes() == np.float32(rg).tobytes()
    rows = np.concatenate([np.arange(0, R - 1, 593), [R - 1]])
    rq, rs, _ = oracle.quantize_nvfp4(x[rows], global_scale=rg)
    np.testing.assert_array_equal(_np(q)[rows], rq)
    np.testing.assert_array_equal(untile_scales(_np(s), 8)[rows], rs)
    del q, s
    torch.cuda.empty_cache()


# The amax pass writes one partial maximum per 4096 16-byte chunks (at most 256);
# every wave of the encode pass folds all of them.  A tensor of [8P, 4096] has
# exactly P partials; the tensor maximum (negative, so that the fold must use
# magnitudes) sits in the first, a middle or the last of them, and with P not a
# multiple of 64 some lanes fold clamped, repeated indices.
@pytest.mark.parametrize("P", [1, 2, 63, 64, 65, 127, 129, 200, 255, 256])
@pytest.mark.parametrize("where", ["first", "middle", "last"])
def test_nvfp4_global_scale_every_partial_count(mxq, P, where):
    R, C = 8 * P, 4096
    n = R * C
    bits = (0x3F80 + (np.arange(n, dtype=np.uint32) * 2654435761 >> 26) % 96).astype(np.uint16)
    bits ^= ((np.arange(n) % 7 == 3).astype(np.uint16) << 15)                      # some negatives
    at = {"first": 5, "middle": (P // 2) * 32768 + 1234, "last": n - 1}[where]
    bits[at] = 0xC47A                                                              # -1000.0
    bits = bits.reshape(R, C)
    _check_nv(mxq, bits, rows=np.array(sorted({0, at // C, R - 1})))


def test_deterministic(mxq):
    import torch
    x = _dev(inputs.flux_activation(512, 3072, seed=9, stream="det"))
    a = [t.clone() for t in mxq.quantize_nvfp4(x)]
    b = mxq.quantize_nvfp4(x)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    a = [t.clone() for t in mxq.quantize_mxfp8(x)]
    b = mxq.quantize_mxfp8(x)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# --------------------------------------------------- tiled scale order

@pytest.mark.parametrize("shape", [(64, 128), (192, 640), (128, 3200), (320, 1152)])
def test_tiled_scales_match_oracle(mxq, shape):
    """Both quantizers with the tiled scale order: codes as in the row-major
    order, scales the oracle's in the tiled order, bit for bit."""
    import torch
    x = inputs.flux_activation(*shape, seed=11, stream="tiled")
    dx = _dev(x)
    for kind, fmt in KINDS:
        q, s = mxq.quantize_mxfp8(dx, kind, scale_layout="tiled")
        rq, rs = oracle.quantize_mxfp8(x, fmt)
        np.testing.assert_array_equal(_np(q), rq)
        np.testing.assert_array_equal(_np(s), tile_scales(rs, 4))
    for static in (None, 0.25):
        gin = None if static is None else torch.tensor([static], dtype=torch.float32, device="cuda")
        q, s, g = mxq.quantize_nvfp4(dx, global_scale=gin, scale_layout="tiled")
        rg = oracle.nvfp4_global_scale(x) if static is None else np.float32(static)
        rq, rs, _ = oracle.quantize_nvfp4(x, global_scale=rg)
        assert np.float32(_np(g)[0]).tobytes() == np.float32(rg).tobytes()
        np.testing.assert_array_equal(_np(q), rq)
        np.testing.assert_array_equal(_np(s), tile_scales(rs, 8))


@pytest.mark.parametrize("layout", ["row", "tiled"])
@pytest.mark.parametrize("shape", [(64, 128), (192, 640), (320, 1152)])
def test_writes_stay_in_bounds(mxq, layout, shape):
    """Codes and scales are written into views of larger buffers filled with a
    canary byte: everything outside the views keeps it, everything inside is
    written (the tiled work split has no per-chunk range check)."""
    import torch
    R, C = shape
    x = _dev(inputs.flux_activation(R, C, seed=13, stream="canary"))
    pad = 4096

    def views(*sizes):
        bufs = [torch.full((n + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda") for n in sizes]
        return bufs, [b[pad:pad + n] for b, n in zip(bufs, sizes)]

    bufs, (q, s) = views(R * C, R * C // 32)
    mxq.quantize_mxfp8(x, out=(q.view(R, C), s.view(R, C // 32)), scale_layout=layout)
    bufs2, (q2, s2) = views(R * C // 2, R * C // 16)
    g = torch.empty((1,), dtype=torch.float32, device="cuda")
    mxq.quantize_nvfp4(x, out=(q2.view(R, C // 2), s2.view(R, C // 16), g), scale_layout=layout)
    torch.cuda.synchronize()
    for b in bufs + bufs2:
        assert (b[:pad] == 0xA5).all().item() and (b[-pad:] == 0xA5).all().item()
    # the views hold the oracle's values (so every byte was written)
    bits = inputs.flux_activation(R, C, seed=13, stream="canary")
    rq, rs = oracle.quantize_mxfp8(bits, oracle.E4M3)
    np.testing.assert_array_equal(_np(q).reshape(R, C), rq)
    np.testing.assert_array_equal(_np(s).reshape(R, -1), tile_scales(rs, 4) if layout == "tiled" else rs)
    rq, rs, _ = oracle.quantize_nvfp4(bits)
    np.testing.assert_array_equal(_np(q2).reshape(R, -1), rq)
    np.testing.assert_array_equal(_np(s2).reshape(R, -1), tile_scales(rs, 8) if layout == "tiled" else rs)


@pytest.mark.parametrize("rows,cols", [(4608, 12288), (18432, 15360)])
def test_tiled_scales_full_size(mxq, rows, cols):
    """At the FLUX activation shapes (18432 x 15360 has 17.7 M NVFP4 scales): the
    tiled scales are the row-major ones reordered, every byte."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(rows + cols)
    x = (torch.randn((rows, cols), generator=gen, device="cuda") * 3).to(torch.bfloat16)
    _, s_row = mxq.quantize_mxfp8(x)
    _, s_til = mxq.quantize_mxfp8(x, scale_layout="tiled")
    np.testing.assert_array_equal(_np(s_til), tile_scales(_np(s_row), 4))
    del s_row, s_til
    q_row, s_row, g_row = mxq.quantize_nvfp4(x)
    q_til, s_til, g_til = mxq.quantize_nvfp4(x, scale_layout="tiled")
    assert torch.equal(q_row, q_til) and torch.equal(g_row, g_til)
    np.testing.assert_array_equal(_np(s_til), tile_scales(_np(s_row), 8))


# ------------------------------------- static-scale calibration (P5 step 1)

def test_nvfp4_static_calibration(mxq):
    """Calibrated static decode scale: folded on the GPU over three calibration
    activations (and an all-zero one), bit-equal to the oracle's; then a fresh
    activation, partly beyond the calibrated range, quantized statically with it."""
    import torch
    batches = [inputs.flux_activation(64, 3072, seed=s, stream="calib/%d" % s) for s in range(3)]
    running = None
    for b in batches + [np.zeros((16, 3072), np.uint16)]:
        running = mxq.nvfp4_calibrate(_dev(b), running)
    g = np.float32(_np(running)[0])
    assert g.tobytes() == oracle.nvfp4_calibrate(batches).tobytes()
    fresh = inputs.flux_activation(128, 3072, seed=9, stream="calib/fresh")
    hot = inputs.gaussian(8, 3072, 400.0, seed=9, stream="calib/hot")
    _check_nv(mxq, np.concatenate([fresh, hot]), static=float(g))
    # a running scale that already exceeds the tensor's stays put
    r = torch.tensor([1e3], dtype=torch.float32, device="cuda")
    assert float(mxq.nvfp4_calibrate(_dev(batches[0]), r)[0]) == 1e3


# --------------------------------------------- weight-only FP8 (per-tensor E4M3)

def _check_w8(mxq, bits, static=None):
    import torch
    sin = None if static is None else torch.tensor([static], dtype=torch.float32, device="cuda")
    q, s = mxq.quantize_fp8_weight(_dev(bits), scale=sin)
    q, s = _np(q), np.float32(_np(s)[0])
    rq, rs = oracle.quantize_fp8_weight(bits, scale=static)
    assert s.tobytes() == np.float32(rs).tobytes()
    np.testing.assert_array_equal(q, rq)


def test_fp8_weight_quantizer(mxq):
    """Per-tensor E4M3 weights bit-exact to the oracle: FLUX weight shapes, every
    finite bf16 pattern under three scales, ties and saturation, extreme scales."""
    _check_w8(mxq, inputs.weight(3072, 3072, seed=0, stream="w8/W"))
    _check_w8(mxq, inputs.weight(1024, 12288, seed=1, stream="w8/W2"), static=2.0 ** -9)
    sweep = _sweep(16, [0x3F80, 0x4B00, 0x0080])
    _check_w8(mxq, sweep)
    _check_w8(mxq, sweep, static=1.0)
    _check_w8(mxq, sweep, static=0.01)
    _check_w8(mxq, sweep, static=2.0 ** -110)            # outside the fp32 bracket range: exact path
    ties = inputs.bf16_bits(np.array([[17.0, 19.0, 21.0, -23.0, 0.0, -0.0, 1e-3, 460.0,
                                       2.25 * 2 ** -7, 500.0, -9.0, 13.0, 448.0, -0.015625, 3.0, 1e-30]]))
    for sc in (1.0, 0.5, 2.0 ** -4, 3.0):
        _check_w8(mxq, np.tile(ties, (2, 2)), static=sc)
    _check_w8(mxq, np.zeros((2, 32), np.uint16))         # all-zero: scale 1
