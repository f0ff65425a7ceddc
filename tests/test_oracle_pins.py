"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

Each test names what it pins.  None of them re-derives an oracle value with the
oracle's own method: value sets are checked against closed forms and counts,
rounding against brute-force argmin in exact rationals (tests/fraction_ref.py),
the GEMM against integer matmul and one-hot identities, GELU against torch.
"""
import json
import math
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
from microscaling_quantized_dit_amd import inputs
from tests import fraction_ref as fr

HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------- P-1..P-4: formats

def test_e2m1_value_set():
    """E2M1 has 16 codes decoding to {0, ±0.5, ±1, ±1.5, ±2, ±3, ±4, ±6}
    (the FP4 element of page 'NVIDIA Blackwell平台FP4量化技术解析…' §1; the value
    set is the one the E2M1 name fixes: 1 sign, 2 exponent, 1 mantissa bit)."""
    vals = [oracle.code_value(oracle.E2M1, c) for c in range(16)]
    assert sorted(set(abs(v) for v in vals)) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert vals[:8] == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert [-v for v in vals[:8]] == vals[8:]
    assert math.copysign(1.0, vals[8]) == -1.0       # code 0x8 is -0


def test_e4m3_layout():
    """E4M3 = 1 sign + 4 exponent + 3 mantissa bits (page '麦橘超然性能实战分析…' §2.2),
    'fn' variant (torch.float8_e4m3fn, §3.2 of that page): no Inf, NaN only at
    0x7F/0xFF, max 448, min normal 2^-6, min subnormal 2^-9, 126 positive values."""
    vals = [oracle.code_value(oracle.E4M3, c) for c in range(256)]
    nan = [c for c, v in enumerate(vals) if v != v]
    assert nan == [0x7F, 0xFF]
    assert not any(math.isinf(v) for v in vals)
    pos = [v for v in vals[:128] if v == v and v > 0]
    assert len(pos) == 126
    assert max(pos) == 448.0 and min(pos) == 2.0 ** -9
    assert vals[0x08] == 2.0 ** -6 and vals[0x07] == 7 * 2.0 ** -9
    assert [Fr(v) for v in vals[:0x7F]] == fr.E4M3        # closed-form value set
    for c in range(128):
        if vals[c] == vals[c]:
            assert vals[c | 0x80] == -vals[c]


def test_e5m2_layout():
    """E5M2 = 1 + 5 + 2 bits (same page §2.2): max 57344, min subnormal 2^-16,
    Inf at 0x7C, NaN above."""
    vals = [oracle.code_value(oracle.E5M2, c) for c in range(256)]
    assert vals[0x7B] == 57344.0 and vals[0x01] == 2.0 ** -16 and vals[0x04] == 2.0 ** -14
    assert math.isinf(vals[0x7C]) and all(vals[c] != vals[c] for c in (0x7D, 0x7E, 0x7F))
    assert [Fr(v) for v in vals[:0x7C]] == fr.E5M2


def test_e8m0_powers_of_two():
    """Every E8M0 code c < 255 is exactly 2^(c-127); 255 is NaN."""
    for c in range(255):
        v = oracle.e8m0_value(c)
        m, e = math.frexp(v)
        assert m == 0.5 and e - 1 == c - 127
    assert oracle.e8m0_value(255) != oracle.e8m0_value(255)


def test_bf16_decode_all_patterns():
    """bf16 decode agrees with the hardware-independent float32 widening for
    every bit pattern (numpy's uint32<<16 view)."""
    bits = np.arange(65536, dtype=np.uint32)
    ref = (bits << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_value(int(b)) for b in range(0, 65536, 7)])
    sel = ref[::7]
    fin = np.isfinite(sel)
    assert np.array_equal(got[fin], sel[fin])


# ------------------------------------------------------- P-5: worked example

def test_worked_example():
    """q = round(0.176 / 0.01) = 18 (page 'FP8量化技术提升SD3.5…', step 2), in E4M3
    as in the integers: 17.6 sits between the E4M3 values 16 and 18."""
    g = json.load(open(os.path.join(HERE, "golden", "worked_example.json")))
    assert abs(g["quotient_num"] / g["quotient_den"] - g["x"] / g["scale"]) < 1e-12
    code = oracle.round_quotient(oracle.E4M3, g["quotient_num"], g["quotient_den"])
    assert oracle.code_value(oracle.E4M3, code) == g["q"]
    assert round(g["x"] / g["scale"]) == g["q"]
    assert abs(oracle.code_value(oracle.E4M3, code) * g["scale"] - g["dequant"]) < 1e-12
    below = oracle.code_value(oracle.E4M3, code - 1)
    assert below == 16.0


# ---------------------------------------------------- P-6: brute-force RNE

def _all_finite_bf16_magnitudes():
    b = np.arange(0x7F80, dtype=np.uint16)
    return b, inputs.bf16_to_f64(b)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("exp", [-133, -20, -3, 0, 5, 100])
def test_rne_bruteforce_power_of_two_scale(fmt, exp):
    """For every finite bf16 magnitude and a power-of-two scale, the oracle's code is
    the argmin over the whole value grid with ties to the even code.  Computed in
    fp64: with q <= 1024 * max every distance that can win is exact; beyond that
    the nearest finite value is the maximum (saturation)."""
    _, x = _all_finite_bf16_magnitudes()
    den = 2.0 ** exp
    got = oracle.round_quotient_array(fmt, x, den).astype(np.int64)
    grid = np.array([float(v) for v in fr.TABLES[fmt]])
    q = x / den                                   # exact: power-of-two divisor
    far = q > 1024 * grid[-1]
    assert np.all(got[far] == grid.size - 1)
    got, q = got[~far], q[~far]
    d = np.abs(q[:, None] - grid[None, :])
    dmin = d.min(axis=1, keepdims=True)
    ties = d == dmin
    idx = np.arange(grid.size)[None, :]
    # among the minimal distances prefer the even index
    score = np.where(ties, np.where(idx % 2 == 0, 0, 1), 2) * 1000 + idx
    want = score.argmin(axis=1)
    assert np.array_equal(got, want)


def test_rne_bruteforce_e2m1_and_e4m3_non_power_scales():
    """Rounding of quotients by a non-power-of-two divisor (the NVFP4 case)
    against exact rational argmin, including exact midpoints."""
    rng = np.random.RandomState(7)
    dens = [1.0, 0.75, 1.125 * 2.0 ** -7, float(np.float32(1 / 3.0)), 6 * float(np.float32(0.0123))]
    for den in dens:
        nums = list(rng.uniform(0, 8 * den, 300))
        # exact midpoints and their neighbours
        for m in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]:
            t = m * den
            nums += [t, float(np.nextafter(t, 0)), float(np.nextafter(t, 1e9))]
        for n in nums:
            got = oracle.round_quotient(oracle.E2M1, n, den)
            assert got == fr.rne_sat(Fr(n) / Fr(den), fr.E2M1), (n, den)
        for n in list(rng.uniform(0, 500 * den, 200)) + [464 * den, 448 * den, 480 * den, 17 * den]:
            got = oracle.round_quotient(oracle.E4M3, n, den)
            assert got == fr.rne_sat(Fr(n) / Fr(den), fr.E4M3), (n, den)


def test_global_scale_rounding_all_bf16():
    """s_g = RN_fp32(amax / 2688) for every positive finite bf16 amax, against
    exact rational rounding."""
    b, x = _all_finite_bf16_magnitudes()
    for i in range(1, b.size, 3):
        a = float(x[i])
        got = oracle.rn_fp32_div(a, 2688.0)
        assert Fr(float(got)) == fr.rn_fp32(Fr(a) / 2688), (a, got)


# ------------------------------------------- P-7: saturation and special cases

def _bits(vals):
    return inputs.bf16_bits(np.array(vals, np.float64))


def test_mx_saturation_and_scale_rule():
    """A 32-block whose scaled amax lies in (448, 512) saturates to 0x7E/0xFE;
    the scale exponent is floor(log2 amax) - 8 for E4M3 (-15 for E5M2)."""
    row = [1.0] * 32
    row[3] = 500.0          # floor(log2) = 8 -> E = 0, 500 > 448 -> saturate
    row[4] = -470.0
    x = _bits([row])
    q, s = oracle.quantize_mxfp8(x, oracle.E4M3)
    assert s[0, 0] == 127 + 0
    assert q[0, 3] == 0x7E and q[0, 4] == 0xFE
    assert q[0, 0] == 0x38                                   # 1.0
    q5, s5 = oracle.quantize_mxfp8(x, oracle.E5M2)
    assert s5[0, 0] == 127 + 8 - 15
    assert q5[0, 3] == 0x7B and q5[0, 4] == 0xFB             # 64000 > 57344 saturates


def test_mx_zero_and_sign_rules():
    """All-zero block -> scale byte 0 (E = -127); -0 and negatives that round to
    zero keep the sign bit."""
    row = [0.0] * 32 + [1.0] + [-1e-6] + [0.0] * 30
    x = _bits([row])
    x[0, 1] = 0x8000                                         # -0
    q, s = oracle.quantize_mxfp8(x, oracle.E4M3)
    assert s[0, 0] == 0 and s[0, 1] == 127 - 8
    assert q[0, 1] == 0x80 and q[0, 0] == 0x00
    assert q[0, 33] == 0x80                                  # -1e-6 / 2^-8 rounds to -0


def test_nv_special_cases():
    """Tensor amax 0 -> s_g = 1, S_b = 0, codes 0 with sign; a block with
    subnormal-range E4M3 scale; a quotient above 6 saturates to code 7."""
    z = _bits([[0.0] * 16])
    z[0, 5] = 0x8000
    q, s, g = oracle.quantize_nvfp4(z)
    assert g == np.float32(1.0) and s[0, 0] == 0
    assert (q[0, 2] & 0xF0) == 0x80 and (q[0, 2] & 0x0F) == 0      # element 5 = high nibble of byte 2
    # static scale forcing a saturated element: amax_b / (6 s_g) = 448 -> S = 448
    row = [2688.0] + [1.0] * 15
    q, s, g = oracle.quantize_nvfp4(_bits([row]), global_scale=1.0)
    assert s[0, 0] == 0x7E and (q[0, 0] & 0xF) == 7
    # tiny block next to a large one: S_b lands in E4M3's subnormal range
    row = [4000.0] + [0.0] * 15 + [0.01] + [0.0] * 15
    q, s, g = oracle.quantize_nvfp4(_bits([row]))
    S1 = oracle.code_value(oracle.E4M3, int(s[0, 1]))
    assert 0 < S1 < 2.0 ** -6


# ----------------------------------------------------- P-15: cross-oracle

def _random_tiny(rows, cols, seed):
    rng = np.random.RandomState(seed)
    v = rng.standard_normal((rows, cols)) * np.exp(rng.standard_normal((1, cols)))
    v[rng.rand(rows, cols) < 0.05] *= 40
    b = _bits(v)
    b[rng.rand(rows, cols) < 0.02] = 0
    b[rng.rand(rows, cols) < 0.01] = 0x8000
    return b


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_mx_matches_bruteforce(seed, fmt):
    x = _random_tiny(4, 96, seed)
    q, s = oracle.quantize_mxfp8(x, fmt)
    rq, rs = fr.quant_mx(x.tolist(), 4, 96, fmt)
    assert np.array_equal(q, np.array(rq)) and np.array_equal(s, np.array(rs))


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_nv_matches_bruteforce(seed):
    x = _random_tiny(3, 64, seed)
    if seed == 3:
        x[0, 0] = _bits([[2688.0 * 8]])[0, 0]     # amax/2688 a power of two: exact ties appear
    q, s, g = oracle.quantize_nvfp4(x)
    rq, rs, rg = fr.quant_nv(x.tolist(), 3, 64)
    assert Fr(float(g)) == rg
    assert np.array_equal(s, np.array(rs))
    nib = np.stack([q & 0xF, q >> 4], axis=-1).reshape(3, 64)
    assert np.array_equal(nib, np.array(rq))


def test_nv_static_scale_matches_bruteforce():
    x = _random_tiny(2, 48, 5)
    for sg in [1.0, 0.0625, float(np.float32(0.0137))]:
        q, s, g = oracle.quantize_nvfp4(x, global_scale=sg)
        rq, rs, rg = fr.quant_nv(x.tolist(), 2, 48, global_in=Fr(float(np.float32(sg))))
        assert g == np.float32(sg)
        assert np.array_equal(s, np.array(rs))
        nib = np.stack([q & 0xF, q >> 4], axis=-1).reshape(2, 48)
        assert np.array_equal(nib, np.array(rq))


# ------------------------------------------------ P-8, P-10, P-11: identities

def test_mx_idempotent():
    """quant(deq(quant(x))) == quant(x): dequantized values are bf16-exact."""
    x = inputs.flux_activation(16, 256, seed=3, stream="pin/idem")
    for fmt in (oracle.E4M3, oracle.E5M2):
        q, s = oracle.quantize_mxfp8(x, fmt)
        d = oracle.dequant_mxfp8(q, s, fmt)
        x2 = inputs.bf16_bits(d)
        assert np.array_equal(inputs.bf16_to_f64(x2), d)
        q2, s2 = oracle.quantize_mxfp8(x2, fmt)
        assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_storage_ratio():
    """NVFP4 stores 4.5 bits per element, about 3.5x less than bf16 (page
    'NVIDIA量化推理…', NVFP4 paragraph); MXFP8 8.25 bits."""
    x = inputs.tiny_activation()
    q, s, g = oracle.quantize_nvfp4(x)
    bits = 8 * (q.nbytes + s.nbytes) / x.size
    assert bits == 4.5 and 3.5 <= 16 / bits < 3.6
    q, s = oracle.quantize_mxfp8(x)
    assert 8 * (q.nbytes + s.nbytes) / x.size == 8.25


def test_mx_powers_of_two_exact():
    rng = np.random.RandomState(3)
    e = rng.randint(-20, 20, size=(8, 64))
    sign = np.where(rng.rand(8, 64) < 0.5, -1.0, 1.0)
    v = sign * 2.0 ** e
    x = _bits(v)
    for fmt in (oracle.E4M3, oracle.E5M2):
        q, s = oracle.quantize_mxfp8(x, fmt)
        d = oracle.dequant_mxfp8(q, s, fmt)
        # exact wherever the power lies inside the block's representable range
        E = s.astype(np.int64).repeat(32, axis=1) - 127
        minexp = (-9 if fmt == oracle.E4M3 else -16) + E
        ok = e >= minexp
        assert np.array_equal(d[ok], v[ok])


# ------------------------------------------------ P-12, P-13: GEMM identities

def test_gemm_textbook_integers():
    """Unit scales and small codes: C equals the integer matmul exactly."""
    rng = np.random.RandomState(11)
    M, N, K = 16, 24, 64
    ia = rng.randint(-4, 5, size=(M, K))
    iw = rng.randint(-4, 5, size=(N, K))
    # E4M3 codes of the small integers with unit E8M0 scales (byte 127)
    qa = np.array([[oracle.round_quotient(oracle.E4M3, abs(float(v)), 1.0) | (0x80 if v < 0 else 0)
                    for v in r] for r in ia], np.uint8)
    qw = np.array([[oracle.round_quotient(oracle.E4M3, abs(float(v)), 1.0) | (0x80 if v < 0 else 0)
                    for v in r] for r in iw], np.uint8)
    sa = np.full((M, K // 32), 127, np.uint8)
    sw = np.full((N, K // 32), 127, np.uint8)
    out = oracle.gemm_mxfp8(qa, sa, qw, sw)
    assert np.array_equal(out, (ia @ iw.T).astype(np.float64))
    # NVFP4 with S_b = 1.0 (code 0x38) and s_g = 1: E2M1 codes of small integers
    fa = rng.choice([0, 0.5, 1, 1.5, 2, 3, 4, 6], size=(M, K)) * np.where(rng.rand(M, K) < 0.5, -1, 1)
    fw = rng.choice([0, 0.5, 1, 1.5, 2, 3, 4, 6], size=(N, K)) * np.where(rng.rand(N, K) < 0.5, -1, 1)

    def pack(f):
        codes = np.array([[fr.E2M1.index(Fr(abs(v))) | (8 if v < 0 else 0) for v in r] for r in f], np.uint8)
        return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)

    out = oracle.gemm_nvfp4(pack(fa), np.full((M, K // 16), 0x38, np.uint8), 1.0,
                            pack(fw), np.full((N, K // 16), 0x38, np.uint8), 1.0)
    assert np.array_equal(out, fa @ fw.T)


def test_gemm_one_hot_rows():
    """A one-hot A row picks out the dequantized W row (+bias): pins per-block
    scale application, including NVFP4's E4M3 mantissas and the global scales."""
    K, N = 64, 8
    w = inputs.weight(N, K, seed=2, stream="pin/onehot")
    b = inputs.bias(N, K, seed=2, stream="pin/onehot/b")
    wq, ws, wg = oracle.quantize_nvfp4(w)
    wdeq = oracle.dequant_nvfp4(wq, ws, wg)
    for k in [0, 17, 63]:
        row = np.zeros((1, K))
        row[0, k] = 1.0
        aq, as_, ag = oracle.quantize_nvfp4(_bits(row))
        a1 = oracle.dequant_nvfp4(aq, as_, ag)[0, k]
        out = oracle.gemm_nvfp4(aq, as_, ag, wq, ws, wg, bias=b, epi=oracle.EPI_BIAS)
        want = a1 * wdeq[:, k] + inputs.bf16_to_f64(b)
        assert np.allclose(out[0], want, rtol=1e-15, atol=0)
    mq, ms = oracle.quantize_mxfp8(w)
    mdeq = oracle.dequant_mxfp8(mq, ms)
    row = np.zeros((1, K))
    row[0, 40] = 2.0
    aq, as_ = oracle.quantize_mxfp8(_bits(row))
    out = oracle.gemm_mxfp8(aq, as_, mq, ms)
    assert np.array_equal(out[0], 2.0 * mdeq[:, 40])


def test_gelu_tanh_epilogue():
    """GELU (tanh form) against torch's own, and gelu(x) - gelu(-x) = x."""
    import torch
    K, N = 32, 64
    a = np.zeros((2, K))
    a[0, 0] = 1.0
    a[1, 0] = -1.0
    w = np.linspace(-6, 6, N * K).reshape(N, K)
    bias = inputs.bf16_bits(np.zeros(N))
    y = oracle.linear(a, w, 1.0, bias, oracle.EPI_BIAS_GELU_TANH)
    pre = oracle.linear(a, w, 1.0, bias, oracle.EPI_BIAS)
    ref = torch.nn.functional.gelu(torch.from_numpy(pre), approximate="tanh").numpy()
    assert np.allclose(y, ref, rtol=1e-14, atol=1e-300)
    assert np.allclose(y[0] - y[1], pre[0], rtol=1e-13)


# ------------------------------ static-scale calibration (NEXT-3 row, P5 step 1)

def _unpack_nibbles(q):
    q = np.asarray(q)
    out = np.empty((q.shape[0], q.shape[1] * 2), np.uint8)
    out[:, 0::2] = q & 0xF
    out[:, 1::2] = q >> 4
    return out


def test_calibrated_scale_pins():
    """The calibrated decode scale is RN_fp32(max amax / 2688) over the
    calibration tensors (exact rational arithmetic), whatever their order; an
    all-zero tensor adds nothing; the tensor with the largest amax quantized
    statically with it reproduces its own dynamic quantization; and a tensor
    beyond the calibrated range quantizes (with saturation) exactly as the
    rational definition says."""
    batches = [inputs.gaussian(4, 64, std, seed=7, stream="calib/%d" % i) for i, std in enumerate((0.5, 3.0, 0.01))]
    zero = np.zeros((2, 32), np.uint16)
    g = oracle.nvfp4_calibrate(batches + [zero])
    amax = max(abs(fr.bf16_value(int(v))) for b in batches for v in b.reshape(-1))
    assert Fr(float(g)) == fr.rn_fp32(amax / 2688)
    assert oracle.nvfp4_calibrate(list(reversed(batches))).tobytes() == g.tobytes()
    assert oracle.nvfp4_calibrate([zero]) == 0.0
    assert oracle.nvfp4_calibrate([zero], running=0.5) == np.float32(0.5)
    big = batches[1]
    q_dyn, s_dyn, g_dyn = oracle.quantize_nvfp4(big)
    q_st, s_st, g_st = oracle.quantize_nvfp4(big, global_scale=g)
    assert g_dyn.tobytes() == g.tobytes() == g_st.tobytes()
    np.testing.assert_array_equal(q_dyn, q_st)
    np.testing.assert_array_equal(s_dyn, s_st)
    # outside the calibrated range: block scales saturate at 448, codes at 6
    hot = inputs.gaussian(2, 32, 40.0, seed=8, stream="calib/hot")
    q, s, _ = oracle.quantize_nvfp4(hot, global_scale=g)
    rq, rs, _ = fr.quant_nv(hot.tolist(), 2, 32, global_in=Fr(float(g)))
    np.testing.assert_array_equal(s, np.array(rs, np.uint8))
    np.testing.assert_array_equal(_unpack_nibbles(q), np.array(rq, np.uint8))
    assert (s == 126).any() and ((_unpack_nibbles(q) & 7) == 7).any()


# ------------------------------------ weight-only FP8 (NEXT-2 row, P4 3.2, P5)

def test_fp8_weight_quantizer_against_rationals():
    """Per-tensor FP8 weights: codes and the decode scale against exact rational
    rounding -- dynamic scale, a power-of-two static scale that puts values on
    E4M3 midpoints (ties), and a small static scale that saturates."""
    w = inputs.weight(6, 48, seed=3, stream="w8/pin")
    q, s = oracle.quantize_fp8_weight(w)
    rq, rs = fr.quant_fp8_tensor(w.tolist(), 6, 48)
    assert Fr(float(s)) == rs
    np.testing.assert_array_equal(q, np.array(rq, np.uint8))
    ties = _bits([[17.0, 19.0, 21.0, -23.0, 0.0, -0.0, 1e-3, 460.0, 2.25 * 2 ** -7, 500.0, -9.0, 13.0]])
    for sc in (1.0, 0.5, 2.0 ** -4):
        q, s = oracle.quantize_fp8_weight(ties, scale=sc)
        rq, _ = fr.quant_fp8_tensor(ties.tolist(), 1, ties.shape[1], scale=Fr(sc))
        np.testing.assert_array_equal(q, np.array(rq, np.uint8))
    q, _ = oracle.quantize_fp8_weight(ties, scale=1.0)
    assert q[0, 0] == 0x58 and q[0, 1] == 0x5A          # 17 -> 16 (even), 19 -> 20 (even)
    assert q[0, 7] == 0x7E and q[0, 9] == 0x7E          # 460, 500 saturate to 448


def test_fp8_weight_worked_example():
    """The pages' worked example: 0.176 with scale 0.01 maps to 18 (E4M3 0x59),
    dequantizing to 0.18."""
    w = _bits([[0.176]])
    q, s = oracle.quantize_fp8_weight(w, scale=0.01)
    assert q[0, 0] == 0x59 and oracle.code_value(oracle.E4M3, int(q[0, 0])) == 18.0
    assert abs(18.0 * float(s) - 0.18) < 1e-8


def test_fp8_weight_gemm_textbook():
    """Scale 1 and integer-valued weights and activations: the weight-only FP8
    linear equals the integer matrix product exactly."""
    rng = np.random.RandomState(4)
    a_int = rng.randint(-8, 9, size=(5, 64))
    w_int = rng.randint(-15, 16, size=(7, 64))
    a = _bits(a_int.astype(np.float64))
    w = _bits(w_int.astype(np.float64))
    q, s = oracle.quantize_fp8_weight(w, scale=1.0)
    r = oracle.gemm_bf16_fp8w(a, q, s)
    np.testing.assert_array_equal(r, (a_int @ w_int.T).astype(np.float64))


# ------------------------------------------------------------------ FP8 attention

def _softmax_attention_two_pass(q, k, v, sm):
    """Textbook attention in fp64: exact row maximum first, then the normalized
    probabilities times V (a different order of the same mathematics)."""
    S = (q @ k.T) * sm
    P = np.exp(S - S.max(axis=1, keepdims=True))
    return (P / P.sum(axis=1, keepdims=True)) @ v


def test_attention_online_equals_two_pass():
    """Without P quantization the oracle's attention is plain softmax attention,
    and so is the blocked running-maximum algorithm for any block size, including 1
    and the whole key range (a missing rescale or a stale maximum would not be)."""
    rng = np.random.RandomState(5)
    q, k, v = rng.randn(7, 16) * 2, rng.randn(200, 16) * 2, rng.randn(200, 16)
    ref = _softmax_attention_two_pass(q, k, v, 0.37)
    np.testing.assert_allclose(oracle.attention_rowmax(q, k, v, 0.37, quantize_p=False), ref, rtol=1e-12, atol=1e-14)
    for block in (1, 7, 64, 200):
        got = oracle.attention_online(q, k, v, 0.37, block=block, quantize_p=False)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_attention_quantized_p_independent_of_blocking():
    """With P quantized, the definition (P against the exact row maximum) is what
    the running-maximum algorithm computes when one block holds every key; with
    smaller blocks the keys before the last maximum move are encoded against a
    lower maximum, so the results differ (the reason the definition is two-pass)."""
    rng = np.random.RandomState(15)
    q, k, v = rng.randn(6, 16), rng.randn(256, 16), rng.randn(256, 16)
    ref = oracle.attention_rowmax(q, k, v, 0.5)
    np.testing.assert_allclose(oracle.attention_online(q, k, v, 0.5, block=256), ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.attention_online(q, k, v, 0.5, block=1000), ref, rtol=1e-13, atol=1e-15)
    assert np.abs(oracle.attention_online(q, k, v, 0.5, block=16) - ref).max() > 1e-6


def test_attention_p_quantizer_worked_values():
    """q(P) = E4M3 value of P * 256, / 256, worked by hand from the E4M3 grid:
    0.3 * 256 = 76.8 lies between 72 and 80 (midpoint 76) -> 80; 0.001 * 256 =
    0.256 lies between 0.25 and 0.28125 (midpoint 0.265625) -> 0.25; 2^-18 * 256 =
    2^-10 is the midpoint of 0 and the smallest subnormal 2^-9 -> even code 0."""
    got = oracle.attention_p_quantize(np.array([1.0, 0.3, 0.001, 2.0 ** -18, 0.5, 0.0])) * 256
    np.testing.assert_array_equal(got, [256.0, 80.0, 0.25, 0.0, 128.0, 0.0])


def test_attention_equal_scores_give_the_mean():
    """All keys equal: every score of a row is the same, P = 1 for every key
    (encoded exactly), so O is the mean of the V rows."""
    rng = np.random.RandomState(6)
    q = rng.randn(5, 8)
    k = np.tile(rng.randn(1, 8), (130, 1))
    v = rng.randn(130, 8)
    got = oracle.attention_rowmax(q, k, v, 0.5)
    np.testing.assert_allclose(got, np.tile(v.mean(axis=0), (5, 1)), rtol=1e-14, atol=1e-15)


def test_attention_dominant_key_selects_its_row():
    """One key whose score exceeds every other by 40: the others' P * 256 is below
    2^-17 and encodes to 0, so the numerator is V of that key, and the normalizer
    1 + sum exp(-40 or less) makes O that row to 1e-16."""
    d = 8
    q = np.zeros((1, d))
    q[0, 0] = 1.0
    k = np.zeros((150, d))
    k[97, 0] = 40.0
    v = np.random.RandomState(7).randn(150, d)
    got = oracle.attention_rowmax(q, k, v, 1.0)
    np.testing.assert_allclose(got[0], v[97], rtol=1e-15, atol=1e-15)


def test_attention_quantized_error_bound():
    """Each q(P) is within 2^-4 P of P (E4M3 relative half-step) or below 2^-18 in
    absolute value, so |O_q - O| <= (2^-4 + 2^-18 L) max|v| per element."""
    rng = np.random.RandomState(8)
    q, k, v = rng.randn(9, 32), rng.randn(256, 32), rng.randn(256, 32)
    exact = _softmax_attention_two_pass(q, k, v, 0.2)
    quant = oracle.attention_rowmax(q, k, v, 0.2)
    assert np.abs(quant - exact).max() <= (2.0 ** -4 + 2.0 ** -18 * 256) * np.abs(v).max()
    assert np.abs(quant - exact).max() > 0          # the quantization is really applied


def test_attention_fp8_codes_and_scales():
    """attention_fp8 forms scores from the code values with s_q s_k / sqrt(d) and
    applies s_v to the result: the same as attention_rowmax on dequantized
    operands."""
    rng = np.random.RandomState(9)
    heads, L, d = 2, 96, 16
    bits = [inputs.bf16_bits(rng.randn(heads * L, d)) for _ in range(3)]
    (qc, qs), (kc, ks), (vc, vs) = [oracle.quantize_fp8_weight(b) for b in bits]
    e43 = np.array([oracle.code_value(oracle.E4M3, c) for c in range(256)])
    got = oracle.attention_fp8(qc, qs, kc, ks, vc, vs, heads)
    for h in range(heads):
        sl = slice(h * L, (h + 1) * L)
        ref = oracle.attention_rowmax(e43[qc[sl]] * float(qs), e43[kc[sl]] * float(ks), e43[vc[sl]] * float(vs),
                                      1.0 / np.sqrt(d))
        np.testing.assert_allclose(got[h], ref, rtol=1e-12, atol=1e-14)
