"""FP8 attention on the GPU against the oracle (the reading of "multi-head
attention in FP8", page "NVIDIA Blackwell平台FP4量化技术解析与图像生成优化", section 2.1:
P encoded as E4M3 codes of 256 P against the row's exact maximum, no blocking).

V quantizer: codes and scale bit-exact (its layout is the oracle's codes
rearranged as documented in include/mxq.h).

Attention tolerance, derived from the kernel's arithmetic.  Both products run on
v_mfma_scale_f32_32x32x64_f8f6f4, whose accumulation was measured on gfx950 with
crafted operands (exact sums known): the products of each group of 8 consecutive
K positions are summed after truncating every product to the bits at or above
2^(e - 13), e the exponent of the group's largest product; group sums and the
accumulator are then added at fp32 precision.  A group's largest product (8
significant bits) is exact, and a truncated product loses less than itself; taking
a 12-bit window for margin, a sum of products p has error at most
    T(p) = sum over groups, over every product but the group's largest, of
           min(|p|, 2^-12 max |p| in the group)  +  2^-22 sum |p|.

The kernel computes, per query row i and key j, x'_ij = fma(s'_ij, c2', 8 - m'_i)
with s'_ij the matrix-core sum of the 128 exact code products of Q_i and K_j, c2'
the fp32 scale s_q s_k log2(e) / sqrt(128) and m'_i = c2' max_j s'_ij, and encodes
2^x'_ij (= 256 P'_ij) with round-to-nearest-even.  Its relative error against the
oracle's exact 256 P_ij is at most
    eps_ij = ln 2 [c2 (E_ij + max_j E_ij) + 2^-21 (|x_ij - m_i| + |m_i| + 16)] + 2^-21,
    E_ij = T(val(q_ic) val(k_jc) over c)   (the score sum's error, for the key and the maximum),
with the head dimension in groups of 8 consecutive channels; c2', the product by
c2', the offset and the fma add at most 2^-24 relative each in the exponent, and the
hardware exp2 at most 2^-21 (measured: 0.78 ulp).  So the kernel's code can differ
from the oracle's only for keys whose exact 256 P lies within eps_ij 256 P of a
rounding midpoint between two E4M3 values ("ambiguous" keys), and then by one code
step D_ij.  The P.V sum groups keys in runs of 8 of the kernel's V layout (columns
8u .. 8u + 7 of each 64-key block of mxq_quantize_fp8_v's order).  Per element:
  F_ic = s_v sum_{j ambiguous} D_ij / 256 |val(v_jc)| / l_i               (code steps)
  B_ic = s_v [T(q(P_ij) val(v_jc) over j) + L 2^-23 sum_j q(P_ij) |val(v_jc)|] / l_i
       + (max_j eps_ij + L 2^-24 + 2^-22) |r_ic|                          (fp32 normalizer, scaling)
  C_ic = 2^-8 (|r_ic| + F_ic + B_ic)                                      (one bf16 rounding)
and |g_ic - r_ic| <= F + B + C
must hold everywhere.  Over the whole output, ||g - r|| <= 3e-3 ||r|| + ||F|| + ||B||:
bf16 rounding alone has a relative rms of about 1.3e-3, the GEMM tests' bound."""
import numpy as np
import pytest

import oracle
from microscaling_quantized_dit_amd import inputs

pytestmark = pytest.mark.gpu

FRO_REL = 3e-3
LN2 = float(np.log(2.0))
# every non-negative finite E4M3 value (codes 0..126), increasing
E4M3_GRID = np.array([oracle.code_value(oracle.E4M3, c) for c in range(127)])
E43 = np.array([oracle.code_value(oracle.E4M3, c) if (c & 0x7F) != 0x7F else np.nan for c in range(256)])


def _t(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _np(t):
    return t.cpu().numpy()


def vt_layout(codes, heads, L, d=128):
    """Oracle codes [heads * L, d] -> the attention's V layout [heads, d, L]."""
    c = np.asarray(codes).reshape(heads, L, d)
    out = np.empty((heads, d, L), np.uint8)
    s = np.arange(32)
    for b in range(L // 64):
        for g in range(2):
            keys = 64 * b + 32 * (s // 16) + 8 * ((s % 16) // 4) + 4 * g + s % 4
            out[:, :, 64 * b + 32 * g + s] = c[:, keys, :].transpose(0, 2, 1)
    return out


def _quantized(mxq, heads, L, seed, gain=1.0):
    """Q, K, V quantized on the GPU, each checked bit for bit against the oracle."""
    q, k, v = inputs.attention_qkv(heads, L, seed=seed, stream="attn%d" % seed, gain=gain)
    dev = {}
    for name, bits in (("q", q), ("k", k)):
        c, s = mxq.quantize_fp8_weight(inputs.to_torch(bits, "cuda"))
        rc, rs = oracle.quantize_fp8_weight(bits)
        np.testing.assert_array_equal(_np(c), rc)
        assert np.float32(_np(s)[0]).tobytes() == np.float32(rs).tobytes()
        dev[name] = (c, s, rc, rs)
    c, s = mxq.quantize_fp8_v(inputs.to_torch(v, "cuda"), heads)
    rc, rs = oracle.quantize_fp8_weight(v)
    np.testing.assert_array_equal(_np(c), vt_layout(rc, heads, L))
    assert np.float32(_np(s)[0]).tobytes() == np.float32(rs).tobytes()
    dev["v"] = (c, s, rc, rs)
    return dev


def _vt_key_groups(L):
    """Keys of each run of 8 positions the P.V matrix-core sum adds as one group:
    columns 8u .. 8u + 7 of every 64-key block in the V layout (column 32g + s holds
    key 32 (s / 16) + 8 ((s % 16) / 4) + 4g + s % 4 of the block).  [L / 8, 8]."""
    col = np.arange(64)
    g, s = col // 32, col % 32
    perm = 32 * (s // 16) + 8 * ((s % 16) // 4) + 4 * g + s % 4
    return (64 * np.arange(L // 64)[:, None] + perm[None, :]).reshape(-1, 8)


def _truncation(prod):
    """The measured matrix-core bound T without its fp32 term: prod [..., n_groups, 8]
    of non-negative |products| -> sum over groups of min(|p|, 2^-12 max) over all
    but each group's largest product."""
    mx = prod.max(axis=-1, keepdims=True)
    lost = np.minimum(prod, 2.0 ** -12 * mx).sum(axis=-1) - np.minimum(mx[..., 0], 2.0 ** -12 * mx[..., 0])
    return lost.sum(axis=-1)


def tolerance(qv, kv, vv, qs, ks, vs, heads, rows, P, l, r):
    """(per-element bound F + B + C, Frobenius allowance ||F|| + ||B||) as derived in
    the module docstring.  qv, kv, vv: code values [heads * L, d]; P, l: the
    oracle's exact probabilities [heads, R, L] and normalizers [heads, R]; r: the
    oracle's output [heads, R, d]."""
    n, d = qv.shape
    L = n // heads
    c2 = float(np.float64(np.float32(qs)) * np.float64(np.float32(ks))) * np.log2(np.e) / np.sqrt(d)
    sv = float(np.float32(vs))
    groups = _vt_key_groups(L)
    bound = np.empty_like(r)
    fro = 0.0
    for h in range(heads):
        qh = qv[h * L:(h + 1) * L][rows]
        kh = kv[h * L:(h + 1) * L]
        vh = np.abs(vv[h * L:(h + 1) * L])
        prod = np.abs(qh)[:, None, :] * np.abs(kh)[None, :, :]                  # [R, L, d]
        E = _truncation(prod.reshape(len(rows), L, d // 8, 8)) + 2.0 ** -22 * prod.sum(axis=2)
        x = c2 * (qh @ kh.T)
        m = x.max(axis=1, keepdims=True)
        eps = LN2 * (c2 * (E + E.max(axis=1, keepdims=True)) + 2.0 ** -21 * (np.abs(x - m) + np.abs(m) + 16.0)) \
            + 2.0 ** -21
        y = 256.0 * P[h]
        i = np.clip(np.searchsorted(E4M3_GRID, y, side="right") - 1, 0, len(E4M3_GRID) - 2)
        lo, hi = E4M3_GRID[i], E4M3_GRID[i + 1]
        lo_prev = E4M3_GRID[np.maximum(i - 1, 0)]
        amb_up = np.abs(y - 0.5 * (lo + hi)) <= eps * y
        amb_dn = (i > 0) & (np.abs(y - 0.5 * (lo_prev + lo)) <= eps * y)
        step = np.where(amb_up, hi - lo, 0.0) + np.where(amb_dn, lo - lo_prev, 0.0)
        li = l[h][:, None]
        F = sv * (step / 256.0) @ vh / li
        qP = oracle.attention_p_quantize(P[h])
        pv = qP[:, groups][:, :, :, None] * vh[groups][None, :, :, :]            # [R, L/8, 8, d]
        Tpv = _truncation(np.moveaxis(pv, 3, 1))                                 # [R, d]
        B = sv * (Tpv + L * 2.0 ** -23 * (qP @ vh)) / li \
            + (eps.max(axis=1, keepdims=True) + L * 2.0 ** -24 + 2.0 ** -22) * np.abs(r[h])
        C = 2.0 ** -8 * (np.abs(r[h]) + F + B)
        bound[h] = F + B + C
        fro += float(np.sum((F + B) ** 2))
    return bound, np.sqrt(fro)


def _run(mxq, dev, heads, L, rows=None):
    """(GPU output, oracle output, per-element bound, Frobenius allowance)."""
    import torch
    (qc, qs, rqc, rqs), (kc, ks, rkc, rks), (vc, vs, rvc, rvs) = dev["q"], dev["k"], dev["v"]
    o = mxq.attention_fp8(qc, qs, kc, ks, vc, vs, heads)
    g = inputs.bf16_to_f64(o.cpu().view(torch.int16).numpy()).reshape(heads, L, 128)
    sel = np.arange(L) if rows is None else np.asarray(rows)
    r, P, l = oracle.attention_fp8(rqc, rqs, rkc, rks, rvc, rvs, heads, row_idx=sel, return_p=True)
    bound, fro = tolerance(E43[np.asarray(rqc)], E43[np.asarray(rkc)], E43[np.asarray(rvc)], rqs, rks, rvs,
                           heads, sel, P, l, r)
    return g[:, sel], r, bound, fro


def _close(g, r, bound, fro, what):
    e = oracle.compare(g, r)
    err = np.abs(g - r)
    assert np.linalg.norm(g - r) <= FRO_REL * np.linalg.norm(r) + fro, (what, e, fro)
    bad = err > bound
    assert not bad.any(), (what, e, int(bad.sum()), float((err / bound).max()))


def test_quantize_fp8_v_static_scale(mxq):
    """Static-scale V codes in the attention layout, bit-exact."""
    import torch
    _, _, v = inputs.attention_qkv(2, 256, seed=3, stream="vstatic")
    sc = torch.tensor([0.004], dtype=torch.float32, device="cuda")
    c, s = mxq.quantize_fp8_v(inputs.to_torch(v, "cuda"), 2, scale=sc)
    rc, rs = oracle.quantize_fp8_weight(v, scale=0.004)
    np.testing.assert_array_equal(_np(c), vt_layout(rc, 2, 256))


@pytest.mark.parametrize("L,gain", [(128, 1.0), (256, 1.0), (512, 3.0), (384, 6.0)])
def test_attention_full(mxq, L, gain):
    """Two heads, every query row: flat (gain 1) to sharp (gain 6) softmax."""
    dev = _quantized(mxq, 2, L, seed=L, gain=gain)
    _close(*_run(mxq, dev, 2, L), "L=%d gain=%g" % (L, gain))


def test_attention_rising_maximum(mxq):
    """Keys whose scores grow along the sequence, so each row's maximum lies in its
    last block: the first pass must carry the maximum over every block."""
    import torch
    heads, L, d = 1, 512, 128
    rng = np.random.RandomState(4)
    q = np.abs(rng.randn(L, d)) * 0.5
    k = np.abs(rng.randn(L, d)) * 0.5 * (1.0 + np.arange(L)[:, None] / 64.0)
    v = rng.randn(L, d)
    bits = [inputs.bf16_bits(a) for a in (q, k, v)]
    dev = {}
    for name, b in (("q", bits[0]), ("k", bits[1])):
        c, s = mxq.quantize_fp8_weight(inputs.to_torch(b, "cuda"))
        rc, rs = oracle.quantize_fp8_weight(b)
        dev[name] = (c, s, rc, rs)
    c, s = mxq.quantize_fp8_v(inputs.to_torch(bits[2], "cuda"), heads)
    rc, rs = oracle.quantize_fp8_weight(bits[2])
    dev["v"] = (c, s, rc, rs)
    _close(*_run(mxq, dev, heads, L), "rising maximum")


def _static_case(mxq, qi, ki, v_bits, ks, heads):
    """Q codes = qi (scale 1), K quantized with the static scale ks, V dynamic."""
    import torch
    dev = {}
    for name, vals, sc in (("q", qi, 1.0), ("k", ki * np.float64(ks), float(ks))):
        b = inputs.bf16_bits(vals)
        st = torch.tensor([sc], dtype=torch.float32, device="cuda")
        c, s = mxq.quantize_fp8_weight(inputs.to_torch(b, "cuda"), scale=st)
        rc, rs = oracle.quantize_fp8_weight(b, scale=sc)
        np.testing.assert_array_equal(_np(c), rc)
        dev[name] = (c, s, rc, rs)
    c, s = mxq.quantize_fp8_v(inputs.to_torch(v_bits, "cuda"), heads)
    rc, rs = oracle.quantize_fp8_weight(v_bits)
    dev["v"] = (c, s, rc, rs)
    return dev


def test_attention_exact_sums_fractional_p(mxq):
    """Scores from a single nonzero code product each (channel 0), so the matrix-core
    sums are exact, with fractional log2 values (E4M3 values in [-6, 0] times a scale
    that makes the log2-domain score that value): P is not a power of two, its 256 P
    lies between E4M3 values, and each row's maximum (log2 score 0) sits in its last
    64-key block.  Encoding P against a running maximum instead of the row's own
    would move almost every code; the derived bound is tight here because the only
    inexact steps are fp32 roundings."""
    heads, L, d = 2, 512, 128
    rng = np.random.RandomState(21)
    grid = np.array([v for v in E4M3_GRID if v <= 6.0])
    qi = np.zeros((heads * L, d))
    qi[:, 0] = 1.0
    ki = np.zeros((heads * L, d))
    ki[:, 0] = -rng.choice(grid[grid > 0.1], size=heads * L)       # log2 scores in (-6, -0.1)
    for h in range(heads):
        ki[h * L + L - 1 - rng.randint(0, 64), 0] = 0.0               # the maximum, in the last block
    ks = np.float32(np.sqrt(128.0) / np.log2(np.e))
    _, _, v = inputs.attention_qkv(heads, L, seed=22, stream="fracp")
    dev = _static_case(mxq, qi, ki, v, ks, heads)
    g, r, bound, fro = _run(mxq, dev, heads, L)
    _close(g, r, bound, fro, "exact sums, fractional P")
    # the case really depends on where P is encoded: the online (running maximum)
    # algorithm over 64-key blocks moves the result far beyond the bound
    e43 = E43
    qv, kv, vv = e43[dev["q"][2]], e43[dev["k"][2]], e43[dev["v"][2]]
    sm = float(np.float64(dev["q"][3]) * np.float64(dev["k"][3])) / np.sqrt(d)
    online = np.stack([float(dev["v"][3]) * oracle.attention_online(qv[h * L:(h + 1) * L], kv[h * L:(h + 1) * L],
                                                                    vv[h * L:(h + 1) * L], sm, block=64)
                       for h in range(heads)])
    assert (np.abs(online - r) > bound).sum() > 100


def test_attention_flux_shape(mxq):
    """FLUX joint attention: 24 heads x 4608 tokens x 128; 16 query rows of every
    head against the oracle."""
    heads, L = 24, 4608
    dev = _quantized(mxq, heads, L, seed=0)
    rows = np.sort(np.concatenate([[0, L - 1], np.random.RandomState(5).choice(L, 14, replace=False)]))
    _close(*_run(mxq, dev, heads, L, rows=rows), "flux")


def test_attention_exact_decisions(mxq):
    """Inputs on which no code can be disputed: Q and K small integers, K quantized
    with the static scale sqrt(128) / log2(e), so every score is an integer in the
    log2 domain and every P an exact power of two (2^0 .. 2^-14 here): 256 P is an
    E4M3 value on both sides, far from any midpoint.  The output must then meet the
    plain GEMM bound, with no allowance -- a wrong key order, scale or rescale
    would not."""
    import torch
    heads, L, d = 2, 384, 128
    rng = np.random.RandomState(11)
    qi = np.zeros((heads * L, d))
    ki = np.zeros((heads * L, d))
    qi[:, 0] = 1.0
    ki[:, 0] = -rng.randint(0, 15, size=heads * L)        # score of key j: -n_j (max 0)
    qi[:, 1:9] = rng.randint(-1, 2, size=(heads * L, 8))  # and cross terms that cancel:
    ki[:, 1:9] = 0.0                                      # K is zero there
    ks = np.float32(np.sqrt(128.0) / np.log2(np.e))
    qb = inputs.bf16_bits(qi)
    kb = inputs.bf16_bits(ki * np.float64(ks))
    _, _, v = inputs.attention_qkv(heads, L, seed=12, stream="exact")
    dev = {}
    for name, b, sc in (("q", qb, 1.0), ("k", kb, float(ks))):
        st = torch.tensor([sc], dtype=torch.float32, device="cuda")
        c, s = mxq.quantize_fp8_weight(inputs.to_torch(b, "cuda"), scale=st)
        rc, rs = oracle.quantize_fp8_weight(b, scale=sc)
        np.testing.assert_array_equal(_np(c), rc)
        dev[name] = (c, s, rc, rs)
    c, s = mxq.quantize_fp8_v(inputs.to_torch(v, "cuda"), heads)
    rc, rs = oracle.quantize_fp8_weight(v)
    dev["v"] = (c, s, rc, rs)
    # the K codes are exactly the integers: the scores are -n_j on both sides
    e43 = np.array([oracle.code_value(oracle.E4M3, cc) for cc in range(256)])
    np.testing.assert_array_equal(e43[dev["k"][2]][:, 0], ki[:, 0])
    g, r, _, _ = _run(mxq, dev, heads, L)
    e = oracle.compare(g, r)
    assert e["max_rel"] <= 1e-2 and e["fro_rel"] <= FRO_REL, e
