"""CPU oracle for microscaling quantization and the block-scaled linear layer.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package; the product path
(``microscaling_quantized_dit_amd``) never does and shares no code with it.

The arithmetic lives in ``mxq_oracle.c`` (plain scalar C, fp64, exact
comparisons); this module builds it with gcc on first use and wraps it for
numpy arrays.  See the header of ``mxq_oracle.c`` for the definitions followed
and the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

E4M3, E5M2, E2M1 = 0, 1, 2
EPI_NONE, EPI_BIAS, EPI_BIAS_GELU_TANH = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxq_oracle.c")
_LIB = os.path.join(_HERE, "liborc.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (OpenMP, no fast-math) into oracle/liborc.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-D_GNU_SOURCE",
               "-Wall", "-Wextra", "-Werror", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i64, i32, f64, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_float
        sig = {
            "orc_bf16_value": (f64, [ctypes.c_uint16]),
            "orc_code_value": (f64, [i32, i32]),
            "orc_e8m0_value": (f64, [i32]),
            "orc_round_quotient": (i32, [i32, f64, f64]),
            "orc_round_quotient_array": (None, [i32, P, f64, i64, P]),
            "orc_rn_fp32_div": (f32, [f64, f64]),
            "orc_quantize_mxfp8": (i32, [P, i64, i64, i32, P, P]),
            "orc_nvfp4_global_scale": (f32, [P, i64]),
            "orc_nvfp4_calibrate": (f32, [P, i64, f32]),
            "orc_fp8_tensor_scale": (f32, [P, i64]),
            "orc_quantize_fp8_tensor": (i32, [P, i64, i64, P, P, P]),
            "orc_quantize_nvfp4": (i32, [P, i64, i64, P, P, P, P]),
            "orc_dequant_mxfp8": (None, [P, P, i64, i32, P, i64, P]),
            "orc_dequant_nvfp4": (None, [P, P, f32, i64, P, i64, P]),
            "orc_linear": (None, [P, P, f64, P, i32, i64, i64, i64, P]),
            "orc_max_threads": (i32, []),
            "orc_set_threads": (None, [i32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _as_u16(x) -> np.ndarray:
    """bf16 bit patterns as a C-contiguous uint16 array (accepts numpy uint16/int16
    arrays or CPU torch bfloat16 tensors)."""
    if hasattr(x, "dtype") and str(x.dtype) == "torch.bfloat16":
        import torch
        x = x.detach().cpu().contiguous().view(torch.int16).numpy()
    a = np.ascontiguousarray(x)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bit patterns (uint16), got %s" % a.dtype)
    return a


# ------------------------------------------------------------------ formats

def bf16_value(bits: int) -> float:
    return _load().orc_bf16_value(bits)


def code_value(fmt: int, code: int) -> float:
    return _load().orc_code_value(fmt, code)


def e8m0_value(code: int) -> float:
    return _load().orc_e8m0_value(code)


def round_quotient(fmt: int, num: float, den: float) -> int:
    """Magnitude code of RNE_sat(num/den) (num >= 0, den > 0)."""
    return _load().orc_round_quotient(fmt, num, den)


def round_quotient_array(fmt: int, num: np.ndarray, den: float) -> np.ndarray:
    num = np.ascontiguousarray(num, dtype=np.float64)
    out = np.empty(num.shape, np.uint8)
    _load().orc_round_quotient_array(fmt, _ptr(num), den, num.size, _ptr(out))
    return out


def rn_fp32_div(a: float, d: float) -> np.float32:
    return np.float32(_load().orc_rn_fp32_div(a, d))


# --------------------------------------------------------------- quantizers

def quantize_mxfp8(x, fmt: int = E4M3):
    """bf16 [rows, cols] -> (codes u8 [rows, cols], E8M0 scales u8 [rows, cols/32])."""
    a = _as_u16(x)
    rows, cols = a.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 32), np.uint8)
    rc = _load().orc_quantize_mxfp8(_ptr(a), rows, cols, fmt, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError("orc_quantize_mxfp8: bad arguments (rc=%d)" % rc)
    return q, s


def nvfp4_global_scale(x) -> np.float32:
    a = _as_u16(x)
    return np.float32(_load().orc_nvfp4_global_scale(_ptr(a), a.size))


def nvfp4_calibrate(batches, running: float = 0.0) -> np.float32:
    """Static NVFP4 decode scale from calibration tensors: the running maximum of
    RN_fp32(amax / 2688) over the batches, starting from `running`."""
    r = np.float32(running)
    for x in batches:
        a = _as_u16(x)
        r = np.float32(_load().orc_nvfp4_calibrate(_ptr(a), a.size, float(r)))
    return r


def quantize_nvfp4(x, global_scale=None):
    """bf16 [rows, cols] -> (packed codes u8 [rows, cols/2], E4M3 scales u8
    [rows, cols/16], fp32 global decode scale).  global_scale None = dynamic."""
    a = _as_u16(x)
    rows, cols = a.shape
    q = np.empty((rows, cols // 2), np.uint8)
    s = np.empty((rows, cols // 16), np.uint8)
    g_out = np.zeros(1, np.float32)
    g_in = None if global_scale is None else np.array([global_scale], np.float32)
    rc = _load().orc_quantize_nvfp4(_ptr(a), rows, cols, None if g_in is None else _ptr(g_in),
                                    _ptr(q), _ptr(s), _ptr(g_out))
    if rc != 0:
        raise ValueError("orc_quantize_nvfp4: bad arguments (rc=%d)" % rc)
    return q, s, np.float32(g_out[0])


def fp8_tensor_scale(x) -> np.float32:
    a = _as_u16(x)
    return np.float32(_load().orc_fp8_tensor_scale(_ptr(a), a.size))


def quantize_fp8_weight(x, scale=None):
    """Weight-only FP8: bf16 [rows, cols] -> (E4M3 codes u8 [rows, cols], fp32
    per-tensor decode scale).  scale None = RN_fp32(amax / 448)."""
    a = _as_u16(x)
    rows, cols = a.shape
    q = np.empty((rows, cols), np.uint8)
    s_out = np.zeros(1, np.float32)
    s_in = None if scale is None else np.array([scale], np.float32)
    rc = _load().orc_quantize_fp8_tensor(_ptr(a), rows, cols, None if s_in is None else _ptr(s_in), _ptr(q),
                                         _ptr(s_out))
    if rc != 0:
        raise ValueError("orc_quantize_fp8_tensor: bad arguments (rc=%d)" % rc)
    return q, np.float32(s_out[0])


# -------------------------------------------------------------- dequant / GEMM

def _rows(row_idx, n_all):
    if row_idx is None:
        return None, n_all
    r = np.ascontiguousarray(row_idx, dtype=np.int64)
    return r, r.size


def dequant_mxfp8(q, s, fmt: int = E4M3, row_idx=None) -> np.ndarray:
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.uint8)
    cols = q.shape[1]
    r, n = _rows(row_idx, q.shape[0])
    out = np.empty((n, cols), np.float64)
    _load().orc_dequant_mxfp8(_ptr(q), _ptr(s), cols, fmt, None if r is None else _ptr(r), n, _ptr(out))
    return out


def dequant_nvfp4(q, s, global_scale, row_idx=None) -> np.ndarray:
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.uint8)
    cols = q.shape[1] * 2
    r, n = _rows(row_idx, q.shape[0])
    out = np.empty((n, cols), np.float64)
    _load().orc_dequant_nvfp4(_ptr(q), _ptr(s), float(global_scale), cols,
                              None if r is None else _ptr(r), n, _ptr(out))
    return out


def linear(a_deq: np.ndarray, w_deq: np.ndarray, alpha: float = 1.0, bias=None,
           epi: int = EPI_NONE) -> np.ndarray:
    """fp64 epi(alpha * a @ w.T + bias), a [m, K], w [N, K] dequantized operands."""
    a = np.ascontiguousarray(a_deq, np.float64)
    w = np.ascontiguousarray(w_deq, np.float64)
    m, K = a.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("K mismatch")
    b = None
    if epi != EPI_NONE:
        b = _as_u16(bias).reshape(-1)
        if b.size != N:
            raise ValueError("bias must have N entries")
    out = np.empty((m, N), np.float64)
    _load().orc_linear(_ptr(a), _ptr(w), float(alpha), None if b is None else _ptr(b), epi, m, N, K, _ptr(out))
    return out


def gemm_mxfp8(a_q, a_s, w_q, w_s, a_fmt=E4M3, w_fmt=E4M3, bias=None, epi=EPI_NONE, row_idx=None):
    """Reference output (fp64, unrounded) of C = A W^T (+bias) (GELU) for MXFP8 operands."""
    a = dequant_mxfp8(a_q, a_s, a_fmt, row_idx)
    w = dequant_mxfp8(w_q, w_s, w_fmt)
    return linear(a, w, 1.0, bias, epi)


_TABLES = {}


def _table(name):
    """Decoded value of every bf16 bit pattern / every E4M3 code (fp64)."""
    if name not in _TABLES:
        if name == "bf16":
            _TABLES[name] = np.array([bf16_value(b) for b in range(65536)], np.float64)
        else:
            _TABLES[name] = np.array([code_value(E4M3, c) if (c & 0x7F) != 0x7F else np.nan for c in range(256)],
                                     np.float64)
    return _TABLES[name]


def gemm_bf16_fp8w(a_bits, w_q, w_scale, bias=None, epi=EPI_NONE, row_idx=None):
    """Weight-only FP8 linear: r = epi(s_w * A . val(W)^T + bias) in fp64, with A
    the exact bf16 values and W the E4M3 values (s_w applied once, like alpha)."""
    a = _as_u16(a_bits)
    if row_idx is not None:
        a = a[np.asarray(row_idx)]
    a_deq = _table("bf16")[a]
    w_deq = _table("e4m3")[np.asarray(w_q, np.uint8)]
    return linear(a_deq, w_deq, float(w_scale), bias, epi)


def gemm_nvfp4(a_q, a_s, a_g, w_q, w_s, w_g, bias=None, epi=EPI_NONE, row_idx=None):
    """Reference output (fp64, unrounded) for NVFP4 operands:
    epi(alpha * sum_k val(qa) S_a val(qw) S_w + bias) with alpha = s_ga * s_gw.
    Operands are dequantized without the global scales so every product is
    exact in fp64 (6 significant bits each); alpha (48 bits) is exact too."""
    a = dequant_nvfp4(a_q, a_s, 1.0, row_idx)
    w = dequant_nvfp4(w_q, w_s, 1.0)
    alpha = float(np.float64(np.float32(a_g)) * np.float64(np.float32(w_g)))
    return linear(a, w, alpha, bias, epi)


# ------------------------------------------------------------- FP8 attention
#
# Reading of "multi-head attention in FP8" (page "NVIDIA Blackwell平台FP4量化技术解析与
# 图像生成优化", section 2.1, mixed-precision configuration: fully connected layers
# in FP4, multi-head attention in FP8, normalization in FP16): per head,
# O = softmax(Q K^T / sqrt(d)) V with
#   - Q, K, V each quantized per tensor to E4M3 (the per-tensor quantizer above);
#   - both products on FP8 operands: S from the Q and K codes, and P V with the
#     probabilities P encoded as E4M3 codes of P * 256 (P <= 1, so at most 256);
#   - softmax against the row's exact maximum: m = max_j S_j over every key,
#     P_j = exp(S_j - m), l = sum_j P_j (unquantized), O = sum_j q(P_j) V_j / l.
# The quantized P depends only on the row's scores, not on any order or blocking
# of the keys.

ATTN_P_SCALE = 256.0     # P is encoded as E4M3 codes of P * 256


def attention_p_quantize(p: np.ndarray) -> np.ndarray:
    """q(P) = val(RN_E4M3(P * 256)) / 256 elementwise for 0 <= P <= 1 (fp64)."""
    p = np.asarray(p, np.float64)
    codes = round_quotient_array(E4M3, (p * ATTN_P_SCALE).ravel(), 1.0)
    return (_table("e4m3")[codes] / ATTN_P_SCALE).reshape(p.shape)


def attention_rowmax(q, k, v, sm_scale: float, quantize_p: bool = True, return_p: bool = False):
    """Softmax attention of fp64 rows q [R, d] over k, v [L, d], in the textbook
    two-pass order: scores S = sm_scale * q . k, the row maximum m over all keys,
    P = exp(S - m), l = sum P, O = sum q(P) v / l (q(P) = P when quantize_p is
    False).  return_p: also (P [R, L], l [R])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    S = (q @ k.T) * sm_scale
    m = S.max(axis=1)
    P = np.exp(S - m[:, None])
    l = P.sum(axis=1)
    Pq = attention_p_quantize(P) if quantize_p else P
    O = (Pq @ v) / l[:, None]
    return (O, P, l) if return_p else O


def attention_online(q, k, v, sm_scale: float, block: int = 64, quantize_p: bool = True):
    """The single-pass (running maximum) algorithm over key blocks of `block`, in
    key order: m' = max(m, max S), P = exp(S - m'), l = l e^(m - m') + sum P,
    acc = acc e^(m - m') + q(P) v, O = acc / l.  Not the definition above (with
    quantize_p its P is encoded against the running maximum); it equals it when
    one block holds every key, and without quantization for any block size, which
    the pins check."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    R, L = q.shape[0], k.shape[0]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, v.shape[1]))
    for b0 in range(0, L, block):
        S = (q @ k[b0:b0 + block].T) * sm_scale
        m_new = np.maximum(m, S.max(axis=1))
        alpha = np.exp(m - m_new)
        P = np.exp(S - m_new[:, None])
        l = l * alpha + P.sum(axis=1)
        Pq = attention_p_quantize(P) if quantize_p else P
        acc = acc * alpha[:, None] + Pq @ v[b0:b0 + block]
        m = m_new
    return acc / l[:, None]


def attention_fp8(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, heads: int, row_idx=None,
                  return_p: bool = False):
    """FP8 attention, fp64 result [heads, R, d]: codes [heads * L, d] (head h is
    rows h*L .. h*L + L - 1), per-tensor fp32 decode scales, softmax scale
    1/sqrt(d).  Scores are formed as (s_q s_k / sqrt(d)) * sum val(q) val(k) -- the
    code products and their sum are exact in fp64 -- and V enters as its code
    values, with s_v applied to the result.  row_idx: query rows within each head
    (all when None).  return_p: also the exact probabilities P [heads, R, L] and
    normalizers l [heads, R] (for the tolerance of a comparison)."""
    e43 = _table("e4m3")
    qv = e43[np.asarray(q_codes, np.uint8)]
    kv = e43[np.asarray(k_codes, np.uint8)]
    vv = e43[np.asarray(v_codes, np.uint8)]
    n, d = qv.shape
    L = n // heads
    sm = float(np.float64(np.float32(q_scale)) * np.float64(np.float32(k_scale))) / np.sqrt(d)
    sv = float(np.float32(v_scale))
    out, ps, ls = [], [], []
    for h in range(heads):
        qh = qv[h * L:(h + 1) * L]
        if row_idx is not None:
            qh = qh[np.asarray(row_idx)]
        o, p, l = attention_rowmax(qh, kv[h * L:(h + 1) * L], vv[h * L:(h + 1) * L], sm, return_p=True)
        out.append(sv * o)
        ps.append(p)
        ls.append(l)
    if return_p:
        return np.stack(out), np.stack(ps), np.stack(ls)
    return np.stack(out)


def max_threads() -> int:
    return _load().orc_max_threads()


def set_threads(n: int) -> None:
    _load().orc_set_threads(n)


# ------------------------------------------------------------- tolerance check

def compare(gpu_bf16_values: np.ndarray, ref: np.ndarray) -> dict:
    """Error of a bf16 GEMM output against the fp64 reference.

    max_rel = max |g - r| / max(|r|, rms(r)) (the rms floor keeps cancellation
    near zero from dominating); also the relative Frobenius error and the max
    absolute error."""
    g = np.asarray(gpu_bf16_values, np.float64)
    r = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    diff = np.abs(g - r)
    floor = np.maximum(np.abs(r), rms if rms > 0 else 1.0)
    return {
        "max_rel": float((diff / floor).max()) if r.size else 0.0,
        "fro_rel": float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)) if r.size else 0.0,
        "max_abs": float(diff.max()) if r.size else 0.0,
        "rms_ref": rms,
    }
