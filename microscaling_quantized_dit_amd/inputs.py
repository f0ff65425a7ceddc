"""Seeded synthetic inputs (bf16 bit patterns) shaped like FLUX-style DiT linears.

This module only draws numbers: it holds none of the quantization or GEMM
arithmetic and imports neither the HIP binding nor the oracle, so both sides
can take their inputs from it.

Generator: counter-based SplitMix64 (Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) -- element i of stream s under
seed k is mix(base(k, s) + (i + 1) * golden) -- then Box-Muller in fp64 and one
round-to-nearest-even to bf16.  Being counter-based, any slice can be drawn
independently, so large tensors are drawn in parallel chunks with identical
results.

Workload recipes (the pages run FLUX.1-dev at 1024x1024 with 512 text tokens,
i.e. 4096 image + 512 text = 4608 tokens per image; the quality datasets and
trained weights they use are not available, so these seeded tensors stand in):
  * activations: N(0, 1) times a per-column log-normal magnitude exp(z_k),
    z_k ~ N(0, 1) shared by every row, then 0.1% of entries (exactly
    round(0.001 * numel) distinct seeded positions) multiplied by 50;
  * the tiny case: N(0, 1) with 1% outliers x20, weights N(0, 0.02);
  * long-sequence case: N(0, 1) with 0.1% outliers x50;
  * weights N(0, 1/sqrt(K)); bias N(0, 1/sqrt(K));
  * attention (FLUX joint attention: 24 heads of dimension 128 over the 4608
    tokens): Q and K N(0, gain) -- FLUX normalizes q and k per head (RMSNorm),
    so unit scale is the plain stand-in, gain > 1 sharpens the softmax -- and
    V N(0, 1), each [heads * L, 128] with head h in rows h*L .. h*L + L - 1.
Standard deviations are the second argument of N(., .).
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _base(seed: int, stream: str) -> np.uint64:
    h = zlib.crc32(stream.encode()) & 0xFFFFFFFF
    with np.errstate(over="ignore"):
        z = np.array([(seed * 0x100000001B3 + h) & 0xFFFFFFFFFFFFFFFF], np.uint64)
        return _mix(z)[0]


def _u64(base: np.uint64, start: int, n: int) -> np.ndarray:
    idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(base + idx * _GOLDEN)


def _normal_chunk(base: np.uint64, start: int, n: int) -> np.ndarray:
    z = _u64(base, 2 * start, 2 * n)
    u1 = ((z[0::2] >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)
    u2 = (z[1::2] >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(n: int, seed: int, stream: str) -> np.ndarray:
    """n draws of N(0, 1) in fp64 from (seed, stream)."""
    base = _base(seed, stream)
    out = np.empty(n, np.float64)
    starts = list(range(0, n, _CHUNK))

    def work(s):
        m = min(_CHUNK, n - s)
        out[s:s + m] = _normal_chunk(base, s, m)

    if len(starts) <= 1:
        for s in starts:
            work(s)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(work, starts))
    return out


def distinct_positions(count: int, numel: int, seed: int, stream: str) -> np.ndarray:
    """`count` distinct indices in [0, numel), in order of first draw."""
    if count <= 0:
        return np.zeros(0, np.int64)
    if count > numel:
        raise ValueError("more positions than elements")
    base = _base(seed, stream)
    got = np.zeros(0, np.int64)
    drawn = 0
    while got.size < count:
        need = int((count - got.size) * 1.25) + 64
        cand = (_u64(base, drawn, need) % np.uint64(numel)).astype(np.int64)
        drawn += need
        allc = np.concatenate([got, cand])
        _, first = np.unique(allc, return_index=True)
        got = allc[np.sort(first)]
    return got[:count]


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp64 values once, to nearest even, to bf16 bit patterns (uint16).
    Values must be zero or within the bf16 normal range."""
    a = np.ascontiguousarray(a, np.float64)
    if a.size <= _CHUNK:
        return _bf16_bits_chunk(a)
    flat = a.reshape(-1)
    out = np.empty(flat.size, np.uint16)

    def work(s):
        out[s:s + _CHUNK] = _bf16_bits_chunk(flat[s:s + _CHUNK])

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(work, range(0, flat.size, _CHUNK)))
    return out.reshape(a.shape)


def _bf16_bits_chunk(a: np.ndarray) -> np.ndarray:
    bits = a.view(np.uint64)
    sign = (bits >> np.uint64(63)).astype(np.uint16) << np.uint16(15)
    mag = bits & np.uint64(0x7FFFFFFFFFFFFFFF)
    lsb = (mag >> np.uint64(45)) & np.uint64(1)
    r = (mag + np.uint64((1 << 44) - 1) + lsb) >> np.uint64(45)      # f64 exponent|7-bit mantissa
    exp = (r >> np.uint64(7)).astype(np.int64) - 1023 + 127
    zero = mag == 0
    if np.any(~zero & ((exp < 1) | (exp > 254))):
        raise ValueError("value outside the bf16 normal range")
    body = ((np.where(zero, 0, exp).astype(np.uint64) << np.uint64(7)) | (r & np.uint64(0x7F))).astype(np.uint16)
    return np.where(zero, np.uint16(0), body) | sign


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact fp64 values of bf16 bit patterns."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ recipes

def activation(rows: int, cols: int, seed: int, stream: str, *, per_channel_lognormal: bool,
               outlier_frac: float, outlier_mult: float) -> np.ndarray:
    """bf16 activations [rows, cols] (see the module docstring for the recipe)."""
    x = normal(rows * cols, seed, stream + "/x").reshape(rows, cols)
    if per_channel_lognormal:
        chan = np.exp(normal(cols, seed, stream + "/chan"))[None, :]
        step = max(1, _CHUNK // cols)

        def work(r):
            x[r:r + step] *= chan

        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(work, range(0, rows, step)))
    n_out = int(round(outlier_frac * rows * cols))
    pos = distinct_positions(n_out, rows * cols, seed, stream + "/outliers")
    flat = x.reshape(-1)
    flat[pos] *= outlier_mult
    return bf16_bits(x)


def gaussian(rows: int, cols: int, std: float, seed: int, stream: str) -> np.ndarray:
    """bf16 [rows, cols] ~ N(0, std)."""
    return bf16_bits(normal(rows * cols, seed, stream) .reshape(rows, cols) * std)


def flux_activation(rows: int, cols: int, seed: int = 0, stream: str = "act") -> np.ndarray:
    return activation(rows, cols, seed, stream, per_channel_lognormal=True, outlier_frac=1e-3, outlier_mult=50.0)


def tiny_activation(rows: int = 128, cols: int = 256, seed: int = 0, stream: str = "tiny/A") -> np.ndarray:
    return activation(rows, cols, seed, stream, per_channel_lognormal=False, outlier_frac=1e-2, outlier_mult=20.0)


def long_sequence_activation(rows: int, cols: int, seed: int = 0, stream: str = "long/A") -> np.ndarray:
    return activation(rows, cols, seed, stream, per_channel_lognormal=False, outlier_frac=1e-3, outlier_mult=50.0)


def weight(n: int, k: int, seed: int = 0, stream: str = "W", std: float | None = None) -> np.ndarray:
    return gaussian(n, k, (1.0 / np.sqrt(k)) if std is None else std, seed, stream)


def bias(n: int, k: int, seed: int = 0, stream: str = "bias") -> np.ndarray:
    return gaussian(1, n, 1.0 / np.sqrt(k), seed, stream).reshape(n)


def attention_qkv(heads: int, L: int, d: int = 128, seed: int = 0, stream: str = "attn", gain: float = 1.0):
    """bf16 (Q, K, V), each [heads * L, d]: Q, K ~ N(0, gain), V ~ N(0, 1)."""
    q = gaussian(heads * L, d, gain, seed, stream + "/Q")
    k = gaussian(heads * L, d, gain, seed, stream + "/K")
    v = gaussian(heads * L, d, 1.0, seed, stream + "/V")
    return q, k, v


def to_torch(bits: np.ndarray, device=None):
    """bf16 bit patterns -> torch.bfloat16 tensor (on `device` if given)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device) if device is not None else t
