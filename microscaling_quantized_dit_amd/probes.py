"""Measurement probes (libmxq_probes.so): attainable matrix-core rates and shader
clock under load, a streaming HBM copy, and single matrix-core instructions on
given operands.  Used by bench.py and the tests; not part of the quantized-linear
library's interface.  Raises if the probe library is not built."""
from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxq_probes.so")
_lib = None

FLOPS_PER_MFMA = {"fp8": 2 * 32 * 32 * 64, "fp16": 2 * 32 * 32 * 16}
MFMAS_PER_ROUND = 8            # per wave and loop round (4 accumulators x 2)


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libmxq_probes.so is not built (%s); run __graft_entry__.build()" % _LIB_PATH)
        import torch  # noqa: F401  (torch's HIP runtime first, as for libmxq)
        lib = ctypes.CDLL(_LIB_PATH)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.probe_mfma_loop.argtypes = [i32, i32, i32, P, P, P]
        lib.probe_copy.argtypes = [P, P, i64, i32, P]
        lib.probe_mfma_once_fp8.argtypes = [P, P, P, P, P]
        lib.probe_mfma_once_16.argtypes = [P, P, P, P, i32, P]
        lib.probe_gemm_mxfp8_a_twice.argtypes = [P, P, P, P, i64, i64, i64, P, P]
        lib.probe_wall_clock_hz.restype = i64
        lib.probe_exp2.argtypes = [P, P, i32, P]
        for f in ("probe_mfma_loop", "probe_copy", "probe_mfma_once_fp8", "probe_mfma_once_16",
                  "probe_gemm_mxfp8_a_twice", "probe_exp2"):
            getattr(lib, f).restype = i32
        _lib = lib
    return _lib


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc):
    if rc != 0:
        raise RuntimeError("probe launch failed (hipError %d)" % rc)


def mfma_rate(kind: str = "fp8", iters: int = 4000, blocks_per_cu: int = 2, reps: int = 3):
    """Back-to-back MFMAs on register data from every compute unit: (TFLOP/s, shader
    clock in MHz) of the fastest of `reps` launches, timed with HIP events on the
    launch stream; the clock is the mean over workgroups of s_memtime ticks per
    s_memrealtime tick."""
    import torch
    lib = load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = cus * blocks_per_cu
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda")
    k = 0 if kind == "fp8" else 1
    _check(lib.probe_mfma_loop(k, blocks, 50, _ptr(sink), _ptr(clocks), _stream()))   # warm-up
    best = None
    stream = torch.cuda.current_stream()
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        _check(lib.probe_mfma_loop(k, blocks, iters, _ptr(sink), _ptr(clocks), _stream()))
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        c = clocks.view(blocks, 4).cpu().numpy().astype("float64")
        ratio = (c[:, 1] - c[:, 0]) / (c[:, 3] - c[:, 2])
        mhz = float(ratio.mean()) * lib.probe_wall_clock_hz() / 1e6
        flops = blocks * 4 * iters * MFMAS_PER_ROUND * FLOPS_PER_MFMA[kind]
        rate = flops / (ms * 1e-3) / 1e12
        if best is None or rate > best[0]:
            best = (rate, mhz)
    return best


def hbm_copy(n_bytes: int = 1 << 30, reps: int = 5):
    """Streaming device copy of n_bytes: GB/s counting the bytes read and written,
    the fastest of `reps` launches."""
    import torch
    lib = load()
    src = torch.empty(n_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = cus * 4
    _check(lib.probe_copy(_ptr(src), _ptr(dst), n_bytes, blocks, _stream()))
    stream = torch.cuda.current_stream()
    best = 0.0
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        _check(lib.probe_copy(_ptr(src), _ptr(dst), n_bytes, blocks, _stream()))
        b.record(stream)
        torch.cuda.synchronize()
        best = max(best, 2 * n_bytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src, dst
    return best


def mfma_once_fp8(a_codes, b_codes, c=None):
    """D = A B^T + C for one v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3, unit scales):
    a_codes, b_codes uint8 [32, 64] (row k = K position k), c fp32 [32, 32]."""
    import numpy as np
    import torch
    lib = load()
    da = torch.from_numpy(np.ascontiguousarray(a_codes, np.uint8)).cuda()
    db = torch.from_numpy(np.ascontiguousarray(b_codes, np.uint8)).cuda()
    dc = torch.from_numpy(np.zeros((32, 32), np.float32) if c is None else np.ascontiguousarray(c, np.float32)).cuda()
    out = torch.empty((32, 32), dtype=torch.float32, device="cuda")
    _check(lib.probe_mfma_once_fp8(_ptr(da), _ptr(db), _ptr(dc), _ptr(out), _stream()))
    return out.cpu().numpy().astype(np.float64)


def mfma_once_16(a_bits, b_bits, kind: str, c=None):
    """D = A B^T + C for one v_mfma_f32_32x32x16_{f16,bf16}: a_bits, b_bits uint16
    [32, 16] bit patterns."""
    import numpy as np
    import torch
    lib = load()
    da = torch.from_numpy(np.ascontiguousarray(a_bits, np.uint16).view(np.int16)).cuda()
    db = torch.from_numpy(np.ascontiguousarray(b_bits, np.uint16).view(np.int16)).cuda()
    dc = torch.from_numpy(np.zeros((32, 32), np.float32) if c is None else np.ascontiguousarray(c, np.float32)).cuda()
    out = torch.empty((32, 32), dtype=torch.float32, device="cuda")
    _check(lib.probe_mfma_once_16(_ptr(da), _ptr(db), _ptr(dc), _ptr(out), 0 if kind == "fp16" else 1, _stream()))
    return out.cpu().numpy().astype(np.float64)


def gemm_mxfp8_a_twice(a_q, a_s, w_q, w_s, out):
    """The MXFP8 GEMM (E4M3, tiled scales, no epilogue) with every A stage DMA'd
    twice -- a GEMM that reads its activation at bf16 size, without the work of
    quantizing it: the lower bound of fusing the quantizer into the prologue.
    Operands as for gemm_mxfp8 with scale_layout="tiled"; out bf16 [M, N]."""
    import torch
    M, K = a_q.shape
    N = w_q.shape[0]
    for t in (a_q, a_s, w_q, w_s, out):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("operands must be contiguous GPU tensors")
    if M % 128 or N % 128 or K % 128 or tuple(out.shape) != (M, N) or out.dtype != torch.bfloat16:
        raise ValueError("M, N, K multiples of 128 and out bf16 [M, N] required")
    _check(load().probe_gemm_mxfp8_a_twice(_ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), M, N, K, _ptr(out),
                                           _stream()))
    return out


def exp2(x):
    """v_exp_f32 of every element of a contiguous fp32 CUDA tensor (a new tensor)."""
    import torch
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 CUDA tensor")
    y = torch.empty_like(x)
    _check(load().probe_exp2(_ptr(x), _ptr(y), x.numel(), _stream()))
    return y
