"""Python binding of libmxq, the gfx950 microscaling-quantized linear layer.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in include/mxq.h.  PyTorch supplies device memory and the current
stream.  If libmxq.so is missing or cannot be loaded, every call raises -- there
is no CPU fallback.

    q, s = quantize_mxfp8(x)                         # x: bf16 [R, C] on cuda
    q, s, g = quantize_nvfp4(x)                      # dynamic per-tensor scale
    c = gemm_mxfp8(aq, as_, wq, ws, bias=b, epi="bias_gelu")
    c = gemm_nvfp4(aq, as_, ag, wq, ws, wg)
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

__all__ = [
    "load", "MXQError", "E4M3", "E5M2", "EPI_NONE", "EPI_BIAS", "EPI_BIAS_GELU_TANH",
    "quantize_mxfp8", "quantize_nvfp4", "quantize_nvfp4_noalloc", "nvfp4_workspace_size", "nvfp4_calibrate", "quantize_fp8_weight",
    "gemm_mxfp8", "gemm_nvfp4", "gemm_bf16_fp8w",
    "library_path",
]

E4M3, E5M2 = 0, 1
EPI_NONE, EPI_BIAS, EPI_BIAS_GELU_TANH = 0, 1, 2
_EPI = {"none": 0, "bias": 1, "bias_gelu": 2, "bias_gelu_tanh": 2, 0: 0, 1: 1, 2: 2, None: 0}
_KIND = {"e4m3": 0, "e5m2": 1, 0: 0, 1: 1}
_LAYOUT = {"row": 0, "tiled": 1, 0: 0, 1: 1}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmxq.so")
_lock = threading.Lock()
_lib = None

SYMBOLS = ["mxq_quantize_mxfp8", "mxq_quantize_nvfp4_workspace_size", "mxq_quantize_nvfp4",
           "mxq_quantize_nvfp4_noalloc",
           "mxq_nvfp4_calibrate", "mxq_quantize_fp8_weight", "mxq_gemm_mxfp8", "mxq_gemm_mxfp8_fused",
           "mxq_gemm_nvfp4_workspace_size",
           "mxq_gemm_nvfp4", "mxq_quantize_fp8_v", "mxq_attention_fp8",
           "mxq_gemm_bf16_fp8w", "mxq_status_string", "mxq_last_error"]


class MXQError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("mxq status %d: %s" % (status, detail))
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libmxq.so (built by __graft_entry__.build()); raises if it is absent."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libmxq.so is not built (%s); run __graft_entry__.build()" % _LIB_PATH)
        # torch first: its HIP runtime (soname libamdhip64.so.7) is then the one
        # libmxq binds to, so both share one device context and one stream space.
        import torch  # noqa: F401
        lib = ctypes.CDLL(_LIB_PATH)
        P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        lib.mxq_quantize_mxfp8.argtypes = [P, i64, i64, i32, P, P, i32, P]
        lib.mxq_quantize_nvfp4_workspace_size.argtypes = [i64, i64]
        lib.mxq_quantize_nvfp4_workspace_size.restype = sz
        lib.mxq_quantize_nvfp4.argtypes = [P, i64, i64, P, P, P, i32, P, P, sz, P]
        lib.mxq_quantize_nvfp4_noalloc.argtypes = [P, i64, i64, P, P, P, i32, P, P]
        lib.mxq_nvfp4_calibrate.argtypes = [P, i64, i64, P, P, sz, P]
        lib.mxq_quantize_fp8_weight.argtypes = [P, i64, i64, P, P, P, P, sz, P]
        lib.mxq_gemm_bf16_fp8w.argtypes = [P, P, P, i64, i64, i64, P, i32, P, P]
        lib.mxq_gemm_mxfp8.argtypes = [P, P, i32, P, P, i32, i32, i64, i64, i64, P, i32, P, P]
        lib.mxq_gemm_mxfp8_fused.argtypes = [P, i32, P, P, i32, i64, i64, i64, P, i32, P, P]
        lib.mxq_gemm_nvfp4_workspace_size.argtypes = [i64, i64, i64]
        lib.mxq_gemm_nvfp4_workspace_size.restype = sz
        lib.mxq_gemm_nvfp4.argtypes = [P, P, P, P, P, P, i32, i64, i64, i64, P, i32, P, P, sz, P]
        lib.mxq_quantize_fp8_v.argtypes = [P, i64, i64, i64, P, P, P, P, sz, P]
        lib.mxq_attention_fp8.argtypes = [P, P, P, P, P, P, i64, i64, i64, P, P]
        lib.mxq_status_string.argtypes = [i32]
        lib.mxq_status_string.restype = ctypes.c_char_p
        lib.mxq_last_error.argtypes = []
        lib.mxq_last_error.restype = ctypes.c_char_p
        for f in ("mxq_quantize_mxfp8", "mxq_quantize_nvfp4", "mxq_quantize_nvfp4_noalloc", "mxq_nvfp4_calibrate", "mxq_quantize_fp8_weight",
                  "mxq_gemm_mxfp8", "mxq_gemm_mxfp8_fused", "mxq_gemm_nvfp4", "mxq_gemm_bf16_fp8w",
                  "mxq_quantize_fp8_v",
                  "mxq_attention_fp8"):
            getattr(lib, f).restype = i32
        _lib = lib
        return lib


def _check(status: int):
    if status != 0:
        lib = load()
        raise MXQError(status, "%s (%s)" % (lib.mxq_status_string(status).decode(),
                                            lib.mxq_last_error().decode()))


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context for a call's allocations and launch: the given stream, so that every
    tensor the binding allocates (outputs and temporaries) belongs to the stream
    its kernels run on and the caching allocator cannot hand its memory to another
    stream while they run; the current stream when none is given."""
    torch = _torch()
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _need(t, dtype, name, device=None, shape=None):
    """Check a tensor argument on the host, before any launch: type, dtype, shape
    (when given), then GPU residency, contiguity and device."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _outputs(out, specs, device):
    """Given outputs (checked against specs = [(name, dtype, shape)]) or new ones."""
    torch = _torch()
    if out is None:
        return tuple(torch.empty(shape, dtype=dtype, device=device) for _, dtype, shape in specs)
    out = tuple(out) if isinstance(out, (tuple, list)) else (out,)
    if len(out) != len(specs):
        raise ValueError("out must hold %d tensors" % len(specs))
    for t, (name, dtype, shape) in zip(out, specs):
        _need(t, dtype, name, device, shape)
    return out


def _bias(bias, N, device):
    if bias is not None:
        torch = _torch()
        _need(bias, torch.bfloat16, "bias", device)
        if bias.numel() != N:
            raise ValueError("bias has %d elements, expected N = %d" % (bias.numel(), N))


def _workspace(workspace, device):
    if workspace is not None:
        torch = _torch()
        _need(workspace, torch.uint8, "workspace", device)
        return workspace.numel()
    return 0


def _x2d(x, name="x"):
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if x.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    _need(x, torch.bfloat16, name)
    return x.shape


# ------------------------------------------------------------------ quantizers

def quantize_mxfp8(x, kind="e4m3", out=None, stream=None, scale_layout="row"):
    """bf16 [R, C] -> (codes uint8 [R, C], E8M0 scales uint8 [R, C/32]).  The
    scales' bytes are in row-major order ("row") or in the GEMM-tiled order
    ("tiled", R % 64 == 0 and C % 128 == 0; the tensor keeps the shape [R, C/32])."""
    torch = _torch()
    R, C = _x2d(x)
    lib = load()
    with _on(stream):
        q, s = _outputs(out, [("q", torch.uint8, (R, C)), ("scales", torch.uint8, (R, C // 32))], x.device)
        _check(lib.mxq_quantize_mxfp8(_ptr(x), R, C, _KIND[kind], _ptr(q), _ptr(s), _LAYOUT[scale_layout],
                                      _stream(stream)))
    return q, s


def nvfp4_workspace_size(rows: int, cols: int) -> int:
    return int(load().mxq_quantize_nvfp4_workspace_size(rows, cols))


def _nvfp4_out_specs(R, C):
    torch = _torch()
    return [("q", torch.uint8, (R, C // 2)), ("scales", torch.uint8, (R, C // 16)),
            ("global_scale_out", torch.float32, (1,))]


def quantize_nvfp4(x, global_scale=None, out=None, workspace=None, stream=None, scale_layout="row"):
    """bf16 [R, C] -> (packed E2M1 uint8 [R, C/2], E4M3 uint8 [R, C/16], fp32 [1]
    decode scale).  global_scale: None (dynamic, from amax(x)) or a 1-element fp32
    CUDA tensor (static).  scale_layout as for quantize_mxfp8."""
    torch = _torch()
    R, C = _x2d(x)
    if global_scale is not None:
        _need(global_scale, torch.float32, "global_scale", x.device, (1,))
    ws_bytes = _workspace(workspace, x.device)
    lib = load()
    with _on(stream):
        q, s, g = _outputs(out, _nvfp4_out_specs(R, C), x.device)
        if global_scale is None and workspace is None:
            ws_bytes = max(nvfp4_workspace_size(R, C), 4)
            workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=x.device)
        _check(lib.mxq_quantize_nvfp4(_ptr(x), R, C, _ptr(global_scale), _ptr(q), _ptr(s), _LAYOUT[scale_layout],
                                      _ptr(g), _ptr(workspace), ws_bytes, _stream(stream)))
    return q, s, g


def quantize_nvfp4_noalloc(x, out, global_scale=None, stream=None, scale_layout="row"):
    """quantize_nvfp4 through the entry point that allocates nothing and takes no
    workspace (its dynamic-mode partial maxima live in the library's static device
    scratch).  out = (q, s, g), allocated by the caller as for quantize_nvfp4."""
    torch = _torch()
    R, C = _x2d(x)
    if global_scale is not None:
        _need(global_scale, torch.float32, "global_scale", x.device, (1,))
    if out is None:
        raise ValueError("quantize_nvfp4_noalloc takes its outputs from the caller")
    q, s, g = _outputs(out, _nvfp4_out_specs(R, C), x.device)
    lib = load()
    _check(lib.mxq_quantize_nvfp4_noalloc(_ptr(x), R, C, _ptr(global_scale), _ptr(q), _ptr(s),
                                          _LAYOUT[scale_layout], _ptr(g), _stream(stream)))
    return q, s, g


def nvfp4_calibrate(x, running=None, workspace=None, stream=None):
    """Fold one calibration tensor into a static NVFP4 decode scale:
    running = max(running, RN_fp32(amax(x) / 2688)).  running: a 1-element fp32
    CUDA tensor (zero-initialised here when None); returned for chaining and for
    quantize_nvfp4(x, global_scale=running)."""
    torch = _torch()
    R, C = _x2d(x)
    if running is not None:
        _need(running, torch.float32, "running", x.device, (1,))
    ws_bytes = _workspace(workspace, x.device)
    lib = load()
    with _on(stream):
        if running is None:
            running = torch.zeros((1,), dtype=torch.float32, device=x.device)
        if workspace is None:
            ws_bytes = max(nvfp4_workspace_size(R, C), 4)
            workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=x.device)
        _check(lib.mxq_nvfp4_calibrate(_ptr(x), R, C, _ptr(running), _ptr(workspace), ws_bytes, _stream(stream)))
    return running


def quantize_fp8_weight(w, scale=None, out=None, workspace=None, stream=None):
    """Weight-only FP8: bf16 [R, C] -> (E4M3 codes uint8 [R, C], fp32 [1] decode
    scale).  scale: None (RN_fp32(amax / 448)) or a 1-element fp32 CUDA tensor."""
    torch = _torch()
    R, C = _x2d(w, "w")
    if scale is not None:
        _need(scale, torch.float32, "scale", w.device, (1,))
    ws_bytes = _workspace(workspace, w.device)
    lib = load()
    with _on(stream):
        q, s = _outputs(out, [("q", torch.uint8, (R, C)), ("scale_out", torch.float32, (1,))], w.device)
        if scale is None and workspace is None:
            ws_bytes = max(nvfp4_workspace_size(R, C), 4)
            workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=w.device)
        _check(lib.mxq_quantize_fp8_weight(_ptr(w), R, C, _ptr(scale), _ptr(q), _ptr(s), _ptr(workspace), ws_bytes,
                                           _stream(stream)))
    return q, s


# ------------------------------------------------------------------------ GEMMs

def _epi(epi, bias):
    e = _EPI[epi]
    if e != 0 and bias is None:
        raise ValueError("epilogue %r needs a bias" % (epi,))
    return e


def gemm_mxfp8(a_q, a_s, w_q, w_s, bias=None, epi=None, a_kind="e4m3", w_kind="e4m3", out=None, stream=None,
               scale_layout="row"):
    """C[M, N] = epi(A . W^T) in bf16 from MXFP8 operands (A [M, K], W [N, K]);
    scale_layout names the order of both scale tensors."""
    torch = _torch()
    for t, n in ((a_q, "a_q"), (w_q, "w_q")):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError("%s must be a 2-D tensor" % n)
    M, K = a_q.shape
    N = w_q.shape[0]
    _need(a_q, torch.uint8, "a_q")
    _need(w_q, torch.uint8, "w_q", a_q.device, (N, K))
    _need(a_s, torch.uint8, "a_s", a_q.device, (M, K // 32))
    _need(w_s, torch.uint8, "w_s", a_q.device, (N, K // 32))
    if epi is None:
        epi = "none" if bias is None else "bias"
    e = _epi(epi, bias)
    _bias(bias, N, a_q.device)
    lib = load()
    with _on(stream):
        (c,) = _outputs(out, [("out", torch.bfloat16, (M, N))], a_q.device)
        _check(lib.mxq_gemm_mxfp8(_ptr(a_q), _ptr(a_s), _KIND[a_kind], _ptr(w_q), _ptr(w_s), _KIND[w_kind],
                                  _LAYOUT[scale_layout], M, N, K, _ptr(bias), e, _ptr(c), _stream(stream)))
    return c


def gemm_mxfp8_fused(a, w_q, w_s, kind="e4m3", bias=None, epi=None, out=None, stream=None, scale_layout="row"):
    """C[M, N] = epi(Q(A) . W^T) in bf16: A bf16 [M, K] quantized to MXFP8 (format
    kind) inside the GEMM, W MXFP8 [N, K] of the same format; bit-identical to
    quantize_mxfp8 followed by gemm_mxfp8.  scale_layout names W's scale order."""
    torch = _torch()
    M, K = _x2d(a, "a")
    if not isinstance(w_q, torch.Tensor) or w_q.dim() != 2:
        raise ValueError("w_q must be a 2-D tensor")
    N = w_q.shape[0]
    _need(w_q, torch.uint8, "w_q", a.device, (N, K))
    _need(w_s, torch.uint8, "w_s", a.device, (N, K // 32))
    if epi is None:
        epi = "none" if bias is None else "bias"
    e = _epi(epi, bias)
    _bias(bias, N, a.device)
    lib = load()
    with _on(stream):
        (c,) = _outputs(out, [("out", torch.bfloat16, (M, N))], a.device)
        _check(lib.mxq_gemm_mxfp8_fused(_ptr(a), _KIND[kind], _ptr(w_q), _ptr(w_s), _LAYOUT[scale_layout], M, N, K,
                                        _ptr(bias), e, _ptr(c), _stream(stream)))
    return c


def gemm_nvfp4_workspace_size(M: int, N: int, K: int) -> int:
    """Bytes of workspace gemm_nvfp4 can use for this shape on the current device."""
    return int(load().mxq_gemm_nvfp4_workspace_size(M, N, K))


def gemm_nvfp4(a_q, a_s, a_g, w_q, w_s, w_g, bias=None, epi=None, out=None, workspace=None, split=True,
               stream=None, scale_layout="row"):
    """C[M, N] = epi(s_ga s_gw A . W^T) in bf16 from NVFP4 operands.  With split
    (default), a workspace (given, or allocated here) lets the tiles of a partial
    last round be split along K.  scale_layout names the order of both scale
    tensors."""
    torch = _torch()
    for t, n in ((a_q, "a_q"), (w_q, "w_q")):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError("%s must be a 2-D tensor" % n)
    M, KP = a_q.shape
    K = 2 * KP
    N = w_q.shape[0]
    _need(a_q, torch.uint8, "a_q")
    _need(w_q, torch.uint8, "w_q", a_q.device, (N, KP))
    _need(a_s, torch.uint8, "a_s", a_q.device, (M, K // 16))
    _need(w_s, torch.uint8, "w_s", a_q.device, (N, K // 16))
    _need(a_g, torch.float32, "a_g", a_q.device, (1,))
    _need(w_g, torch.float32, "w_g", a_q.device, (1,))
    if epi is None:
        epi = "none" if bias is None else "bias"
    e = _epi(epi, bias)
    _bias(bias, N, a_q.device)
    nbytes = _workspace(workspace, a_q.device) if split else 0
    ws = workspace if split else None
    lib = load()
    with _on(stream):
        (c,) = _outputs(out, [("out", torch.bfloat16, (M, N))], a_q.device)
        if split and workspace is None:
            need = int(lib.mxq_gemm_nvfp4_workspace_size(M, N, K))
            if need:
                ws = torch.empty((need,), dtype=torch.uint8, device=a_q.device)
                nbytes = need
        _check(lib.mxq_gemm_nvfp4(_ptr(a_q), _ptr(a_s), _ptr(a_g), _ptr(w_q), _ptr(w_s), _ptr(w_g),
                                  _LAYOUT[scale_layout], M, N, K, _ptr(bias), e, _ptr(c), _ptr(ws), nbytes,
                                  _stream(stream)))
    return c


def quantize_fp8_v(v, heads: int, scale=None, out=None, workspace=None, stream=None):
    """V of the FP8 attention: bf16 [heads * L, d] (or [heads, L, d]) -> (codes u8
    [heads, d, L] in the attention's V layout, fp32 per-tensor scale [1])."""
    torch = _torch()
    _need(v, torch.bfloat16, "v")
    d = v.shape[-1]
    L = v.numel() // (heads * d)
    if scale is not None:
        _need(scale, torch.float32, "scale", v.device, (1,))
    nbytes = _workspace(workspace, v.device)
    lib = load()
    with _on(stream):
        q, s_out = _outputs(out, [("vt", torch.uint8, (heads, d, L)), ("scale_out", torch.float32, (1,))], v.device)
        ws = workspace
        if scale is None and workspace is None:
            nbytes = max(int(lib.mxq_quantize_nvfp4_workspace_size(heads * L, d)), 4)
            ws = torch.empty((nbytes,), dtype=torch.uint8, device=v.device)
        _check(lib.mxq_quantize_fp8_v(_ptr(v), heads, L, d, _ptr(scale), _ptr(q), _ptr(s_out), _ptr(ws), nbytes,
                                      _stream(stream)))
    return q, s_out


def attention_fp8(q, q_scale, k, k_scale, vt, v_scale, heads: int, out=None, stream=None):
    """FP8 multi-head attention: E4M3 codes q, k [heads * L, d], V in the layout of
    quantize_fp8_v, fp32 scales [1] -> bf16 [heads * L, d]."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (vt, "vt")):
        _need(t, torch.uint8, n)
    for t, n in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        _need(t, torch.float32, n, q.device, (1,))
    d = q.shape[-1]
    L = q.numel() // (heads * d)
    if k.numel() != q.numel() or vt.numel() != q.numel():
        raise ValueError("q, k, vt sizes disagree")
    lib = load()
    with _on(stream):
        (o,) = _outputs(out, [("out", torch.bfloat16, (heads * L, d))], q.device)
        _check(lib.mxq_attention_fp8(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(vt), _ptr(v_scale),
                                     heads, L, d, _ptr(o), _stream(stream)))
    return o


def gemm_bf16_fp8w(a, w_q, w_scale, bias=None, epi=None, out=None, stream=None):
    """Weight-only FP8: C[M, N] = epi(s_w A . val(W)^T) in bf16, A bf16 [M, K], W E4M3 [N, K]."""
    torch = _torch()
    M, K = _x2d(a, "a")
    if not isinstance(w_q, torch.Tensor) or w_q.dim() != 2:
        raise ValueError("w_q must be a 2-D tensor")
    N = w_q.shape[0]
    _need(w_q, torch.uint8, "w_q", a.device, (N, K))
    _need(w_scale, torch.float32, "w_scale", a.device, (1,))
    if epi is None:
        epi = "none" if bias is None else "bias"
    e = _epi(epi, bias)
    _bias(bias, N, a.device)
    lib = load()
    with _on(stream):
        (c,) = _outputs(out, [("out", torch.bfloat16, (M, N))], a.device)
        _check(lib.mxq_gemm_bf16_fp8w(_ptr(a), _ptr(w_q), _ptr(w_scale), M, N, K, _ptr(bias), e, _ptr(c),
                                      _stream(stream)))
    return c
