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
           "mxq_nvfp4_calibrate", "mxq_quantize_fp8_weight", "mxq_gemm_mxfp8", "mxq_gemm_nvfp4_workspace_size",
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
                  "mxq_gemm_mxfp8", "mxq_gemm_nvfp4", "mxq_gemm_bf16_fp8w", "mxq_quantize_fp8_v",
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


def _need(t, dtype, name, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


# ------------------------------------------------------------------ quantizers

def quantize_mxfp8(x, kind="e4m3", out=None, stream=None, scale_layout="row"):
    """bf16 [R, C] -> (codes uint8 [R, C], E8M0 scales uint8 [R, C/32]).  The
    scales' bytes are in row-major order ("row") or in the GEMM-tiled order
    ("tiled", R % 64 == 0 and C % 128 == 0; the tensor keeps the shape [R, C/32])."""
    torch = _torch()
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, C = x.shape
    q, s = out if out is not None else (
        torch.empty((R, C), dtype=torch.uint8, device=x.device),
        torch.empty((R, C // 32), dtype=torch.uint8, device=x.device))
    lib = load()
    _check(lib.mxq_quantize_mxfp8(_ptr(x), R, C, _KIND[kind], _ptr(q), _ptr(s), _LAYOUT[scale_layout],
                                  _stream(stream)))
    return q, s


def nvfp4_workspace_size(rows: int, cols: int) -> int:
    return int(load().mxq_quantize_nvfp4_workspace_size(rows, cols))


def quantize_nvfp4(x, global_scale=None, out=None, workspace=None, stream=None, scale_layout="row"):
    """bf16 [R, C] -> (packed E2M1 uint8 [R, C/2], E4M3 uint8 [R, C/16], fp32 [1]
    decode scale).  global_scale: None (dynamic, from amax(x)) or a 1-element fp32
    CUDA tensor (static).  scale_layout as for quantize_mxfp8."""
    torch = _torch()
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, C = x.shape
    if global_scale is not None:
        _need(global_scale, torch.float32, "global_scale", x.device)
    if out is not None:
        q, s, g = out
    else:
        q = torch.empty((R, C // 2), dtype=torch.uint8, device=x.device)
        s = torch.empty((R, C // 16), dtype=torch.uint8, device=x.device)
        g = torch.empty((1,), dtype=torch.float32, device=x.device)
    ws_bytes = 0
    if global_scale is None:
        ws_bytes = nvfp4_workspace_size(R, C)
        if workspace is None:
            workspace = torch.empty((max(ws_bytes, 4),), dtype=torch.uint8, device=x.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    lib = load()
    _check(lib.mxq_quantize_nvfp4(_ptr(x), R, C, _ptr(global_scale), _ptr(q), _ptr(s), _LAYOUT[scale_layout],
                                  _ptr(g), _ptr(workspace), ws_bytes, _stream(stream)))
    return q, s, g


def quantize_nvfp4_noalloc(x, out, global_scale=None, stream=None, scale_layout="row"):
    """quantize_nvfp4 through the entry point that allocates nothing and takes no
    workspace (its dynamic-mode partial maxima live in the library's static device
    scratch).  out = (q, s, g), allocated by the caller as for quantize_nvfp4."""
    torch = _torch()
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, C = x.shape
    if global_scale is not None:
        _need(global_scale, torch.float32, "global_scale", x.device)
    q, s, g = out
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
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, C = x.shape
    if running is None:
        running = torch.zeros((1,), dtype=torch.float32, device=x.device)
    _need(running, torch.float32, "running", x.device)
    ws_bytes = nvfp4_workspace_size(R, C)
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 4),), dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    lib = load()
    _check(lib.mxq_nvfp4_calibrate(_ptr(x), R, C, _ptr(running), _ptr(workspace), ws_bytes, _stream(stream)))
    return running


def quantize_fp8_weight(w, scale=None, out=None, workspace=None, stream=None):
    """Weight-only FP8: bf16 [R, C] -> (E4M3 codes uint8 [R, C], fp32 [1] decode
    scale).  scale: None (RN_fp32(amax / 448)) or a 1-element fp32 CUDA tensor."""
    torch = _torch()
    _need(w, torch.bfloat16, "w")
    if w.dim() != 2:
        raise ValueError("w must be 2-D")
    R, C = w.shape
    if scale is not None:
        _need(scale, torch.float32, "scale", w.device)
    if out is not None:
        q, s = out
    else:
        q = torch.empty((R, C), dtype=torch.uint8, device=w.device)
        s = torch.empty((1,), dtype=torch.float32, device=w.device)
    ws_bytes = 0
    if scale is None:
        ws_bytes = nvfp4_workspace_size(R, C)
        if workspace is None:
            workspace = torch.empty((max(ws_bytes, 4),), dtype=torch.uint8, device=w.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    lib = load()
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
    for t, n in ((a_q, "a_q"), (a_s, "a_s"), (w_q, "w_q"), (w_s, "w_s")):
        _need(t, torch.uint8, n)
    M, K = a_q.shape
    N = w_q.shape[0]
    if w_q.shape[1] != K or a_s.shape != (M, K // 32) or w_s.shape != (N, K // 32):
        raise ValueError("operand shapes disagree")
    if epi is None:
        epi = "none" if bias is None else "bias"
    e = _epi(epi, bias)
    if bias is not None:
        _need(bias, torch.bfloat16, "bias")
    c = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
    lib = load()
    _check(lib.mxq_gemm_mxfp8(_ptr(a_q), _ptr(a_s), _KIND[a_kind], _ptr(w_q), _ptr(w_s), _KIND[w_kind],
                              _LAYOUT[scale_layout], M, N, K, _ptr(bias), e, _ptr(c), _stream(stream)))
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
    for t, n in ((a_q, "a_q"), (a_s, "a_s"), (w_q, "w_q"), (w_s, "w_s")):
        _need(t, torch.uint8, n)
    _need(a_g, torch.float32, "a_g")
    _need(w_g, torch.float32, "w_g")
    M, KP = a_q.shape
    K = 2 * KP
    N = w_q.shape[0]
    if w_q.shape[1] != KP or a_s.shape != (M, K // 16) or w_s.shape != (N, K // 16):
        raise ValueError("operand shapes disagree")
    if epi is None:
        epi = "none" if bias is None else "bias"
    e = _epi(epi, bias)
    if bias is not None:
        _need(bias, torch.bfloat16, "bias")
    c = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
    lib = load()
    ws, nbytes = None, 0
    if split:
        need = int(lib.mxq_gemm_nvfp4_workspace_size(M, N, K))
        if workspace is not None:
            _need(workspace, torch.uint8, "workspace")
            ws, nbytes = workspace, workspace.numel()
        elif need:
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
    q, s_out = out if out is not None else (torch.empty((heads, d, L), dtype=torch.uint8, device=v.device),
                                            torch.empty((1,), dtype=torch.float32, device=v.device))
    lib = load()
    ws, nbytes = None, 0
    if scale is None:
        nbytes = int(lib.mxq_quantize_nvfp4_workspace_size(heads * L, d))
        ws = workspace if workspace is not None else torch.empty((max(nbytes, 4),), dtype=torch.uint8,
                                                                 device=v.device)
        nbytes = ws.numel()
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
        _need(t, torch.float32, n)
    d = q.shape[-1]
    L = q.numel() // (heads * d)
    if k.numel() != q.numel() or vt.numel() != q.numel():
        raise ValueError("q, k, vt sizes disagree")
    o = out if out is not None else torch.empty((heads * L, d), dtype=torch.bfloat16, device=q.device)
    _check(load().mxq_attention_fp8(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(vt), _ptr(v_scale),
                                    heads, L, d, _ptr(o), _stream(stream)))
    return o


def gemm_bf16_fp8w(a, w_q, w_scale, bias=None, epi=None, out=None, stream=None):
    """Weight-only FP8: C[M, N] = epi(s_w A . val(W)^T) in bf16, A bf16 [M, K], W E4M3 [N, K]."""
    torch = _torch()
    _need(a, torch.bfloat16, "a")
    _need(w_q, torch.uint8, "w_q")
    _need(w_scale, torch.float32, "w_scale")
    M, K = a.shape
    N = w_q.shape[0]
    if w_q.shape[1] != K:
        raise ValueError("operand shapes disagree")
    if epi is None:
        epi = "none" if bias is None else "bias"
    e = _epi(epi, bias)
    if bias is not None:
        _need(bias, torch.bfloat16, "bias")
    c = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    lib = load()
    _check(lib.mxq_gemm_bf16_fp8w(_ptr(a), _ptr(w_q), _ptr(w_scale), M, N, K, _ptr(bias), e, _ptr(c),
                                  _stream(stream)))
    return c
