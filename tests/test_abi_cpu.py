"""The C-ABI library loads, exports every symbol include/mxq.h declares, and
rejects invalid calls on the host, before any launch or device query.

No compute call is made here: every call below fails validation (fake but
aligned pointers are never dereferenced).  The device gate is exercised only
where no GPU is present.
"""
import ctypes
import os
import re

import pytest

import microscaling_quantized_dit_amd as mxq
from tests.conftest import ROOT, gpu_available

HEADER = os.path.join(ROOT, "include", "mxq.h")
FAKE = 0x10000          # aligned, never dereferenced
FAKE2 = 0x20000
MIS = 0x10008           # 8 mod 16

SUCCESS, INVALID, SHAPE, MISALIGNED, WORKSPACE, DEVICE, LAUNCH = range(7)
ROW, TILED = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mxq.library_path()):
        import microscaling_quantized_dit_amd.build as b
        b.build()
    return mxq.load()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(mxq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for s in ["mxq_quantize_mxfp8", "mxq_quantize_nvfp4", "mxq_quantize_nvfp4_workspace_size",
              "mxq_gemm_mxfp8", "mxq_gemm_nvfp4_workspace_size", "mxq_gemm_nvfp4", "mxq_quantize_fp8_v",
              "mxq_attention_fp8", "mxq_status_string", "mxq_last_error"]:
        assert s in syms


def test_library_exports_every_declared_symbol(lib):
    for s in declared_symbols():
        assert hasattr(lib, s), s
    assert sorted(mxq.SYMBOLS) == declared_symbols()


def test_status_strings(lib):
    for code, word in [(SUCCESS, b"success"), (INVALID, b"invalid"), (SHAPE, b"shape"),
                       (MISALIGNED, b"misaligned"), (WORKSPACE, b"workspace"), (DEVICE, b"device"),
                       (LAUNCH, b"launch")]:
        assert word in lib.mxq_status_string(code)


def _q8(lib, x=FAKE, rows=4, cols=64, kind=0, q=FAKE, s=FAKE2, layout=ROW):
    return lib.mxq_quantize_mxfp8(x, rows, cols, kind, q, s, layout, None)


def test_quantize_mxfp8_validation(lib):
    assert _q8(lib, x=None) == INVALID
    assert _q8(lib, q=None) == INVALID
    assert _q8(lib, rows=0) == INVALID
    assert _q8(lib, cols=-32) == INVALID
    assert _q8(lib, kind=2) == INVALID
    assert _q8(lib, cols=48) == SHAPE
    assert _q8(lib, rows=1 << 62, cols=64) == SHAPE
    assert _q8(lib, x=MIS) == MISALIGNED
    assert _q8(lib, s=MIS) == MISALIGNED
    assert b"multiple of 32" in (_q8(lib, cols=48) and lib.mxq_last_error())
    # the tiled scale order groups rows by 64 and K by 128
    assert _q8(lib, layout=2) == INVALID
    assert _q8(lib, layout=TILED) == SHAPE                      # 4 rows
    assert _q8(lib, rows=64, cols=96, layout=TILED) == SHAPE
    assert _q8(lib, rows=64, cols=128, layout=TILED, s=MIS) == MISALIGNED
    assert _q8(lib, rows=1 << 37, cols=1 << 7, layout=TILED) == SHAPE   # workgroups past 2^31


def test_quantize_nvfp4_validation(lib):
    ws = lib.mxq_quantize_nvfp4_workspace_size
    assert ws(128, 256) >= 4 and ws(128, 24) == 0 and ws(0, 16) == 0
    need = ws(4, 64)

    def call(x=FAKE, rows=4, cols=64, gin=None, q=FAKE, s=FAKE2, gout=FAKE, w=FAKE2, wsb=need, layout=ROW):
        return lib.mxq_quantize_nvfp4(x, rows, cols, gin, q, s, layout, gout, w, wsb, None)

    assert call(x=None) == INVALID
    assert call(gout=None) == INVALID
    assert call(cols=0) == INVALID
    assert call(cols=24) == SHAPE
    assert call(q=MIS) == MISALIGNED
    assert call(gout=FAKE + 2) == MISALIGNED
    assert call(w=None) == WORKSPACE
    assert call(wsb=need - 4) == WORKSPACE
    assert call(layout=-1) == INVALID
    assert call(layout=TILED) == SHAPE
    assert call(rows=128, cols=64, layout=TILED) == SHAPE


def test_quantize_nvfp4_noalloc_validation(lib):
    """The entry point without a workspace validates like mxq_quantize_nvfp4 (minus
    the workspace checks): nothing is looked up or launched for an invalid call."""
    def call(x=FAKE, rows=4, cols=64, gin=None, q=FAKE, s=FAKE2, gout=FAKE, layout=ROW):
        return lib.mxq_quantize_nvfp4_noalloc(x, rows, cols, gin, q, s, layout, gout, None)

    assert call(x=None) == INVALID
    assert call(s=None) == INVALID
    assert call(gout=None) == INVALID
    assert call(rows=0) == INVALID
    assert call(cols=24) == SHAPE
    assert call(rows=1 << 62, cols=64) == SHAPE
    assert call(q=MIS) == MISALIGNED
    assert call(gout=FAKE + 2) == MISALIGNED
    assert call(gin=FAKE + 1) == MISALIGNED
    assert call(layout=3) == INVALID
    assert call(layout=TILED) == SHAPE
    if not gpu_available():
        assert call() == DEVICE              # valid arguments reach the device check
        assert call(gin=FAKE) == DEVICE


def test_nvfp4_calibrate_validation(lib):
    need = lib.mxq_quantize_nvfp4_workspace_size(4, 64)

    def call(x=FAKE, rows=4, cols=64, run=FAKE, w=FAKE2, wsb=need):
        return lib.mxq_nvfp4_calibrate(x, rows, cols, run, w, wsb, None)

    assert call(x=None) == INVALID
    assert call(run=None) == INVALID
    assert call(rows=-1) == INVALID
    assert call(cols=40) == SHAPE
    assert call(x=MIS) == MISALIGNED
    assert call(run=FAKE + 2) == MISALIGNED
    assert call(w=None) == WORKSPACE
    assert call(wsb=need - 4) == WORKSPACE


def test_fp8_weight_validation(lib):
    need = lib.mxq_quantize_nvfp4_workspace_size(4, 64)

    def quant(w=FAKE, rows=4, cols=64, sin=None, q=FAKE2, sout=FAKE, ws=FAKE2, wsb=need):
        return lib.mxq_quantize_fp8_weight(w, rows, cols, sin, q, sout, ws, wsb, None)

    assert quant(w=None) == INVALID
    assert quant(sout=None) == INVALID
    assert quant(cols=24) == SHAPE
    assert quant(q=MIS) == MISALIGNED
    assert quant(sout=FAKE + 2) == MISALIGNED
    assert quant(ws=None) == WORKSPACE
    assert quant(sin=FAKE, ws=None) == DEVICE          # static mode needs no workspace; no GPU here

    def gemm(a=FAKE, w=FAKE2, s=FAKE, M=128, N=256, K=256, bias=None, epi=0, c=FAKE):
        return lib.mxq_gemm_bf16_fp8w(a, w, s, M, N, K, bias, epi, c, None)

    assert gemm(s=None) == INVALID
    assert gemm(K=192) == SHAPE
    assert gemm(epi=1) == INVALID
    assert gemm(a=MIS) == MISALIGNED
    assert gemm(s=FAKE + 2) == MISALIGNED
    assert gemm(M=1 << 20, K=1024) == SHAPE              # A > 2 GiB at 2 bytes per element
    assert gemm() == DEVICE


def _g8(lib, M=128, N=256, K=256, bias=None, epi=0, c=FAKE, a=FAKE, ak=0, wk=0, layout=ROW):
    return lib.mxq_gemm_mxfp8(a, FAKE2, ak, FAKE, FAKE2, wk, layout, M, N, K, bias, epi, c, None)


def test_gemm_mxfp8_validation(lib):
    assert _g8(lib, a=None) == INVALID
    assert _g8(lib, c=None) == INVALID
    assert _g8(lib, M=0) == INVALID
    assert _g8(lib, epi=3) == INVALID
    assert _g8(lib, epi=1) == INVALID            # bias required
    assert _g8(lib, ak=5) == INVALID
    assert _g8(lib, K=192) == SHAPE               # 128 alignment rule
    assert _g8(lib, M=200) == SHAPE
    assert _g8(lib, M=1 << 20, K=1 << 12) == SHAPE  # A would exceed 2 GiB
    assert _g8(lib, c=MIS) == MISALIGNED
    assert _g8(lib, epi=2, bias=MIS) == MISALIGNED
    assert _g8(lib, layout=7) == INVALID
    assert _g8(lib, layout=TILED, K=192) == SHAPE


def test_gemm_mxfp8_fused_validation(lib):
    def call(a=FAKE, kind=0, w=FAKE2, ws=FAKE, layout=ROW, M=128, N=256, K=256, bias=None, epi=0, c=FAKE):
        return lib.mxq_gemm_mxfp8_fused(a, kind, w, ws, layout, M, N, K, bias, epi, c, None)

    assert call(a=None) == INVALID
    assert call(ws=None) == INVALID
    assert call(kind=2) == INVALID
    assert call(layout=3) == INVALID
    assert call(epi=1) == INVALID                    # bias required
    assert call(K=192) == SHAPE
    assert call(M=1 << 20, K=1024) == SHAPE          # A > 2 GiB at 2 bytes per element
    assert call(a=MIS) == MISALIGNED
    assert call(ws=MIS) == MISALIGNED
    assert call() == DEVICE                          # valid arguments, no GPU here


def test_gemm_nvfp4_validation(lib):
    def call(M=128, N=256, K=256, ag=FAKE, bias=None, epi=0, c=FAKE, ws=None, nbytes=0, layout=ROW):
        return lib.mxq_gemm_nvfp4(FAKE, FAKE2, ag, FAKE, FAKE2, FAKE, layout, M, N, K, bias, epi, c, ws, nbytes,
                                  None)

    assert call(ag=None) == INVALID
    assert call(N=100) == SHAPE
    assert call(epi=2) == INVALID
    assert call(ag=FAKE + 1) == MISALIGNED
    assert call(layout=2) == INVALID
    # a shape with a partial last round (17 x 16 tiles on 256 compute units, the
    # count assumed without a device) wants a workspace; too small a one is refused
    def scales(M, N, K):                                 # both operands' scales, re-laid out
        return M * K // 16 + N * K // 16

    need = lib.mxq_gemm_nvfp4_workspace_size(4352, 4096, 1024)
    assert need == 16 * 4 * 256 * 256 * 4 + scales(4352, 4096, 1024)   # 16 leftover tiles, 4 K-parts, fp32
    assert call(M=4352, N=4096, K=1024, ws=FAKE, nbytes=need - 1) == WORKSPACE
    assert call(M=4352, N=4096, K=1024, ws=FAKE + 8, nbytes=need) == MISALIGNED
    assert lib.mxq_gemm_nvfp4_workspace_size(4096, 4096, 1024) == scales(4096, 4096, 1024)   # one full round
    assert lib.mxq_gemm_nvfp4_workspace_size(4352, 4096, 1152) == scales(4352, 4096, 1152)   # odd stages: no split
    assert lib.mxq_gemm_nvfp4_workspace_size(128, 384, 128) == 128 * 8 + 384 * 8
    assert lib.mxq_gemm_nvfp4_workspace_size(100, 4096, 1024) == 0


def test_attention_validation(lib):
    def att(q=FAKE, qs=FAKE, heads=2, L=256, d=128, o=FAKE):
        return lib.mxq_attention_fp8(q, qs, FAKE, FAKE, FAKE, FAKE, heads, L, d, o, None)

    def vq(v=FAKE, heads=2, L=256, d=128, scale=None, ws=FAKE, nbytes=1 << 20):
        return lib.mxq_quantize_fp8_v(v, heads, L, d, scale, FAKE, FAKE, ws, nbytes, None)

    assert att(q=None) == INVALID
    assert att(heads=0) == INVALID
    assert att(d=64) == SHAPE
    assert att(L=192) == SHAPE                     # multiple of 128
    assert att(L=1 << 24) == SHAPE                 # L * 128 must stay below 2^31
    assert att(o=FAKE + 2) == MISALIGNED
    assert att(qs=FAKE + 2) == MISALIGNED
    assert vq(v=None) == INVALID
    assert vq(d=256) == SHAPE
    assert vq(ws=None) == WORKSPACE                # dynamic scale needs the partials
    assert vq(nbytes=4) == WORKSPACE
    assert vq(v=FAKE + 8) == MISALIGNED


@pytest.mark.skipif(gpu_available(), reason="device gate is only observable without a GPU")
def test_device_gate_without_gpu(lib):
    """Valid arguments reach the device check, which refuses without a gfx950."""
    assert _q8(lib) == DEVICE
    assert _q8(lib, rows=64, cols=128, layout=TILED) == DEVICE
    assert _g8(lib) == DEVICE
    assert _g8(lib, layout=TILED) == DEVICE


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """The binding never falls back to anything when libmxq.so is absent."""
    import importlib
    m = importlib.reload(mxq)
    monkeypatch.setattr(m, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(m, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        m.load()
    importlib.reload(mxq)
