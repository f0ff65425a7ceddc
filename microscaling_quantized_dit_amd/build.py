"""Build libmxq.so (the gfx950 HIP kernels + C-ABI host layer) in-tree with hipcc,
and libmxq_probes.so (measurement probes for the bench and the tests).

    python -m microscaling_quantized_dit_amd.build

Flags: -O3, gfx950 only, no fast-math (fp32 division stays correctly rounded),
packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmxq.so")
PROBES_LIB = os.path.join(PKG, "libmxq_probes.so")
# the probes library also holds a probe build of the MXFP8 GEMM (MXQ_PROBE_BUILD)
PROBES_SOURCES = ["probes.hip", "gemm_mxfp8.hip"]
SOURCES = ["quant_mxfp8.hip", "quant_nvfp4.hip", "gemm_mxfp8.hip", "gemm_mxfp8_fused.hip", "gemm_nvfp4.hip", "gemm_w8.hip", "gemm_fixup.hip",
           "attention_fp8.hip", "mxq_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def build(verbose: bool = False) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(job):
        src, probe = job
        obj = os.path.join(objdir, os.path.splitext(src)[0] + (".probe.o" if probe else ".o"))
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        defs = ["-DMXQ_PROBE_BUILD"] if probe else []
        cmd = [HIPCC] + FLAGS + defs + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    with ThreadPoolExecutor(len(SOURCES) + len(PROBES_SOURCES)) as ex:
        objs = list(ex.map(compile_one, [(f, False) for f in SOURCES] + [(f, True) for f in PROBES_SOURCES]))
    for lib, lib_objs in ((LIB, objs[:len(SOURCES)]), (PROBES_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + lib_objs
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
