#!/usr/bin/env python3
"""Throughput of the microscaling-quantized DiT linear hot path on one MI355X.

One step = the linears of one FLUX DiT double-stream block and one single-stream
block, each preceded by the dynamic quantization of its bf16 activation:

  MXFP8 E4M3, M = 4608 tokens (1024x1024 image + 512 text tokens):
    quantize [4608,3072]  -> QKV      3072 -> 9216
    quantize [4608,3072]  -> out-proj 3072 -> 3072
    quantize [4608,3072]  -> MLP-up   3072 -> 12288  (+bias, GELU-tanh)
    quantize [4608,12288] -> MLP-down 12288 -> 3072
  NVFP4 (dynamic per-tensor activation scale), batch 4, M = 18432:
    quantize [18432,3072]  -> linear1 3072 -> 21504
    quantize [18432,15360] -> linear2 15360 -> 3072

Weights are quantized once before timing (static, as in offline weight
quantization); inputs are seeded synthetic tensors resident in HBM before the
timed region.  value = GEMM flops of the step / step time (TFLOP/s).  Per-op
times come from HIP events on the launch stream around every launch.  The CPU
oracle is timed on a bounded sample of the same work (cpu_baseline).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-scaled GEMM TFLOP/s at FLUX shapes (% MFMA peak); quantizer GB/s (% HBM)"
# MI355X published peaks (dense): HBM3E 8 TB/s; MFMA fp8 5.0 PF, fp4 10.1 PF, fp16/bf16 2.5 PF
PEAK_HBM_GBPS = 8000.0
PEAK_TFLOPS = {"fp8": 5000.0, "fp4": 10100.0, "fp16": 2500.0, "bf16": 2500.0}
PEAK_BF16_TFLOPS = PEAK_TFLOPS["bf16"]

MX_LINEARS = [  # name, N, K, epilogue   (M = 4608)
    ("qkv", 9216, 3072, "none"),
    ("out_proj", 3072, 3072, "none"),
    ("mlp_up", 12288, 3072, "bias_gelu"),
    ("mlp_down", 3072, 12288, "none"),
]
NV_LINEARS = [  # name, N, K, epilogue   (M = 18432)
    ("linear1", 21504, 3072, "none"),
    ("linear2", 3072, 15360, "none"),
]
M_MX, M_NV = 4608, 18432
# block scales travel in the GEMM-tiled order: the quantizers write it, the GEMMs
# fetch a K step's scales for 64 rows as one contiguous load
SCALES = "tiled"
TILED_NAME = "true" if SCALES == "tiled" else "false"   # template argument in kernel names


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter runs
    (profiles/hbm_traffic.json: FETCH_SIZE and WRITE_SIZE per dispatch, scaled by a
    1 GiB copy), or None when there is no record or the kernel's sources have
    changed since the counters were taken."""
    try:
        with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        try:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        except OSError:
            return None
    if h.hexdigest() != rec["sha256"]:
        return None
    return rec


KERNEL_SOURCES = {  # HIP kernel -> sources whose text decides its code
    "k_quant_mxfp8": ["quant_mxfp8.hip"],
    "k_amax_partials": ["quant_nvfp4.hip"],
    "k_quant_nvfp4": ["quant_nvfp4.hip"],
    "k_gemm_mxfp8": ["gemm_mxfp8.hip"],
    "k_gemm_nvfp4": ["gemm_nvfp4.hip", "gemm_fixup.hip"],
}
# dispatches a GEMM op may add after its main kernel (split tiles of a partial
# last round, then their fixup); counted with the op
SPLIT_KERNELS = ("k_gemm_nvfp4<0, true,", "k_gemm_fixup<")


def step_dispatches():
    """(op name, kernel function) of every dispatch of one step, in launch order."""
    out = []
    for name, _, _, epi in MX_LINEARS:
        out.append(("quant_mxfp8_" + name, "k_quant_mxfp8<0, %s>" % TILED_NAME))
        out.append(("gemm_mxfp8_" + name, "k_gemm_mxfp8<0, 0, %d, %s>" % ({"none": 0, "bias": 1, "bias_gelu": 2}[epi],
                                                                           TILED_NAME)))
    for name, _, _, epi in NV_LINEARS:
        out.append(("quant_nvfp4_" + name, "k_amax_partials"))
        out.append(("quant_nvfp4_" + name, "k_quant_nvfp4<%s>" % TILED_NAME))
        out.append(("gemm_nvfp4_" + name, "k_gemm_nvfp4<%d, false, true>" % {"none": 0, "bias": 1, "bias_gelu": 2}[epi]))
    return out


def record_traffic(fetch_db, write_db):
    """profiles/hbm_traffic.json from the two counter runs
        rocprofv3 --pmc FETCH_SIZE --kernel-trace ... -- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --copy-calibration
        rocprofv3 --pmc WRITE_SIZE --kernel-trace ... (same)
    The step's dispatches are the ones right after the 1 GiB calibration copy (a
    GEMM's split and fixup dispatches, when there are any, counted with it); each
    counter is scaled by what it reads for that copy (1 GiB read, 1 GiB written)."""
    import sqlite3

    def per_dispatch(db):
        cur = sqlite3.connect(db).cursor()
        rows = cur.execute("select k.dispatch_id, k.name, sum(p.counter_value) from pmc_events p join kernels k "
                           "on k.dispatch_id = p.dispatch_id group by k.dispatch_id order by k.dispatch_id")
        out = []
        for did, name, kib in rows:
            short = name.replace("mxq::(anonymous namespace)::", "").replace("void ", "").split("(")[0].strip()
            out.append((did, short, float(kib)))
        return out

    fetch, write = per_dispatch(fetch_db), per_dispatch(write_db)
    scale, step = {}, {}
    for counter, rows in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
        copies = [i for i, (_, n, _) in enumerate(rows) if "copyBuffer" in n]
        if not copies:
            raise SystemExit("no calibration copy in %s" % counter)
        i = max(copies, key=lambda j: rows[j][2])
        scale[counter] = round((1 << 20) / rows[i][2], 3)       # KiB of a 1 GiB transfer / counted KiB
        expect = step_dispatches()
        vals, j = [], i + 1
        for _, kernel in expect:
            if j >= len(rows) or rows[j][1] != kernel:
                raise SystemExit("%s: expected %s at dispatch %d, found %s" % (
                    counter, kernel, j, rows[j][1] if j < len(rows) else None))
            kib = rows[j][2]
            j += 1
            while j < len(rows) and rows[j][1].startswith(SPLIT_KERNELS):
                kib += rows[j][2]
                j += 1
            vals.append(kib)
        step[counter] = vals
    rec = {}
    for idx, (op, kernel) in enumerate(step_dispatches()):
        base = kernel.split("<")[0]
        r = rec.setdefault(kernel, {
            "sources": ["microscaling_quantized_dit_amd/csrc/" + f for f in KERNEL_SOURCES[base]] +
                       ["microscaling_quantized_dit_amd/csrc/mxq_internal.h"],
            "launches": {}, "scale": scale, "summary": "profiles/flux_dit_step_hbm_counters.md"})
        r["launches"][op] = {"FETCH_SIZE_KiB": step["FETCH_SIZE"][idx], "WRITE_SIZE_KiB": step["WRITE_SIZE"][idx]}
    for kernel, r in rec.items():
        n = len(r["launches"])
        rd = sum(v["FETCH_SIZE_KiB"] for v in r["launches"].values()) * 1024 * scale["FETCH_SIZE"] / n
        wr = sum(v["WRITE_SIZE_KiB"] for v in r["launches"].values()) * 1024 * scale["WRITE_SIZE"] / n
        r["read_bytes_per_launch"], r["write_bytes_per_launch"] = int(rd), int(wr)
        r["bytes_per_launch"] = int(rd) + int(wr)
        h = hashlib.sha256()
        for src in r["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        r["sha256"] = h.hexdigest()
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print("scale: FETCH_SIZE x%.3f, WRITE_SIZE x%.3f" % (scale["FETCH_SIZE"], scale["WRITE_SIZE"]))
    print("| Dispatch | FETCH KiB | WRITE KiB | HBM read | HBM write |")
    print("|---|---:|---:|---:|---:|")
    for idx, (op, kernel) in enumerate(step_dispatches()):
        fk, wk = step["FETCH_SIZE"][idx], step["WRITE_SIZE"][idx]
        print("| `%s` %s | %.0f | %.0f | %.1f MB | %.1f MB |" % (kernel, op, fk, wk, fk * 1024 * scale["FETCH_SIZE"] / 1e6,
                                                              wk * 1024 * scale["WRITE_SIZE"] / 1e6))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--eager", action="store_true",
                   help="time the step as individual launches instead of one captured HIP graph")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    p.add_argument("--cpu-rows", type=int, default=1536, help="rows per linear in the CPU-baseline sample")
    p.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                   help="write profiles/hbm_traffic.json from two rocprofv3 counter databases (no GPU needed)")
    return p.parse_args()


class Workload:
    """Device tensors of one step: bf16 activations, pre-quantized weights, outputs."""

    def __init__(self, torch, mxq, inputs):
        dev = "cuda"
        self.mx, self.nv = [], []
        for name, N, K, epi in MX_LINEARS:
            x = inputs.to_torch(inputs.flux_activation(M_MX, K, seed=0, stream="bench/%s/A" % name), dev)
            w = inputs.to_torch(inputs.weight(N, K, seed=0, stream="bench/%s/W" % name), dev)
            b = inputs.to_torch(inputs.bias(N, K, seed=0, stream="bench/%s/b" % name), dev) if epi != "none" else None
            wq, ws = mxq.quantize_mxfp8(w, scale_layout=SCALES)
            aq = torch.empty((M_MX, K), dtype=torch.uint8, device=dev)
            as_ = torch.empty((M_MX, K // 32), dtype=torch.uint8, device=dev)
            c = torch.empty((M_MX, N), dtype=torch.bfloat16, device=dev)
            self.mx.append(dict(name=name, N=N, K=K, epi=epi, x=x, wq=wq, ws=ws, b=b, aq=aq, as_=as_, c=c))
            del w
        for name, N, K, epi in NV_LINEARS:
            x = inputs.to_torch(inputs.flux_activation(M_NV, K, seed=0, stream="bench/%s/A" % name), dev)
            w = inputs.to_torch(inputs.weight(N, K, seed=0, stream="bench/%s/W" % name), dev)
            wq, ws, wg = mxq.quantize_nvfp4(w, scale_layout=SCALES)
            aq = torch.empty((M_NV, K // 2), dtype=torch.uint8, device=dev)
            as_ = torch.empty((M_NV, K // 16), dtype=torch.uint8, device=dev)
            ag = torch.empty((1,), dtype=torch.float32, device=dev)
            ws_buf = torch.empty((max(mxq.nvfp4_workspace_size(M_NV, K), 4),), dtype=torch.uint8, device=dev)
            g_ws = mxq.gemm_nvfp4_workspace_size(M_NV, N, K)
            g_buf = torch.empty((g_ws,), dtype=torch.uint8, device=dev) if g_ws else None
            c = torch.empty((M_NV, N), dtype=torch.bfloat16, device=dev)
            self.nv.append(dict(name=name, N=N, K=K, epi=epi, x=x, wq=wq, ws=ws, wg=wg, aq=aq, as_=as_, ag=ag,
                                wsb=ws_buf, gws=g_buf, c=c))
            del w
        torch.cuda.synchronize()

    @staticmethod
    def kernel_of(name, epi):
        """HIP kernel function an op launches (the GEMM kernels are templated on the epilogue)."""
        e = {"none": 0, "bias": 1, "bias_gelu": 2}[epi]
        if name.startswith("gemm_mxfp8"):
            return "k_gemm_mxfp8<0, 0, %d, %s>" % (e, TILED_NAME)
        if name.startswith("gemm_nvfp4"):
            return "k_gemm_nvfp4<%d, false, true>" % e
        if name.startswith("quant_mxfp8"):
            return "k_quant_mxfp8<0, %s>" % TILED_NAME
        return "k_amax_partials + k_quant_nvfp4<%s>" % TILED_NAME

    def ops(self, mxq):
        """(op name, kind, callable) in step order."""
        out = []
        for L in self.mx:
            out.append(("quant_mxfp8_" + L["name"], "quant_mx",
                        lambda L=L: mxq.quantize_mxfp8(L["x"], "e4m3", out=(L["aq"], L["as_"]), scale_layout=SCALES)))
            out.append(("gemm_mxfp8_" + L["name"], "gemm_mx",
                        lambda L=L: mxq.gemm_mxfp8(L["aq"], L["as_"], L["wq"], L["ws"], bias=L["b"], epi=L["epi"],
                                                   out=L["c"], scale_layout=SCALES)))
        for L in self.nv:
            out.append(("quant_nvfp4_" + L["name"], "quant_nv",
                        lambda L=L: mxq.quantize_nvfp4(L["x"], out=(L["aq"], L["as_"], L["ag"]), workspace=L["wsb"],
                                                       scale_layout=SCALES)))
            out.append(("gemm_nvfp4_" + L["name"], "gemm_nv",
                        lambda L=L: mxq.gemm_nvfp4(L["aq"], L["as_"], L["ag"], L["wq"], L["ws"], L["wg"],
                                                   out=L["c"], workspace=L["gws"], scale_layout=SCALES)))
        return out

    def outputs(self):
        """Every tensor one step writes (codes, scales, GEMM outputs)."""
        out = []
        for L in self.mx:
            out += [L["aq"], L["as_"], L["c"]]
        for L in self.nv:
            out += [L["aq"], L["as_"], L["ag"], L["c"]]
        return out

    def work(self):
        """Algorithmic work per op: flops for GEMMs, bytes for quantizers (one read of
        the bf16 input, the codes and the scales written)."""
        w = {}
        for L in self.mx:
            n = M_MX * L["K"]
            w["quant_mxfp8_" + L["name"]] = ("bytes", 2 * n + n + n // 32)
            w["gemm_mxfp8_" + L["name"]] = ("flops", 2 * M_MX * L["N"] * L["K"])
        for L in self.nv:
            n = M_NV * L["K"]
            w["quant_nvfp4_" + L["name"]] = ("bytes", 2 * n + n // 2 + n // 16 + 4)
            w["gemm_nvfp4_" + L["name"]] = ("flops", 2 * M_NV * L["N"] * L["K"])
        return w


def static_scale_variant(torch, mxq, inputs, wl, reps: int = 20):
    """The single-stream NVFP4 activation quantizers with a static, calibrated
    decode scale instead of the dynamic one: calibration folds two synthetic
    activations per linear (the step's recipe, other seeds, 4608 rows) into the
    scale on the GPU; then the static (one-pass) and dynamic (two-pass)
    quantizers are timed back to back on the step's activation."""
    out = {"calibration": "2 synthetic activations per linear (4608 rows each, same recipe, other seeds)"}
    stream = torch.cuda.current_stream()
    for L in wl.nv:
        running = None
        for i in range(2):
            cal = inputs.to_torch(inputs.flux_activation(4608, L["K"], seed=0, stream="bench/%s/calib%d" % (L["name"], i)),
                                  "cuda")
            running = mxq.nvfp4_calibrate(cal, running)
            del cal
        g = torch.empty((1,), dtype=torch.float32, device="cuda")

        def run_static():
            mxq.quantize_nvfp4(L["x"], global_scale=running, out=(L["aq"], L["as_"], g), scale_layout=SCALES)

        def run_dynamic():
            mxq.quantize_nvfp4(L["x"], out=(L["aq"], L["as_"], g), workspace=L["wsb"], scale_layout=SCALES)

        res = {}
        for tag, f in (("static", run_static), ("dynamic", run_dynamic)):
            for _ in range(3):
                f()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                f()
            b.record(stream)
            torch.cuda.synchronize()
            res[tag] = a.elapsed_time(b) / reps
        n = M_NV * L["K"]
        nbytes = 2 * n + n // 2 + n // 16 + 4
        rate = nbytes / (res["static"] * 1e-3) / 1e9
        out["quant_nvfp4_" + L["name"]] = {
            "static_ms": round(res["static"], 4), "dynamic_ms": round(res["dynamic"], 4),
            "static_GB/s": round(rate, 1), "static_frac_of_hbm": round(rate / PEAK_HBM_GBPS, 4),
            "calibrated_scale": float(running[0])}
    return out


def weight_only_fp8_variant(torch, mxq, inputs, wl, reps: int = 20):
    """Weight-only FP8 on the double-stream linears: per-tensor E4M3 weights (quantized
    once, timed separately), the step's bf16 activations taken as they are, the same
    epilogues.  torch's bf16 GEMM on the same shapes is timed beside it for context."""
    out = {"weights": "per-tensor E4M3, dynamic scale from the weight's amax",
           "peak_TFLOP/s": PEAK_BF16_TFLOPS}
    stream = torch.cuda.current_stream()

    def timed(f):
        for _ in range(3):
            f()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            f()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    for L in wl.mx:
        w = inputs.to_torch(inputs.weight(L["N"], L["K"], seed=0, stream="bench/%s/W" % L["name"]), "cuda")
        q_ms = timed(lambda: mxq.quantize_fp8_weight(w))
        wq, ws = mxq.quantize_fp8_weight(w)
        c = torch.empty((M_MX, L["N"]), dtype=torch.bfloat16, device="cuda")
        g_ms = timed(lambda: mxq.gemm_bf16_fp8w(L["x"], wq, ws, bias=L["b"], epi=L["epi"], out=c))
        t_ms = timed(lambda: torch.matmul(L["x"], w.t()))
        flops = 2 * M_MX * L["N"] * L["K"]
        rate = flops / (g_ms * 1e-3) / 1e12
        out["gemm_bf16_fp8w_" + L["name"]] = {
            "shape": [M_MX, L["N"], L["K"]], "epi": L["epi"], "ms": round(g_ms, 4), "TFLOP/s": round(rate, 1),
            "frac": round(rate / PEAK_BF16_TFLOPS, 4), "torch_bf16_ms": round(t_ms, 4),
            "quantize_weight_ms": round(q_ms, 4)}
        del w, wq, ws, c
    return out


def fp8_attention_variant(torch, mxq, inputs, reps: int = 20):
    """FP8 multi-head attention at FLUX's joint attention shape (24 heads of 128
    over 4608 tokens): per-tensor E4M3 quantization of Q, K and V (timed apart),
    then the attention kernel; torch's bf16 scaled_dot_product_attention on the
    same tensors is timed beside it for context."""
    heads, L, d = 24, 4608, 128
    qb, kb, vb = inputs.attention_qkv(heads, L, d, seed=0, stream="bench/attn")
    q, k, v = (inputs.to_torch(x, "cuda") for x in (qb, kb, vb))
    stream = torch.cuda.current_stream()

    def timed(f):
        for _ in range(3):
            f()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            f()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    qc, qs = mxq.quantize_fp8_weight(q)
    kc, ks = mxq.quantize_fp8_weight(k)
    vc, vs = mxq.quantize_fp8_v(v, heads)
    o = torch.empty((heads * L, d), dtype=torch.bfloat16, device="cuda")
    a_ms = timed(lambda: mxq.attention_fp8(qc, qs, kc, ks, vc, vs, heads, out=o))
    q_ms = timed(lambda: (mxq.quantize_fp8_weight(q), mxq.quantize_fp8_weight(k), mxq.quantize_fp8_v(v, heads)))
    q4, k4, v4 = (x.view(1, heads, L, d) for x in (q, k, v))
    t_ms = timed(lambda: torch.nn.functional.scaled_dot_product_attention(q4, k4, v4))
    flops = 4 * heads * L * L * d
    rate = flops / (a_ms * 1e-3) / 1e12
    return {"shape": {"heads": heads, "tokens": L, "head_dim": d}, "flops": flops, "ms": round(a_ms, 4),
            "TFLOP/s": round(rate, 1), "frac_of_fp8_peak": round(rate / PEAK_TFLOPS["fp8"], 4),
            "quantize_qkv_ms": round(q_ms, 4), "torch_bf16_sdpa_ms": round(t_ms, 4)}


def cpu_baseline(rows_per_linear: int):
    """The oracle (as it is) on a bounded sample: `rows_per_linear` activation rows of
    every linear of the step, quantized (dynamic scales over the sampled rows) and
    multiplied against the full dequantized weights.  Weight dequantization is
    offline work, done before the clock starts, like the GPU's weight quantization."""
    import numpy as np

    import oracle
    from microscaling_quantized_dit_amd import inputs

    threads = oracle.max_threads()
    jobs = []
    for name, N, K, epi in MX_LINEARS:
        xa = inputs.flux_activation(rows_per_linear, K, seed=1, stream="cpu/%s/A" % name)
        w = inputs.weight(N, K, seed=0, stream="bench/%s/W" % name)
        wq, ws = oracle.quantize_mxfp8(w)
        b = inputs.bias(N, K, seed=0, stream="bench/%s/b" % name) if epi != "none" else None
        jobs.append(("mx", xa, oracle.dequant_mxfp8(wq, ws), b, epi, N, K))
    for name, N, K, epi in NV_LINEARS:
        xa = inputs.flux_activation(rows_per_linear, K, seed=1, stream="cpu/%s/A" % name)
        w = inputs.weight(N, K, seed=0, stream="bench/%s/W" % name)
        wq, ws, wg = oracle.quantize_nvfp4(w)
        jobs.append(("nv", xa, oracle.dequant_nvfp4(wq, ws, 1.0), wg, epi, N, K))
    flops = 0
    t0 = time.perf_counter()
    for kind, xa, wdeq, extra, epi, N, K in jobs:
        if kind == "mx":
            q, s = oracle.quantize_mxfp8(xa)
            a = oracle.dequant_mxfp8(q, s)
            e = {"none": oracle.EPI_NONE, "bias_gelu": oracle.EPI_BIAS_GELU_TANH}[epi]
            oracle.linear(a, wdeq, 1.0, extra, e)
        else:
            q, s, g = oracle.quantize_nvfp4(xa)
            a = oracle.dequant_nvfp4(q, s, 1.0)
            oracle.linear(a, wdeq, float(np.float64(g) * np.float64(extra)))
        flops += 2 * rows_per_linear * N * K
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d activation rows of each of the 6 linears (quantize + dequantize + fp64 GEMM "
                      "against full weights dequantized beforehand), %.1f s" % (rows_per_linear, dt)}


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the hot path runs on a single MI355X); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import microscaling_quantized_dit_amd as mxq
    from microscaling_quantized_dit_amd import inputs

    torch.cuda.set_device(0)
    mxq.load()
    t_gen = time.perf_counter()
    wl = Workload(torch, mxq, inputs)
    print("bench: inputs ready in %.1f s" % (time.perf_counter() - t_gen), file=sys.stderr, flush=True)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ops = wl.ops(mxq)
    work = wl.work()
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        for _, _, f in ops:
            f()
    torch.cuda.synchronize()

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ops]
          for _ in range(args.steps)]
    step_start, step_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_start.record(stream)
    for s in range(args.steps):
        for i, (_, _, f) in enumerate(ops):
            ev[s][i][0].record(stream)
            f()
            ev[s][i][1].record(stream)
    step_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = step_start.elapsed_time(step_end)
    ms_per_step = ms_per_step_eager = total_ms / args.steps

    # The step as one HIP graph (captured once, replayed per step): the same
    # launches without the host's launch gaps.  Every replay's outputs must equal
    # the eager step's bit for bit (checked after the first replay and after the
    # timed ones).
    graph_check = None
    if not args.eager:
        outs = wl.outputs()
        ref = [t.clone() for t in outs]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _, _, f in ops:
                f()
        for t in outs:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        first_ok = all(torch.equal(a, b) for a, b in zip(outs, ref))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step_start.record(stream)
        for _ in range(args.steps):
            graph.replay()
        step_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_per_step = step_start.elapsed_time(step_end) / args.steps
        last_ok = all(torch.equal(a, b) for a, b in zip(outs, ref))
        graph_check = {"first_replay_equals_eager": first_ok, "last_replay_equals_eager": last_ok}
        if not (first_ok and last_ok):
            raise SystemExit("bench.py: graph replay differs from the eager step")

    per_op = {}
    for i, (name, kind, _) in enumerate(ops):
        ms = sum(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)) / args.steps
        unit, amount = work[name]
        if unit == "flops":
            peak = PEAK_TFLOPS["fp8"] if kind == "gemm_mx" else PEAK_TFLOPS["fp4"]
            rate = amount / (ms * 1e-3) / 1e12
            per_op[name] = {"ms": round(ms, 4), "TFLOP/s": round(rate, 1), "frac_of_peak": round(rate / peak, 4),
                            "peak_TFLOP/s": peak}
            if kind == "gemm_nv":
                per_op[name]["frac_of_fp16_mfma_peak"] = round(rate / PEAK_TFLOPS["fp16"], 4)
        else:
            rate = amount / (ms * 1e-3) / 1e9
            per_op[name] = {"ms": round(ms, 4), "GB/s": round(rate, 1), "frac_of_hbm": round(rate / PEAK_HBM_GBPS, 4)}

    gemm_flops = sum(a for u, a in work.values() if u == "flops")
    q_bytes = sum(a for u, a in work.values() if u == "bytes")
    q_ms = sum(per_op[n]["ms"] for n in per_op if n.startswith("quant"))
    g_ms = sum(per_op[n]["ms"] for n in per_op if n.startswith("gemm"))
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12

    # dominant kernel: the HIP kernel function with the largest share of the step,
    # over all its launches (per launch: mean algorithmic work / mean duration)
    epis = {("gemm_mxfp8_" + L["name"]): L["epi"] for L in wl.mx}
    epis.update({("gemm_nvfp4_" + L["name"]): L["epi"] for L in wl.nv})
    by_kernel = {}
    for name in per_op:
        k = wl.kernel_of(name, epis.get(name, "none"))
        per_op[name]["kernel"] = k
        d = by_kernel.setdefault(k, {"ms": 0.0, "amount": 0, "launches": 0, "unit": work[name][0], "ops": []})
        d["ms"] += per_op[name]["ms"]
        d["amount"] += work[name][1]
        d["launches"] += 1
        d["ops"].append(name)
    dom = max(by_kernel, key=lambda k: by_kernel[k]["ms"])
    d = by_kernel[dom]
    avg_ms = d["ms"] / d["launches"]
    per_launch = d["amount"] / d["launches"]
    if d["unit"] == "flops":
        peak = PEAK_TFLOPS["fp8"] if "mxfp8" in dom else PEAK_TFLOPS["fp4"]
        achieved = per_launch / (avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": None}
    else:
        achieved = per_launch / (avg_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None}
    rec = measured_traffic(dom)
    if rec is not None:
        roofline["traffic"] = rec["bytes_per_launch"]
        roofline["traffic_read"] = rec["read_bytes_per_launch"]
        roofline["traffic_write"] = rec["write_bytes_per_launch"]
    roofline.update({"kernel": dom, "launches_per_step": d["launches"], "ops": d["ops"],
                     "avg_launch_ms": round(avg_ms, 4), "work_per_launch": per_launch,
                     "work_unit": d["unit"]})
    if "nvfp4" in dom:
        roofline["frac_of_fp16_mfma_peak"] = round(achieved / PEAK_TFLOPS["fp16"], 4)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8-e4m3 + nvfp4-e2m1 (bf16 out)",
        "data": "synthetic",
        "config": {
            "workload": "FLUX DiT block linears: double-stream MXFP8 E4M3 at M=4608 (QKV, out-proj, "
                        "MLP-up +bias+GELU, MLP-down) + single-stream NVFP4 at M=18432 (linear1, linear2); "
                        "each activation quantized per step, weights pre-quantized",
            "scale_layout": SCALES,
            "global_batch": 1, "seq_len": M_MX, "parallelism": "single GPU",
        },
        "gemm_TFLOP/s": round(gemm_flops / (g_ms * 1e-3) / 1e12, 1),
        "quantizer_GB/s": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
        "quantizer_frac_of_hbm": round(q_bytes / (q_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "wall_s": round(wall, 3),
        "timing": "one HIP graph per step" if graph_check else "individual launches",
        "ms_per_step_eager": round(ms_per_step_eager, 4),
        "graph_check": graph_check,
        "ops": per_op,
        "roofline": roofline,
    }
    result["static_activation_scale"] = static_scale_variant(torch, mxq, inputs, wl)
    result["weight_only_fp8"] = weight_only_fp8_variant(torch, mxq, inputs, wl)
    result["fp8_attention"] = fp8_attention_variant(torch, mxq, inputs)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
