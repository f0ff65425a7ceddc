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
times come from HIP events on the launch stream around every launch (mean,
median, 10th and 90th percentile over the timed steps).  The CPU
oracle is timed on a bounded sample of the same work (cpu_baseline).

Beside the step the line carries legs that are not part of it: measured_peaks
(fp8 / fp16 matrix-core rates under load with the shader clock, a streaming
copy), quantizer_only (cold / warm), long_sequence_chain (M = 32768, K = 4096),
fused_quantize_gemm, torch_mxfp8_gemm (torch's own MXFP8 GEMM on the same
operands), static_activation_scale, weight_only_fp8 and fp8_attention.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --trace-table DB            # summaries of rocprofv3 databases
    python bench.py --record-traffic FETCH_DB WRITE_DB
    python bench.py --counter-table DB [DB ...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import statistics
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
        out.append(("gemm_mxfp8_" + name, "k_gemm_mxfp8<0, 0, %d, %s, 1>" % ({"none": 0, "bias": 1, "bias_gelu": 2}[epi],
                                                                           TILED_NAME)))
    for name, _, _, epi in NV_LINEARS:
        out.append(("quant_nvfp4_" + name, "k_amax_partials"))
        out.append(("quant_nvfp4_" + name, "k_quant_nvfp4<%s>" % TILED_NAME))
        out.append(("gemm_nvfp4_" + name, "k_gemm_nvfp4<%d, false, true>" % {"none": 0, "bias": 1, "bias_gelu": 2}[epi]))
    return out


def _step_rows(db):
    """Per dispatch of the step in a rocprofv3 counter database: (op, kernel,
    duration in ns, {counter: value summed over its instances}).  The step's
    dispatches are the ones right after the 1 GiB calibration copy; a GEMM's split
    and fixup dispatches, when there are any, are counted with it (durations
    added)."""
    import sqlite3
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute("select k.dispatch_id, k.name, k.end - k.start, p.counter_name, sum(p.counter_value) "
                       "from pmc_events p join kernels k on k.dispatch_id = p.dispatch_id "
                       "group by k.dispatch_id, p.counter_name order by k.dispatch_id").fetchall()
    disp = {}
    for did, name, dur, counter, value in rows:
        short = name.replace("mxq::(anonymous namespace)::", "").replace("void ", "").split("(")[0].strip()
        e = disp.setdefault(did, [short, float(dur), {}])
        e[2][counter] = float(value)
    order = sorted(disp)
    copies = [i for i, d in enumerate(order) if "copyBuffer" in disp[d][0]]
    if not copies:
        raise SystemExit("no calibration copy in %s" % db)
    j = max(copies, key=lambda i: disp[order[i]][1]) + 1
    out = []
    for op, kernel in step_dispatches():
        if j >= len(order) or disp[order[j]][0] != kernel:
            raise SystemExit("%s: expected %s at dispatch %d, found %s" % (
                db, kernel, j, disp[order[j]][0] if j < len(order) else None))
        name, dur, vals = disp[order[j]]
        vals = dict(vals)
        j += 1
        while j < len(order) and disp[order[j]][0].startswith(SPLIT_KERNELS):
            dur += disp[order[j]][1]
            for c, v in disp[order[j]][2].items():
                vals[c] = vals.get(c, 0.0) + v
            j += 1
        out.append((op, name, dur, vals))
    return out


def trace_table(db):
    """Markdown summary of a rocprofv3 kernel trace of
        python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline
    (1) per kernel function: calls, total and average duration, share of the
    traced GPU time (kernels under 0.2% left out); (2) per op of the step: the mean
    duration over every complete step sequence found in the trace (an op's split
    and fixup dispatches added to it), and the mean per launch of each step kernel
    over those sequences."""
    import sqlite3
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute("select name, end - start from kernels order by start").fetchall()

    def short(name):
        return name.replace("mxq::(anonymous namespace)::", "").replace("void ", "").split("(")[0].strip()
    names = [short(n) for n, _ in rows]
    durs = [float(d) for _, d in rows]
    total = sum(durs)
    stats = {}
    for n, d in zip(names, durs):
        e = stats.setdefault(n, [0, 0.0, float("inf"), 0.0])
        e[0] += 1
        e[1] += d
        e[2] = min(e[2], d)
        e[3] = max(e[3], d)
    print("| Kernel | Calls | Total (ns) | Average (ns) | % | Min (ns) | Max (ns) |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for n, (c, t, lo, hi) in sorted(stats.items(), key=lambda kv: -kv[1][1]):
        if t / total < 0.002:
            continue
        print("| `%s` | %d | %.0f | %.0f | %.2f | %.0f | %.0f |" % (n[:90], c, t, t / c, 100 * t / total, lo, hi))
    expect = step_dispatches()
    seqs, i = [], 0
    while i < len(names):
        j, ok, seq = i, True, []
        for op, kernel in expect:
            if j >= len(names) or names[j] != kernel:
                ok = False
                break
            d = durs[j]
            j += 1
            while j < len(names) and names[j].startswith(SPLIT_KERNELS):
                d += durs[j]
                j += 1
            seq.append(d)
        if ok:
            seqs.append(seq)
            i = j
        else:
            i += 1
    print()
    print("%d complete step sequences in the trace.  Per op (mean over them):" % len(seqs))
    print()
    print("| Op | Kernel | Mean (us) |")
    print("|---|---|---:|")
    for k, (op, kernel) in enumerate(expect):
        if seqs:
            print("| %s | `%s` | %.1f |" % (op, kernel, sum(s[k] for s in seqs) / len(seqs) / 1e3))


XCDS, SIMDS = 8, 1024          # MI355X: GRBM_GUI_ACTIVE is summed over the 8 XCDs; 256 CUs x 4 SIMDs


def counter_table(dbs):
    """Markdown table of the step's dispatches from rocprofv3 counter runs of
        python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --copy-calibration
    (each database one pass; GRBM_GUI_ACTIVE in every pass).  Derived columns:
      clock   = GRBM_GUI_ACTIVE / 8 / duration (the GPU clock over the dispatch)
      MFMA    = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8)
      VALU    = 4 SQ_ACTIVE_INST_VALU / (1024 x GRBM_GUI_ACTIVE / 8)
      LDS cf  = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (share of LDS cycles stalled)
      TA      = TA_BUSY_avr / (GRBM_GUI_ACTIVE / 8)
      L2 hit  = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)"""
    merged = None
    for db in dbs:
        rows = _step_rows(db)
        if merged is None:
            merged = [(op, k, [d], dict(v)) for op, k, d, v in rows]
        else:
            for m, (op, k, d, v) in zip(merged, rows):
                m[2].append(d)
                for c, x in v.items():
                    if c != "GRBM_GUI_ACTIVE":
                        m[3][c] = x
    print("| Op | Kernel | us | clock MHz | MFMA | VALU | LDS cf | TA | L2 hit |")
    print("|---|---|---:|---:|---:|---:|---:|---:|---:|")
    for op, kernel, durs, v in merged:
        ns = sum(durs) / len(durs)
        g = v.get("GRBM_GUI_ACTIVE", 0.0) / XCDS

        def ratio(num, den):
            return "%.2f" % (num / den) if den else "-"
        mfma = ratio(v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), SIMDS * g) if "SQ_VALU_MFMA_BUSY_CYCLES" in v else "-"
        valu = ratio(4 * v.get("SQ_ACTIVE_INST_VALU", 0.0), SIMDS * g) if "SQ_ACTIVE_INST_VALU" in v else "-"
        lds = ratio(v.get("SQ_LDS_BANK_CONFLICT", 0.0), v.get("SQ_LDS_IDX_ACTIVE", 0.0)) \
            if "SQ_LDS_BANK_CONFLICT" in v else "-"
        ta = ratio(v.get("TA_BUSY_avr", 0.0), g) if "TA_BUSY_avr" in v else "-"
        hit = ratio(v.get("TCC_HIT_sum", 0.0), v.get("TCC_HIT_sum", 0.0) + v.get("TCC_MISS_sum", 0.0)) \
            if "TCC_HIT_sum" in v else "-"
        print("| %s | `%s` | %.1f | %.0f | %s | %s | %s | %s | %s |" % (
            op, kernel, ns / 1e3, g / ns * 1e3 if ns else 0.0, mfma, valu, lds, ta, hit))


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
    p.add_argument("--trace-table", metavar="DB",
                   help="print per-kernel and per-op tables from a rocprofv3 kernel-trace database (no GPU needed)")
    p.add_argument("--counter-table", nargs="+", metavar="DB",
                   help="print the step's per-dispatch counter table from rocprofv3 counter databases (no GPU needed)")
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
            return "k_gemm_mxfp8<0, 0, %d, %s, 1>" % (e, TILED_NAME)
        if name.startswith("gemm_nvfp4"):
            return "k_gemm_nvfp4<%d, false, true>" % e
        if name.startswith("quant_mxfp8"):
            return "k_quant_mxfp8<0, %s>" % TILED_NAME
        return "k_amax_partials + k_quant_nvfp4<%s>" % TILED_NAME

    def single_launch(self, mxq, name):
        """Does this op run as one kernel launch?  The MXFP8 GEMMs do; an NVFP4 GEMM
        does unless its workspace holds split tiles (its size beyond the two
        operands' re-laid scales, which the tiled order leaves unused), and the
        dynamic NVFP4 quantizer is two launches (amax, encode)."""
        if name.startswith("quant_nvfp4"):
            return False
        if name.startswith("gemm_nvfp4"):
            L = next(L for L in self.nv if "gemm_nvfp4_" + L["name"] == name)
            r256 = lambda b: (b + 255) // 256 * 256
            scales = r256(M_NV * L["K"] // 16) + r256(L["N"] * L["K"] // 16)
            return mxq.gemm_nvfp4_workspace_size(M_NV, L["N"], L["K"]) <= scales
        return True

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


def static_scale_variant(torch, mxq, inputs, wl):
    """The single-stream NVFP4 activation quantizers with a static, calibrated
    decode scale instead of the dynamic one: calibration folds two synthetic
    activations per linear (the step's recipe, other seeds, 4608 rows) into the
    scale on the GPU; then the static (one-pass) and dynamic (two-pass)
    quantizers are timed in alternating rounds on the step's activation."""
    out = {"calibration": "2 synthetic activations per linear (4608 rows each, same recipe, other seeds)"}
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

        res = _interleaved_ms(torch, {"static": run_static, "dynamic": run_dynamic})
        n = M_NV * L["K"]
        nbytes = 2 * n + n // 2 + n // 16 + 4
        rate = nbytes / (res["static"] * 1e-3) / 1e9
        out["quant_nvfp4_" + L["name"]] = {
            "static_ms": round(res["static"], 4), "dynamic_ms": round(res["dynamic"], 4),
            "static_GB/s": round(rate, 1), "static_frac_of_hbm": round(rate / PEAK_HBM_GBPS, 4),
            "calibrated_scale": float(running[0])}
    return out


def spread(samples):
    """Median, 10th and 90th percentile (ms) of one op's per-step times; the three
    are the same value when there is a single sample."""
    if len(samples) < 2:
        v = round(float(samples[0]), 4) if samples else None
        return {"ms_median": v, "ms_p10": v, "ms_p90": v}
    q = statistics.quantiles(samples, n=10, method="inclusive")
    return {"ms_median": round(statistics.median(samples), 4), "ms_p10": round(q[0], 4), "ms_p90": round(q[8], 4)}


def _interleaved_ms(torch, fns, rounds: int = 15, inner: int = 5):
    """Median ms per call of each function in `fns` (name -> callable), timed in
    alternating rounds of `inner` back-to-back calls each (events on the current
    stream), so that clock and thermal drift during the measurement fall on all of
    them alike.  Each function is called three times first."""
    stream = torch.cuda.current_stream()
    for f in fns.values():
        for _ in range(3):
            f()
    times = {k: [] for k in fns}
    for _ in range(rounds):
        for k, f in fns.items():
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(inner):
                f()
            b.record(stream)
            torch.cuda.synchronize()
            times[k].append(a.elapsed_time(b) / inner)
    return {k: statistics.median(v) for k, v in times.items()}


def weight_only_fp8_variant(torch, mxq, inputs, wl):
    """Weight-only FP8 on the double-stream linears: per-tensor E4M3 weights (quantized
    once, timed separately), the step's bf16 activations taken as they are, the same
    epilogues.  torch's bf16 GEMM on the same shapes is timed beside it for context."""
    out = {"weights": "per-tensor E4M3, dynamic scale from the weight's amax",
           "peak_TFLOP/s": PEAK_BF16_TFLOPS, "timing": "ours and torch's in alternating rounds, medians"}
    for L in wl.mx:
        w = inputs.to_torch(inputs.weight(L["N"], L["K"], seed=0, stream="bench/%s/W" % L["name"]), "cuda")
        wq, ws = mxq.quantize_fp8_weight(w)
        c = torch.empty((M_MX, L["N"]), dtype=torch.bfloat16, device="cuda")
        if L["epi"] == "bias_gelu":   # torch's bf16 GEMM with the same epilogue
            ref = lambda: torch.nn.functional.gelu(torch.addmm(L["b"], L["x"], w.t()), approximate="tanh")
        else:
            ref = lambda: torch.matmul(L["x"], w.t())
        ms = _interleaved_ms(torch, {"ours": lambda: mxq.gemm_bf16_fp8w(L["x"], wq, ws, bias=L["b"], epi=L["epi"],
                                                                        out=c),
                                     "torch": ref, "quantize": lambda: mxq.quantize_fp8_weight(w)})
        g_ms, t_ms, q_ms = ms["ours"], ms["torch"], ms["quantize"]
        flops = 2 * M_MX * L["N"] * L["K"]
        rate = flops / (g_ms * 1e-3) / 1e12
        out["gemm_bf16_fp8w_" + L["name"]] = {
            "shape": [M_MX, L["N"], L["K"]], "epi": L["epi"], "ms": round(g_ms, 4), "TFLOP/s": round(rate, 1),
            "frac": round(rate / PEAK_BF16_TFLOPS, 4), "torch_bf16_ms": round(t_ms, 4),
            "vs_torch_bf16": round(g_ms / t_ms, 4),
            "quantize_weight_ms": round(q_ms, 4)}
        del w, wq, ws, c
    return out


def torch_mxfp8_gemm(torch, mxq, inputs, wl):
    """torch's own MXFP8 GEMM beside ours, on the same E4M3 codes and E8M0 scales:
    torch.nn.functional.scaled_mm with one scale per 32 K-values on both operands
    (row-major scales, no swizzle; ROCm builds run it on hipBLASLt), against
    mxq_gemm_mxfp8 with the scales in the row-major and in the tiled order.  No
    epilogue on either side (torch's call fuses no GELU).  Shapes: the step's
    double-stream linears and the long-sequence ones (32768 tokens, K = 4096).
    deviation: |torch - ours| over the whole output, relative to ours (Frobenius),
    and its largest element relative to max |ours|."""
    F = torch.nn.functional
    if not hasattr(F, "scaled_mm") or not hasattr(torch, "float8_e8m0fnu"):
        return {"error": "this torch has no scaled_mm with E8M0 scales"}
    out = {"call": "torch.nn.functional.scaled_mm, ScalingType.BlockWise1x32 on both operands, bf16 out",
           "timing": "alternating rounds, medians", "peak_TFLOP/s": PEAK_TFLOPS["fp8"]}
    shapes = [(L["name"], M_MX, L["N"], L["K"], L["x"], "bench/%s/W" % L["name"]) for L in wl.mx]
    xl = inputs.to_torch(inputs.long_sequence_activation(32768, 4096, seed=0, stream="cfg5/A"), "cuda")
    shapes += [("long_sequence_n%d" % n, 32768, n, 4096, xl, "cfg5/W%d" % n) for n in (4096, 16384)]
    for name, M, N, K, x, wstream in shapes:
        w = inputs.to_torch(inputs.weight(N, K, seed=0, stream=wstream), "cuda")
        aq, as_ = mxq.quantize_mxfp8(x, "e4m3")
        wq, ws = mxq.quantize_mxfp8(w, "e4m3")
        aqt, ast = mxq.quantize_mxfp8(x, "e4m3", scale_layout="tiled")
        wqt, wst = mxq.quantize_mxfp8(w, "e4m3", scale_layout="tiled")
        c_row = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        c_tiled = torch.empty_like(c_row)
        a8, b8 = aq.view(torch.float8_e4m3fn), wq.view(torch.float8_e4m3fn).t()
        sa, sb = as_.view(torch.float8_e8m0fnu), ws.view(torch.float8_e8m0fnu)

        def theirs():
            return F.scaled_mm(a8, b8, sa, F.ScalingType.BlockWise1x32, sb, F.ScalingType.BlockWise1x32,
                               swizzle_a=F.SwizzleType.NO_SWIZZLE, swizzle_b=F.SwizzleType.NO_SWIZZLE,
                               output_dtype=torch.bfloat16)
        try:
            ref = theirs()
            torch.cuda.synchronize()
        except Exception as e:      # a torch build without this path: say so, keep the rest of the line
            out[name] = {"error": "%s: %s" % (type(e).__name__, str(e).splitlines()[0][:200])}
            continue
        mine = mxq.gemm_mxfp8(aqt, ast, wqt, wst, out=c_tiled, scale_layout="tiled")
        d = (ref.float() - mine.float())
        mf = mine.float()
        dev = {"fro_rel": round((d.norm() / mf.norm()).item(), 6),
               "max_rel": round((d.abs().max() / mf.abs().max()).item(), 6)}
        ms = _interleaved_ms(torch, {
            "tiled": lambda: mxq.gemm_mxfp8(aqt, ast, wqt, wst, out=c_tiled, scale_layout="tiled"),
            "row": lambda: mxq.gemm_mxfp8(aq, as_, wq, ws, out=c_row),
            "torch": theirs})
        flops = 2 * M * N * K
        tf = lambda k: round(flops / (ms[k] * 1e-3) / 1e12, 1)
        out[name] = {"shape": [M, N, K], "ms": round(ms["tiled"], 4), "TFLOP/s": tf("tiled"),
                     "ms_row_scales": round(ms["row"], 4), "TFLOP/s_row_scales": tf("row"),
                     "torch_ms": round(ms["torch"], 4), "torch_TFLOP/s": tf("torch"),
                     "speedup_vs_torch": round(ms["torch"] / ms["tiled"], 3),
                     "speedup_vs_torch_row_scales": round(ms["torch"] / ms["row"], 3), "deviation": dev}
        del w, aq, as_, wq, ws, aqt, ast, wqt, wst, c_row, c_tiled, ref, mine, d, mf
    del xl
    torch.cuda.empty_cache()
    return out


def fp8_attention_variant(torch, mxq, inputs):
    """FP8 multi-head attention at FLUX's joint attention shape (24 heads of 128
    over 4608 tokens): per-tensor E4M3 quantization of Q, K and V (timed apart),
    then the attention kernel; torch's bf16 scaled_dot_product_attention on the
    same tensors is timed beside it for context."""
    heads, L, d = 24, 4608, 128
    qb, kb, vb = inputs.attention_qkv(heads, L, d, seed=0, stream="bench/attn")
    q, k, v = (inputs.to_torch(x, "cuda") for x in (qb, kb, vb))
    qc, qs = mxq.quantize_fp8_weight(q)
    kc, ks = mxq.quantize_fp8_weight(k)
    vc, vs = mxq.quantize_fp8_v(v, heads)
    o = torch.empty((heads * L, d), dtype=torch.bfloat16, device="cuda")
    q4, k4, v4 = (x.view(1, heads, L, d) for x in (q, k, v))
    ms = _interleaved_ms(torch, {
        "attention": lambda: mxq.attention_fp8(qc, qs, kc, ks, vc, vs, heads, out=o),
        "quantize": lambda: (mxq.quantize_fp8_weight(q), mxq.quantize_fp8_weight(k), mxq.quantize_fp8_v(v, heads)),
        "torch": lambda: torch.nn.functional.scaled_dot_product_attention(q4, k4, v4)})
    a_ms, q_ms, t_ms = ms["attention"], ms["quantize"], ms["torch"]
    flops = 4 * heads * L * L * d
    rate = flops / (a_ms * 1e-3) / 1e12
    return {"shape": {"heads": heads, "tokens": L, "head_dim": d}, "flops": flops, "ms": round(a_ms, 4),
            "TFLOP/s": round(rate, 1), "frac_of_fp8_peak": round(rate / PEAK_TFLOPS["fp8"], 4),
            "quantize_qkv_ms": round(q_ms, 4), "torch_bf16_sdpa_ms": round(t_ms, 4)}


def measured_peaks(torch):
    """What this machine attains, measured in the same run (libmxq_probes.so): the
    scaled fp8 and the fp16 matrix-core rates on back-to-back MFMAs from every
    compute unit with random register data, with the shader clock observed under
    that load, and a streaming 1 GiB device copy (bytes read + written)."""
    from microscaling_quantized_dit_amd import probes
    fp8, clk8 = probes.mfma_rate("fp8")
    fp16, clk16 = probes.mfma_rate("fp16")
    copy = probes.hbm_copy(1 << 30)
    return {"mfma_fp8_TFLOP/s": round(fp8, 1), "sclk_MHz_under_fp8": round(clk8, 0),
            "mfma_fp16_TFLOP/s": round(fp16, 1), "sclk_MHz_under_fp16": round(clk16, 0),
            "hbm_copy_GB/s": round(copy, 1),
            "note": "random register data; spec peaks: fp8 5000, fp16 2500 TFLOP/s at 2.4 GHz, HBM 8000 GB/s"}


def _graph_time(torch, fn, reps):
    """Mean ms of one replay of fn() captured as a HIP graph (replayed `reps` times
    back to back after one warm replay), timed with events on the replay stream."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                          # the calls once outside the graph (allocator warm-up)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def quantizer_only(torch, mxq, inputs, copy_gbps, reps: int = 10):
    """The quantizer-only workload: bf16 activations [4608, 3072] and [4608, 12288]
    (FLUX recipe), MXFP8 E4M3 (and E5M2) and NVFP4 with a dynamic scale, block
    scales in the GEMM-tiled order.  Cold: launches rotate over copies of the
    tensor and their outputs totalling >= 1 GiB (more than the 256 MB last-level
    cache), so every input comes from HBM.  Warm: one copy launched repeatedly.
    All launches of a pass are one captured graph (no host gaps)."""
    out = {"recipe": "flux_activation seed 0; cold = rotating copies totalling >= 1 GiB; warm = one copy",
           "nvfp4_two_read_bound_frac": round(2.5625 / 4.5625, 4)}
    for rows, cols in ((4608, 3072), (4608, 12288)):
        x0 = inputs.to_torch(inputs.flux_activation(rows, cols, seed=0, stream="cfg2/%dx%d" % (rows, cols)), "cuda")
        n = rows * cols
        for fmt in ("mxfp8_e4m3", "mxfp8_e5m2", "nvfp4"):
            if fmt == "nvfp4":
                per_set = 2 * n + n // 2 + n // 16
                algo = 2 * n + n // 2 + n // 16 + 4
            else:
                per_set = 2 * n + n + n // 32
                algo = per_set
            sets = max(2, -(-(1 << 30) // per_set))
            xs = [x0] + [x0.clone() for _ in range(sets - 1)]
            if fmt == "nvfp4":
                outs = [(torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda"),
                         torch.empty((rows, cols // 16), dtype=torch.uint8, device="cuda"),
                         torch.empty((1,), dtype=torch.float32, device="cuda")) for _ in range(sets)]
                ws = torch.empty((max(mxq.nvfp4_workspace_size(rows, cols), 4),), dtype=torch.uint8, device="cuda")

                def one(i):
                    mxq.quantize_nvfp4(xs[i], out=outs[i], workspace=ws, scale_layout=SCALES)
            else:
                kind = fmt.split("_")[1]
                outs = [(torch.empty((rows, cols), dtype=torch.uint8, device="cuda"),
                         torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")) for _ in range(sets)]

                def one(i, kind=kind):
                    mxq.quantize_mxfp8(xs[i], kind, out=outs[i], scale_layout=SCALES)

            cold = _graph_time(torch, lambda: [one(i) for i in range(sets)], reps) / sets
            warm = _graph_time(torch, lambda: [one(0) for _ in range(sets)], reps) / sets
            rec = {}
            for tag, ms in (("cold", cold), ("warm", warm)):
                gbps = algo / (ms * 1e-3) / 1e9
                rec[tag] = {"ms": round(ms, 4), "GB/s": round(gbps, 1), "frac_of_hbm": round(gbps / PEAK_HBM_GBPS, 4),
                            "frac_of_measured_copy": round(gbps / copy_gbps, 4) if copy_gbps else None}
                if fmt == "nvfp4":
                    rec[tag]["frac_of_two_read_bound"] = round(gbps / (PEAK_HBM_GBPS * 2.5625 / 4.5625), 4)
            rec["buffer_sets"] = sets
            rec["algorithmic_bytes"] = algo
            out["%s_%dx%d" % (fmt, rows, cols)] = rec
            del xs, outs
        del x0
    torch.cuda.synchronize()
    return out


def chain_long_sequence(torch, mxq, inputs, reps: int = 5):
    """The long-sequence chain: bf16 activations [32768, 4096] (N(0, 1), 0.1%
    outliers x50) quantized per call (tiled scales), then the block-scaled GEMM
    with bias against a weight [N, 4096] quantized beforehand, N in {4096, 16384},
    MXFP8 E4M3, MXFP8 E5M2 and NVFP4 (dynamic activation scale).  Each stage and the
    chain are timed as captured graphs."""
    M, K = 32768, 4096
    x = inputs.to_torch(inputs.long_sequence_activation(M, K, seed=0, stream="cfg5/A"), "cuda")
    out = {"shape": {"M": M, "K": K}, "recipe": "long_sequence_activation seed 0; weights N(0, 1/sqrt(K)); bias"}
    for N in (4096, 16384):
        w = inputs.to_torch(inputs.weight(N, K, seed=0, stream="cfg5/W%d" % N), "cuda")
        b = inputs.to_torch(inputs.bias(N, K, seed=0, stream="cfg5/b%d" % N), "cuda")
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        cf = torch.empty_like(c)
        flops = 2 * M * N * K
        for fmt in ("e4m3", "e5m2", "nvfp4"):
            if fmt == "nvfp4":
                wq, ws_, wg = mxq.quantize_nvfp4(w, scale_layout=SCALES)
                aq = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
                as_ = torch.empty((M, K // 16), dtype=torch.uint8, device="cuda")
                ag = torch.empty((1,), dtype=torch.float32, device="cuda")
                qws = torch.empty((max(mxq.nvfp4_workspace_size(M, K), 4),), dtype=torch.uint8, device="cuda")
                gsz = mxq.gemm_nvfp4_workspace_size(M, N, K)
                gws = torch.empty((gsz,), dtype=torch.uint8, device="cuda") if gsz else None
                qbytes = 2 * M * K + M * K // 2 + M * K // 16 + 4

                def quant():
                    mxq.quantize_nvfp4(x, out=(aq, as_, ag), workspace=qws, scale_layout=SCALES)

                def gemm():
                    mxq.gemm_nvfp4(aq, as_, ag, wq, ws_, wg, bias=b, epi="bias", out=c, workspace=gws,
                                   scale_layout=SCALES)
                peak = PEAK_TFLOPS["fp4"]
            else:
                wq, ws_ = mxq.quantize_mxfp8(w, fmt, scale_layout=SCALES)
                aq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
                as_ = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
                qbytes = 2 * M * K + M * K + M * K // 32

                def quant(fmt=fmt):
                    mxq.quantize_mxfp8(x, fmt, out=(aq, as_), scale_layout=SCALES)

                def gemm(fmt=fmt):
                    mxq.gemm_mxfp8(aq, as_, wq, ws_, bias=b, epi="bias", a_kind=fmt, w_kind=fmt, out=c,
                                   scale_layout=SCALES)
                peak = PEAK_TFLOPS["fp8"]
            q_ms = _graph_time(torch, quant, reps)
            g_ms = _graph_time(torch, gemm, reps)
            t_ms = _graph_time(torch, lambda: (quant(), gemm()), reps)
            gemm_rate = flops / (g_ms * 1e-3) / 1e12
            rec = {
                "quantize_ms": round(q_ms, 4), "quantize_GB/s": round(qbytes / (q_ms * 1e-3) / 1e9, 1),
                "gemm_ms": round(g_ms, 4), "gemm_TFLOP/s": round(gemm_rate, 1),
                "gemm_frac_of_peak": round(gemm_rate / peak, 4), "peak_TFLOP/s": peak,
                "chain_ms": round(t_ms, 4), "chain_TFLOP/s": round(flops / (t_ms * 1e-3) / 1e12, 1)}
            if fmt != "nvfp4":   # the same chain with the quantizer fused into the GEMM
                def fused(fmt=fmt):
                    mxq.gemm_mxfp8_fused(x, wq, ws_, kind=fmt, bias=b, epi="bias", out=cf, scale_layout=SCALES)
                f_ms = _graph_time(torch, fused, reps)
                quant(), gemm(), fused()
                torch.cuda.synchronize()
                rec["fused_ms"] = round(f_ms, 4)
                rec["fused_bit_identical"] = bool(torch.equal(c.view(torch.int16), cf.view(torch.int16)))
            out["%s_N%d" % (fmt, N)] = rec
        del w, b, c, cf
    del x
    torch.cuda.synchronize()
    return out


def fused_quantize_gemm(torch, mxq, inputs, wl, reps: int = 20):
    """The activation quantizer fused into the MXFP8 GEMM's prologue
    (mxq_gemm_mxfp8_fused, E4M3, the step's epilogues) against the separate
    quantize + GEMM on the double-stream linears.  Beside them: the GEMM alone, and
    a lower bound of any prologue fusion -- the GEMM with every A stage DMA'd twice
    (the bf16-sized A traffic) and no quantization work (libmxq_probes.so).  Each
    sequence is one captured graph replayed back to back; the fused output is
    checked bit-identical to the separate one."""
    from microscaling_quantized_dit_amd import probes
    out = {"lower_bound_probe": "k_gemm_mxfp8 with each A stage DMA'd twice (same bytes, same place)"}
    for L in wl.mx:
        c = torch.empty((M_MX, L["N"]), dtype=torch.bfloat16, device="cuda")
        cf = torch.empty_like(c)

        def quant():
            mxq.quantize_mxfp8(L["x"], "e4m3", out=(L["aq"], L["as_"]), scale_layout=SCALES)

        def gemm():
            mxq.gemm_mxfp8(L["aq"], L["as_"], L["wq"], L["ws"], bias=L["b"], epi=L["epi"], out=c,
                           scale_layout=SCALES)

        def fused():
            mxq.gemm_mxfp8_fused(L["x"], L["wq"], L["ws"], kind="e4m3", bias=L["b"], epi=L["epi"], out=cf,
                                 scale_layout=SCALES)

        def gemm2():
            probes.gemm_mxfp8_a_twice(L["aq"], L["as_"], L["wq"], L["ws"], c)

        sep = _graph_time(torch, lambda: (quant(), gemm()), reps)
        g_ms = _graph_time(torch, gemm, reps)
        f_ms = _graph_time(torch, fused, reps)
        lb = _graph_time(torch, gemm2, reps)
        quant(), gemm(), fused()
        torch.cuda.synchronize()
        same = bool(torch.equal(c.view(torch.int16), cf.view(torch.int16)))
        flops = 2 * M_MX * L["N"] * L["K"]
        out[L["name"]] = {"separate_quantize_then_gemm_ms": round(sep, 4), "gemm_ms": round(g_ms, 4),
                          "fused_ms": round(f_ms, 4), "fused_TFLOP/s": round(flops / (f_ms * 1e-3) / 1e12, 1),
                          "fused_over_separate": round(f_ms / sep, 4), "fused_bit_identical": same,
                          "a_twice_lower_bound_ms": round(lb, 4)}
        del c, cf
    return out


def cpu_model() -> str:
    """The host CPU's model name as the kernel reports it (empty if unknown)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


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
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle", "cpu": cpu_model(),
            "sample": "%d activation rows of each of the 6 linears (quantize + dequantize + fp64 GEMM "
                      "against full weights dequantized beforehand), %.1f s" % (rows_per_linear, dt)}


def main():
    args = parse()
    if args.trace_table:
        trace_table(args.trace_table)
        return
    if args.counter_table:
        counter_table(args.counter_table)
        return
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU (the hot path runs on a single MI355X); "
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
        samples = [ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]
        ms = sum(samples) / args.steps
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
        per_op[name].update(spread(samples))

    gemm_flops = sum(a for u, a in work.values() if u == "flops")
    q_bytes = sum(a for u, a in work.values() if u == "bytes")
    q_ms = sum(per_op[n]["ms"] for n in per_op if n.startswith("quant"))
    g_ms = sum(per_op[n]["ms"] for n in per_op if n.startswith("gemm"))
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12

    # dominant kernel: the HIP kernel function with the largest share of the step.
    # Its per-launch figures (mean algorithmic work / mean duration) are taken over
    # the ops that consist of that one launch (HIP events around the op time exactly
    # that kernel); an op that adds launches (an NVFP4 GEMM whose partial last round
    # is split along K adds the split launch and a fixup) is left out of the mean.
    epis = {("gemm_mxfp8_" + L["name"]): L["epi"] for L in wl.mx}
    epis.update({("gemm_nvfp4_" + L["name"]): L["epi"] for L in wl.nv})
    by_kernel = {}
    for name in per_op:
        k = wl.kernel_of(name, epis.get(name, "none"))
        per_op[name]["kernel"] = k
        single = wl.single_launch(mxq, name)
        per_op[name]["single_launch"] = single
        d = by_kernel.setdefault(k, {"ms": 0.0, "ms1": 0.0, "amount1": 0, "launches1": 0, "unit": work[name][0],
                                     "ops": [], "excluded": []})
        d["ms"] += per_op[name]["ms"]
        if single:
            d["ms1"] += per_op[name]["ms"]
            d["amount1"] += work[name][1]
            d["launches1"] += 1
            d["ops"].append(name)
        else:
            d["excluded"].append(name)
    dom = max(by_kernel, key=lambda k: by_kernel[k]["ms"])
    d = by_kernel[dom]
    avg_ms = d["ms1"] / d["launches1"]
    per_launch = d["amount1"] / d["launches1"]
    if d["unit"] == "flops":
        peak = PEAK_TFLOPS["fp8"] if "mxfp8" in dom else PEAK_TFLOPS["fp4"]
        achieved = per_launch / (avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": None}
    else:
        achieved = per_launch / (avg_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None}
    # HBM bytes per launch from the committed counter record, over the same ops
    rec = measured_traffic(dom)
    if rec is not None and all(op in rec["launches"] for op in d["ops"]):
        got = [rec["launches"][op] for op in d["ops"]]
        rd = sum(v["FETCH_SIZE_KiB"] for v in got) * 1024 * rec["scale"]["FETCH_SIZE"] / len(got)
        wr = sum(v["WRITE_SIZE_KiB"] for v in got) * 1024 * rec["scale"]["WRITE_SIZE"] / len(got)
        roofline["traffic"] = int(rd) + int(wr)
        roofline["traffic_read"] = int(rd)
        roofline["traffic_write"] = int(wr)
    roofline.update({"kernel": dom, "launches_per_step": d["launches1"] + len(d["excluded"]), "ops": d["ops"],
                     "ops_left_out": d["excluded"], "avg_launch_ms": round(avg_ms, 4),
                     "work_per_launch": per_launch, "work_unit": d["unit"]})
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
    print("bench: measured peaks", file=sys.stderr, flush=True)
    peaks = measured_peaks(torch)
    result["measured_peaks"] = peaks
    if roofline["bound"] == "mfma":
        # the MXFP8 GEMM runs on the scaled fp8 matrix core, the NVFP4 GEMM's exact
        # scheme on the fp16 one
        mp = peaks["mfma_fp8_TFLOP/s"] if "mxfp8" in dom else peaks["mfma_fp16_TFLOP/s"]
    else:
        mp = peaks["hbm_copy_GB/s"]
    roofline["peak_measured"] = mp
    roofline["frac_measured"] = round(achieved / mp, 4)
    print("bench: quantizer-only and long-sequence chain legs", file=sys.stderr, flush=True)
    result["quantizer_only"] = quantizer_only(torch, mxq, inputs, peaks["hbm_copy_GB/s"])
    result["long_sequence_chain"] = chain_long_sequence(torch, mxq, inputs)
    result["fused_quantize_gemm"] = fused_quantize_gemm(torch, mxq, inputs, wl)
    print("bench: torch's MXFP8 GEMM on the same operands", file=sys.stderr, flush=True)
    result["torch_mxfp8_gemm"] = torch_mxfp8_gemm(torch, mxq, inputs, wl)
    result["static_activation_scale"] = static_scale_variant(torch, mxq, inputs, wl)
    result["weight_only_fp8"] = weight_only_fp8_variant(torch, mxq, inputs, wl)
    result["fp8_attention"] = fp8_attention_variant(torch, mxq, inputs)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
