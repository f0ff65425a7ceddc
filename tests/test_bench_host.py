"""Host-side logic of bench.py, on the CPU: the summaries it writes from rocprofv3
databases (kernel trace, counter passes, the HBM byte record and its source hash)
and its refusal of more than one GPU.  The databases here are small SQLite files
with the two tables the bench queries (`kernels`, `pmc_events`), filled with a
made-up sequence of dispatches: a calibration copy, then one step's dispatches in
launch order (the NVFP4 linear2 GEMM followed by its split launch and fixup),
then unrelated kernels."""
import importlib.util
import io
import json
import os
import sqlite3
import subprocess
import sys
from contextlib import redirect_stdout

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _mangled(short):
    """A kernel name as rocprofv3 records it for one of the library's kernels."""
    if short.startswith("__amd") or short.startswith("other"):
        return short
    return "void mxq::(anonymous namespace)::%s(int, int)" % short


def _step(bench):
    """(name, duration ns, {counter: value}) of one step's dispatches: every
    dispatch of the step takes 1000 + 10 i ns and reads i + 1 KiB; linear2's GEMM
    is followed by a split launch and a fixup of 100 ns and 5 KiB each."""
    out = []
    for i, (op, kernel) in enumerate(bench.step_dispatches()):
        out.append((kernel, 1000.0 + 10 * i, {"FETCH_SIZE": i + 1.0, "GRBM_GUI_ACTIVE": 8000.0 + i,
                                                "SQ_VALU_MFMA_BUSY_CYCLES": 512.0}))
        if op == "gemm_nvfp4_linear2":
            out.append(("k_gemm_nvfp4<0, true, true>", 100.0, {"FETCH_SIZE": 5.0, "GRBM_GUI_ACTIVE": 800.0,
                                                               "SQ_VALU_MFMA_BUSY_CYCLES": 0.0}))
            out.append(("k_gemm_fixup<0>", 100.0, {"FETCH_SIZE": 5.0, "GRBM_GUI_ACTIVE": 800.0,
                                                  "SQ_VALU_MFMA_BUSY_CYCLES": 0.0}))
    return out


def _db(path, dispatches):
    con = sqlite3.connect(path)
    con.execute("create table kernels (dispatch_id integer, name text, start integer, end integer)")
    con.execute("create table pmc_events (dispatch_id integer, counter_name text, counter_value real)")
    t = 0
    for did, (name, dur, counters) in enumerate(dispatches):
        con.execute("insert into kernels values (?, ?, ?, ?)", (did, _mangled(name), t, t + int(dur)))
        for c, v in counters.items():   # two instances per counter, summed by the reader
            con.execute("insert into pmc_events values (?, ?, ?)", (did, c, v / 2))
            con.execute("insert into pmc_events values (?, ?, ?)", (did, c, v / 2))
        t += int(dur) + 50
    con.commit()
    con.close()
    return str(path)


def _dispatches(bench, copy_kib):
    copy = ("__amd_rocclr_copyBuffer", 300000.0, {"FETCH_SIZE": copy_kib, "WRITE_SIZE": copy_kib,
                                                  "GRBM_GUI_ACTIVE": 1.0})
    small_copy = ("__amd_rocclr_copyBuffer", 10.0, {"FETCH_SIZE": 1.0, "WRITE_SIZE": 1.0, "GRBM_GUI_ACTIVE": 1.0})
    other = ("other_kernel", 500.0, {"FETCH_SIZE": 9.0, "GRBM_GUI_ACTIVE": 1.0})
    return [small_copy, other, copy] + _step(bench) + [other]


def test_trace_table_sequences_and_split_launches(bench, tmp_path):
    """Two complete step sequences among other kernels: both are found, and
    linear2's op mean includes its split launch and fixup."""
    seq = _step(bench)
    disp = [("other_kernel", 500.0, {})] + seq + [("other_kernel", 500.0, {})] + seq
    db = _db(tmp_path / "trace.db", disp)
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench.trace_table(db)
    text = buf.getvalue()
    assert "2 complete step sequences" in text
    ops = bench.step_dispatches()
    i2 = [k for k, (op, _) in enumerate(ops) if op == "gemm_nvfp4_linear2"][0]
    want = (1000.0 + 10 * i2 + 200.0) / 1e3
    assert "| gemm_nvfp4_linear2 | `k_gemm_nvfp4<0, false, true>` | %.1f |" % want in text
    i0 = [k for k, (op, _) in enumerate(ops) if op == "gemm_mxfp8_qkv"][0]
    assert "| gemm_mxfp8_qkv | `%s` | %.1f |" % (ops[i0][1], (1000.0 + 10 * i0) / 1e3) in text


def test_counter_table_derived_columns(bench, tmp_path):
    """clock = GRBM_GUI_ACTIVE / 8 / duration; MFMA = busy / (1024 x GRBM / 8),
    from the step right after the largest copy."""
    db = _db(tmp_path / "pmc.db", _dispatches(bench, 1 << 19))
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench.counter_table([db])
    lines = [l for l in buf.getvalue().splitlines() if l.startswith("| quant_mxfp8_qkv")]
    assert len(lines) == 1
    cols = [c.strip() for c in lines[0].split("|")]
    # first dispatch: 1000 ns, GRBM 8000 -> 1000 cycles per XCD -> 1000 MHz; MFMA 512 / (1024 * 1000)
    assert cols[3] == "1.0" and cols[4] == "1000" and cols[5] == "%.2f" % (512 / (1024 * 1000))


def test_record_traffic_and_source_hash(bench, tmp_path, monkeypatch):
    """The byte record: scaled by the calibration copy (1 GiB = 2^20 KiB read and
    written: here the counters read half of it, so FETCH scales x2), split and fixup
    bytes added to linear2, and measured_traffic() honoured only while the
    recorded sources are unchanged."""
    root = tmp_path / "root"
    (root / "profiles").mkdir(parents=True)
    csrc = root / "microscaling_quantized_dit_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("quant_mxfp8.hip", "quant_nvfp4.hip", "gemm_mxfp8.hip", "gemm_nvfp4.hip", "gemm_fixup.hip",
              "mxq_internal.h"):
        (csrc / f).write_text("// " + f + "\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    # each pass holds its one counter, as a --pmc run of that counter alone does
    fetch = _db(tmp_path / "fetch.db", [(n, d, {"FETCH_SIZE": v.get("FETCH_SIZE", 0.0)}) for n, d, v in
                                        _dispatches(bench, float(1 << 19))])
    write = _db(tmp_path / "write.db", [(n, d, {"WRITE_SIZE": v.get("FETCH_SIZE", 0.0)}) for n, d, v in
                                        _dispatches(bench, float(1 << 20))])
    with redirect_stdout(io.StringIO()):
        bench.record_traffic(fetch, write)
    rec = json.loads((root / "profiles" / "hbm_traffic.json").read_text())
    ops = bench.step_dispatches()
    i2 = [k for k, (op, _) in enumerate(ops) if op == "gemm_nvfp4_linear2"][0]
    nv = rec["k_gemm_nvfp4<0, false, true>"]
    assert nv["scale"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    assert nv["launches"]["gemm_nvfp4_linear2"]["FETCH_SIZE_KiB"] == i2 + 1.0 + 10.0
    i1 = [k for k, (op, _) in enumerate(ops) if op == "gemm_nvfp4_linear1"][0]
    mean_kib = (i1 + 1.0 + i2 + 1.0 + 10.0) / 2
    assert nv["read_bytes_per_launch"] == int(mean_kib * 1024 * 2.0)
    assert bench.measured_traffic("k_gemm_nvfp4<0, false, true>")["bytes_per_launch"] == nv["bytes_per_launch"]
    (csrc / "gemm_fixup.hip").write_text("// changed\n")
    assert bench.measured_traffic("k_gemm_nvfp4<0, false, true>") is None
    assert bench.measured_traffic("k_gemm_mxfp8<0, 0, 0, true, 1>") is not None


def test_step_dispatches_match_the_workload(bench):
    """Two dispatches per MXFP8 linear, three plus the GEMM per NVFP4 linear, named
    as the kernels the step launches."""
    ops = bench.step_dispatches()
    assert len(ops) == 2 * len(bench.MX_LINEARS) + 3 * len(bench.NV_LINEARS)
    for op, kernel in ops:
        base = kernel.split("<")[0]
        assert base in bench.KERNEL_SOURCES, kernel


def test_more_than_one_gpu_is_refused():
    """--gpus 2 exits with status 2 and a message, before anything touches a GPU."""
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, env=env, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_per_op_spread(bench):
    """Per-op median and 10th / 90th percentiles over the timed steps."""
    s = bench.spread([float(v) for v in range(1, 12)])      # 1 .. 11
    assert s == {"ms_median": 6.0, "ms_p10": 2.0, "ms_p90": 10.0}
    assert bench.spread([0.25]) == {"ms_median": 0.25, "ms_p10": 0.25, "ms_p90": 0.25}
    s = bench.spread([3.0, 1.0])
    assert s["ms_p10"] <= s["ms_median"] <= s["ms_p90"] and s["ms_median"] == 2.0
