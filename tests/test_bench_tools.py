"""CPU checks of bench.py's command-line contract and of the summarizers that
turn rocprofv3 output into the committed profile summaries (synthetic CSVs
with known values)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

READ = "void at::native::elementwise_kernel_manual_unroll<128, 8, Foo>(int, Foo)"
STEP = "void (anonymous namespace)::k_step_fast<HIP_vector_type<int, 4u>, 2>(ns_state_view, int const*)"
PROJ = "void (anonymous namespace)::k_proj_mfma<1, 1, false, 1, 4, true>(uint4 const*, int)"
MERGE = "void (anonymous namespace)::k_merge_cols<4, true, 4, false>(float const*, int)"
FPROJ = "void (anonymous namespace)::k_proj_mfma<1, 1, false, 1, 4, true, true>(uint4 const*, int)"
FMERGE = "void (anonymous namespace)::k_merge_fused<4>(float const*, int)"


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kind", "Queue_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for name, t0, t1, q in rows:
            w.writerow(["KERNEL_DISPATCH", q, name, t0, t1])


def test_step_trace_summary(tmp_path):
    """Two cold indexed steps with spans of 5/5 and 4/6 us per kernel, one
    step broken by a kernel of another name, and a step on two queues: only
    the two intact steps are counted; two decode steps of 6 + 4 and 5 + 5
    us, and a decode step's first launch alone (not a step)."""
    rows, t = [], 1_000_000
    for durs in ((6000, 4000), (5000, 5000)):
        rows.append((READ, t, t + 90_000, 1))
        t += 90_000
        for name, d in zip((FPROJ, FMERGE), durs):
            rows.append((name, t, t + d, 1))
            t += d
    rows += [(READ, t, t + 90_000, 1), (FPROJ, t + 90_000, t + 96_000, 1)]
    t += 100_000
    for durs in ((5000, 5000, 4000), (4000, 6000, 5000)):
        rows.append((READ, t, t + 90_000, 1))
        t += 90_000
        for name, d in zip((STEP, PROJ, MERGE), durs):
            rows.append((name, t, t + d, 1))
            t += d
    rows.append((READ, t, t + 90_000, 1))
    t += 90_000
    rows.append((STEP, t, t + 5000, 1))
    rows.append(("void k_other(int)", t + 5000, t + 6000, 1))
    rows.append((MERGE, t + 6000, t + 9000, 1))
    t += 20_000
    rows.append((READ, t, t + 90_000, 1))
    t += 90_000
    rows += [(STEP, t, t + 5000, 1), (PROJ, t + 5000, t + 9000, 2), (MERGE, t + 9000, t + 12000, 1)]
    p = tmp_path / "trace.csv"
    _trace(p, rows)
    out = bench.step_trace_summary(str(p))
    assert "| indexed | 2 | k_step_fast | 4.500 | 4.500 | 4.000 | 5.000 |" in out
    assert "| indexed | 2 | k_proj_mfma | 5.500 |" in out
    assert "| indexed | 2 | k_merge_cols | 4.500 |" in out
    assert "Per-step kernel time (indexed, cold; the sum of its kernels' spans over 2 steps): " \
           "p10 14.10 us, median 14.50 us" in out
    assert "| decode | 2 | k_proj_mfma | 5.500 |" in out
    assert "| decode | 2 | k_merge_fused | 4.500 |" in out
    assert "Per-step kernel time (decode, cold; the sum of its kernels' spans over 2 steps): " \
           "p10 10.00 us, median 10.00 us" in out
    assert "| packed |" not in out


def _counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, val) in enumerate(rows):
            # two rows per dispatch, summed by the reader
            w.writerow([i + 1, name, "C", val / 2])
            w.writerow([i + 1, name, "C", val / 2])


def test_counter_summary_and_traffic_lookup(tmp_path):
    """FETCH_SIZE reads half the copy's bytes (calibration 2), WRITE_SIZE all
    of them (1): the summary scales each counter, for the indexed and the
    decode steps, and measured_traffic reads the result back only for a mean
    |I| within 5% of the recorded one."""
    step = [(READ, 1.0), (STEP, 10.0), (PROJ, 4000.0), (MERGE, 100.0)]
    dstep = [(READ, 1.0), (FPROJ, 4500.0), (FMERGE, 150.0)]
    _counters(tmp_path / "f.csv", step * 3 + [(READ, 1.0), (FPROJ, 1.0)] + dstep * 2)
    _counters(tmp_path / "w.csv", [(READ, 1.0), (STEP, 20.0), (PROJ, 100.0), (MERGE, 1.0)] * 3 +
              [(READ, 1.0), (FPROJ, 1.0)] + [(READ, 1.0), (FPROJ, 120.0), (FMERGE, 30.0)] * 2)
    kib = bench.COPY_PROBE_BYTES / 1024
    _counters(tmp_path / "cf.csv", [("__amd_rocclr_copyBuffer", kib / 2)] * 3)
    _counters(tmp_path / "cw.csv", [("__amd_rocclr_copyBuffer", kib)] * 3)
    line = {"metric": "m", "config": {"workload": "w", "mean_active": 1000.0, "mode": "decode",
                                "decode_two_launch_form": True},
            "roofline": {"bytes_per_launch": 8.05e6, "projection_stage": {"bytes_per_launch": 8.0e6},
                         "draft_call": {"bytes": 8.1e6}}}
    (tmp_path / "bench.out").write_text("progress\n" + json.dumps(line) + "\n")
    out = bench.counter_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                                str(tmp_path / "cw.csv"), str(tmp_path / "bench.out"))
    kv = dict(l.split(":", 1) for l in out.splitlines() if ":" in l and not l.startswith((" ", "#")))
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    assert float(kv["fetch_calibration"]) == pytest.approx(2.0)
    assert float(kv["write_calibration"]) == pytest.approx(1.0)
    proj = (4000.0 * 2 + 100.0) * 1024
    call = proj + (100.0 * 2 + 1.0) * 1024
    assert float(kv["traffic_bytes_per_projection"]) == pytest.approx(proj, abs=1)
    assert float(kv["traffic_bytes_per_call"]) == pytest.approx(call, abs=1)
    dproj = (4500.0 * 2 + 120.0) * 1024
    assert float(kv["traffic_bytes_per_decode_project"]) == pytest.approx(dproj, abs=1)
    assert float(kv["traffic_bytes_per_decode_step"]) == pytest.approx(dproj + (150.0 * 2 + 30.0) * 1024, abs=1)
    assert float(kv["algorithmic_bytes_per_decode_project"]) == pytest.approx(8.05e6)
    assert kv["source_sha256"] == bench.kernel_source_hash() and kv["modes"].split() == ["indexed", "decode"]
    p = tmp_path / "traffic.txt"
    p.write_text(out)
    assert bench.measured_traffic("w", "indexed", 1040.0, path=str(p)) == pytest.approx(call, abs=1)
    assert bench.measured_traffic("w", "decode", 1000.0, "traffic_bytes_per_decode_project",
                                  path=str(p)) == pytest.approx(dproj, abs=1)
    assert bench.measured_traffic("w", "indexed", 1060.0, path=str(p)) is None
    assert bench.measured_traffic("w", "packed", 1000.0, path=str(p)) is None


def test_committed_traffic_summary_matches_the_sources():
    """The committed draft-head counters were taken on the current kernel
    sources (else bench reports traffic null)."""
    path = os.path.join(ROOT, "profiles", "draft_head_llama3_8b_traffic.txt")
    kv = dict(l.split(":", 1) for l in open(path) if ":" in l and not l.startswith((" ", "#")))
    assert kv["source_sha256"].strip() == bench.kernel_source_hash()


def test_prefill_counter_summary(tmp_path):
    """k_prefill dispatches among others: counters are averaged over the
    k_prefill dispatches only and scaled by the copy calibration; the trace
    gives the mean duration."""
    PRE = "void (anonymous namespace)::k_prefill<0, true, 4>(void const*, int)"
    _counters(tmp_path / "f.csv", [(READ, 7.0), (PRE, 500000.0), (READ, 7.0), (PRE, 500010.0)])
    _counters(tmp_path / "w.csv", [(READ, 7.0), (PRE, 190.0), (READ, 7.0), (PRE, 200.0)])
    kib = bench.COPY_PROBE_BYTES / 1024
    _counters(tmp_path / "cf.csv", [("__amd_rocclr_copyBuffer", kib / 2)] * 3)
    _counters(tmp_path / "cw.csv", [("__amd_rocclr_copyBuffer", kib)] * 3)
    _trace(tmp_path / "t.csv", [(READ, 0, 90_000, 1), (PRE, 100_000, 280_000, 1), (PRE, 300_000, 500_000, 1)])
    out = bench.prefill_counter_summary(*(str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv", "t.csv")))
    kv = dict(l.split(":", 1) for l in out.splitlines() if ":" in l and not l.startswith((" ", "#")))
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    assert float(kv["traffic_bytes_per_call"]) == pytest.approx((500005.0 * 2 + 195.0) * 1024, abs=1)
    assert kv["source_sha256"] == bench.kernel_source_hash(bench.PREFILL_SOURCES)
    assert "mean 190.0 us, min 180.0, max 200.0" in out
