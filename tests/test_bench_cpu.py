"""Host-side checks of the measurement code in bench.py (no GPU): the kernel-trace and
counter summaries it writes into profiles/, the HBM traffic from request counts, the
source hash that voids a stale counter summary, and the
command-line contract."""
import csv
import os
import statistics
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write_csv(path, fields, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summarize_trace_groups_by_kernel_and_shape(tmp_path):
    fields = ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"]
    rows = [{"Kernel_Name": "void plr::k_copy_direct<1>(plr::CopyArgs)", "Grid_Size_X": 1024,
             "Workgroup_Size_X": 128, "Start_Timestamp": 1000 * k, "End_Timestamp": 1000 * k + d}
            for k, d in enumerate([3000, 1000, 2000])]
    rows.append({"Kernel_Name": "void plr::k_copy_direct<1>(plr::CopyArgs)", "Grid_Size_X": 2048,
                 "Workgroup_Size_X": 128, "Start_Timestamp": 0, "End_Timestamp": 5000})
    rows.append({"Kernel_Name": "some_other_kernel", "Grid_Size_X": 1, "Workgroup_Size_X": 1,
                 "Start_Timestamp": 0, "End_Timestamp": 1})
    p = tmp_path / "t.csv"
    _write_csv(p, fields, rows)
    lines = bench.summarize_trace(str(p)).splitlines()
    assert len(lines) == 3 and "some_other" not in "".join(lines)
    f = lines[1].split()
    assert f[-7] == "1024" and f[-5] == "3"  # grid, calls
    assert [float(v) for v in f[-4:]] == [2.0, 2.0, 3.0, 1.0]  # avg, p50, p90, min (us)
    assert lines[2].split()[-4] == "5.00"


def test_counter_profiles_count_request_bytes(tmp_path, monkeypatch):
    """Traffic is request counts times request sizes, unscaled: 128-byte reads count 128
    bytes, 64-byte writes 64 (other writes 32); FETCH_SIZE, which weighs such reads at 64
    bytes, is reported beside it; ops that launch the same kernel share its mean."""
    fields = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    names = {op: k for op, (k, _) in bench.OP_KERNELS.items()}
    rows = {p: [] for p in bench.TRAFFIC_PASSES}
    for i, op in enumerate(names):
        k = names[op] + "(x)"
        r128, r64, r32, w64, wall = 1000 * (i + 1), 10 * (i + 1), i, 500 * (i + 1), 500 * (i + 1) + 3
        for c, v in (("TCC_EA0_RDREQ_128B_sum", r128), ("TCC_EA0_RDREQ_64B_sum", r64),
                     ("TCC_EA0_RDREQ_32B_sum", r32), ("TCC_EA0_RDREQ_sum", r128 + r64 + r32)):
            rows["rd"].append({"Kernel_Name": k, "Grid_Size": 1, "Counter_Name": c, "Counter_Value": v})
        for c, v in (("TCC_EA0_WRREQ_64B_sum", w64), ("TCC_EA0_WRREQ_sum", wall)):
            rows["wr"].append({"Kernel_Name": k, "Grid_Size": 1, "Counter_Name": c, "Counter_Value": v})
        rows["fetch"].append({"Kernel_Name": k, "Grid_Size": 1, "Counter_Name": "FETCH_SIZE",
                              "Counter_Value": (64 * (r128 + r64) + 32 * r32) / 1024})
        rows["write"].append({"Kernel_Name": k, "Grid_Size": 1, "Counter_Name": "WRITE_SIZE",
                              "Counter_Value": (64 * w64 + 32 * (wall - w64)) / 1024})
    for p, rr in rows.items():
        (tmp_path / p).mkdir()
        _write_csv(tmp_path / p / "b_counter_collection.csv", fields, rr)
    cal = {"rd": [("TCC_EA0_RDREQ_128B_sum", 1 << 23), ("TCC_EA0_RDREQ_64B_sum", 0), ("TCC_EA0_RDREQ_32B_sum", 0),
                  ("TCC_EA0_RDREQ_sum", 1 << 23)],
           "wr": [("TCC_EA0_WRREQ_64B_sum", 1 << 24), ("TCC_EA0_WRREQ_sum", 1 << 24)],
           "fetch": [("FETCH_SIZE", (1 << 29) / 1024)], "write": [("WRITE_SIZE", (1 << 30) / 1024)]}
    for p, cv in cal.items():
        (tmp_path / f"cal_{p}").mkdir()
        _write_csv(tmp_path / f"cal_{p}" / "c_counter_collection.csv", fields,
                   [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": 1, "Counter_Name": c, "Counter_Value": v}
                    for c, v in cv])
    out = tmp_path / "profiles"
    out.mkdir()
    bench.write_counter_profiles(str(tmp_path), str(out))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for op in names:
        same = [i for i, o in enumerate(names) if names[o] == names[op]]
        want = statistics.mean(128 * 1000 * (i + 1) + 64 * 10 * (i + 1) + 32 * i + 64 * 500 * (i + 1) + 32 * 3
                               for i in same)
        assert bench.counters_traffic(op) == pytest.approx(want), op
    text = (out / "reduce_counters.txt").read_text()
    assert "calibration_copy_1GiB_read_bytes: 1073741824" in text
    assert "calibration_copy_1GiB_fetch_size_bytes: 536870912" in text
    # a summary taken on other sources is void
    p = out / "reduce_counters.txt"
    p.write_text(p.read_text().replace(bench.source_hash("reduce"), "0" * 16))
    assert bench.counters_traffic("reduce") is None


def test_source_hash_covers_kernel_and_launch_code():
    for op, files in bench.OP_SOURCES.items():
        assert {"device_common.h", "kernels.h", "layout.cpp", "api.cpp"} <= set(files)
        assert any(f.endswith(".hip") for f in files)
        assert len(bench.source_hash(op)) == 16


@pytest.mark.parametrize("args,msg", [(["--gpus", "2"], "one GPU only"), (["--steps", "0"], "at least 1"),
                                      (["--collective", "ag", "--min-bytes", "100"], "powers of two")])
def test_command_line_contract(args, msg):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0 and msg in r.stderr, (r.returncode, r.stderr)


def test_parse_decode_trace_walks_the_schedule(tmp_path):
    """The decode kernel trace is cut along the child's schedule: warmup dispatches are
    skipped, producers count only where the mode has one, and a trace that does not match
    the schedule is reported, not misattributed."""
    import bench

    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    t = 0

    def add(name, us):
        nonlocal t
        rows.append(f"\"{name}\",{t},{t + int(us * 1000)}")
        t += 100000

    add("at::native::fill_kernel", 1.0)
    for us in (9.0, 3.0, 3.0, 5.0):  # notify_off warm: 1 warmup + 3 timed
        add("void plr::k_reduce_direct<0, 8, 1>(plr::ReduceArgs)", us)
    for us in (9.0, 4.0, 6.0, 4.0):  # notify_on warm
        add("void plr::k_notify(plr::NotifyArgs)", 2.0)
        add("void plr::k_reduce_direct<0, 8, 1>(plr::ReduceArgs)", us)
    for us in (8.0, 4.5, 4.0, 4.25):  # the local reduce, warm
        add("void plr::k_reduce_direct<0, 8, 1>(plr::ReduceArgs)", us)
    path = tmp_path / "dec_kernel_trace.csv"
    path.write_text("\n".join(rows) + "\n")
    sched = [[1, "notify_off", "warm", 1, 3], [1, "notify_on", "warm", 1, 3],
             [bench.LOCAL_KEY, "notify_off", "warm", 1, 3]]
    out = bench.parse_decode_trace(str(path), sched)
    assert out["T=1"]["notify_off"]["warm"]["p50_us"] == 3.0
    assert out["T=1"]["notify_off"]["warm"]["calls"] == 3
    assert out["T=1"]["notify_on"]["warm"]["p50_us"] == 4.0
    assert out["T=1"]["notify_on"]["warm"]["producer_p50_us"] == 2.0
    assert out[bench.LOCAL_KEY]["notify_off"]["warm"]["p50_us"] == 4.25
    assert "producer_p50_us" not in out[bench.LOCAL_KEY]["notify_off"]["warm"]
    assert "error" in bench.parse_decode_trace(str(path), sched + [[8, "notify_off", "warm", 1, 3]])
    assert "error" in bench.parse_decode_trace(str(path), sched[:1])


def test_cpu_baseline_on_a_small_step(monkeypatch):
    """The oracle baseline leg end to end on a miniature step (the same code path, small
    constants): every op and config is timed on all cores and on one, GB/s are positive."""
    import argparse

    import numpy as np

    import synth

    W = bench.W
    monkeypatch.setattr(bench, "R3", 64)
    monkeypatch.setattr(bench, "C3", 64)
    monkeypatch.setattr(bench, "B4", 16 * W * 64)
    monkeypatch.setattr(bench, "R5", 40)
    monkeypatch.setattr(bench, "RB5", 64)
    monkeypatch.setattr(bench, "BYTES", {"reduce": (W + 1) * 64 * 64 * 2, "allgather": 2 * W * bench.B4,
                                         "alltoall": 2 * W * bench.B4, "alltoallv": 2 * W * 40 * 64 + W * 40 * 4})
    p = synth.zipf_weights(1.1, W)
    host = {"r_src": [synth.normal_np(0, 3, w, 64 * 64, 0.5) for w in range(W)],
            "c_src": [synth.bits_np(0, 4, s, bench.B4) for s in range(W)],
            "v_src": [synth.bits_np(0, 6, s, 40 * 64) for s in range(W)],
            "v_dest": [synth.categorical_np(0, 5, s, 40, p) for s in range(W)]}
    args = argparse.Namespace(cpu_fraction=0.5, cpu_reps=1, seed=0)
    out = bench.run_cpu_baseline(args, host)
    assert out["kind"] == "oracle" and out["value"] > 0 and out["single_core"]["value"] > 0
    assert out["cores"] >= 1 and out["host"]["hardware_threads"] >= 1
    for k in ("reduce", "allgather", "alltoall", "alltoallv", "local_reduce_8x1M", "decode_T64"):
        assert out["per_op"][k]["GB/s_all_cores"] > 0 and out["per_op"][k]["GB/s_one_core"] > 0, k
    assert np.isfinite(out["seconds"])
