"""Benchmark of the single-GPU Atom datapath on one MI355X.

One step = one pass of the whole datapath over one batch of synthetic inputs, all
resident in HBM before timing starts, every consumer call notified (producer-side
plr_notify, then the consumer checks its per-chunk flags):
  1. reduce    W=8 contributions of [8192, 7168] bf16, N(0, 0.5)  -> one [8192, 7168] share
  2. allgather W=8 sources of 64 MiB random bits                  -> 512 MiB, packed by rank
  3. alltoall  W=8 sources of 8 x 8 MiB tiles                     -> 512 MiB, out[d][s] = in[s][d]
  4. alltoallv W=8 x 4096 rows of 7168 bf16, Zipf(1.1) destinations -> 32768 packed rows
`value` is the step's algorithmic HBM bytes (bytes read + bytes written) divided by
the wall-clock time of a step, K steps timed back to back with nothing in the stream
but the library's kernels. The same K steps are then run again with every op's
datapath kernels carrying a pair of timing-only HIP events (plr_set_timing_events);
their mean durations give `per_op` (with medians beside them) and the `roofline` of the
dominant kernel, the one with the largest share of the step's time (the copy kernel, which
runs twice per step), the figure a kernel trace of the same command reports for it.
Defaults: 10 warmup steps, then 50 timed.
Decode-size latency (W=8 x [T, 7168] bf16, T in 1/8/32/64) is reported beside it,
notify off and on and through packets: the time per call of 50 calls captured in a
HIP graph and replayed back to back (for notify on, a call is the producer's notify
plus the reduce), and p50/p90 of per-call timing-event pairs on the reduce kernel.

Prints one JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (W=8 bf16 reduce, layout copy) + p50 µs at decode size"
PEAK_HBM_GBS = 8000.0
W = 8
R3, C3 = 8192, 7168                 # reduce share [rows, cols] bf16
B4 = 64 << 20                       # bytes per copy source
R5, RB5 = 4096, 7168 * 2            # rows per source, row bytes
DECODE_T = (1, 8, 32, 64)

# algorithmic bytes per launch (bytes read + bytes written)
BYTES = {
    "reduce": (W + 1) * R3 * C3 * 2,
    "allgather": 2 * W * B4,
    "alltoall": 2 * W * B4,
    "alltoallv": 2 * W * R5 * RB5 + W * R5 * 4,
}
CSRC = os.path.join(ROOT, "reduce_atom_amd", "csrc")


# the sources a kernel and its launch are built from (the kernel's own file, the shared
# device code and argument blocks, and the host code that resolves its launch policy):
# a counter summary taken on other text of these files no longer describes the kernel
_HOST = ("device_common.h", "kernels.h", "layout.cpp", "api.cpp")
OP_SOURCES = {"reduce": ("reduce.hip",) + _HOST, "allgather": ("copy.hip",) + _HOST,
              "alltoall": ("copy.hip",) + _HOST, "alltoallv": ("copy_v.hip",) + _HOST}


def source_hash(op: str) -> str:
    h = hashlib.sha256()
    for name in OP_SOURCES[op]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def counters_traffic(op: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{op}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash(op):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def summarize_trace(path: str) -> str:
    """Per-kernel, per-launch-shape durations from a rocprofv3 kernel-trace CSV."""
    import collections
    import csv

    groups = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if "plr::" not in name and "direct_copy_kernel" not in name:
                continue
            short = name.split("(")[0].replace("void ", "")[:60]
            key = (short, int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
            groups[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    lines = [f"{'kernel':60s} {'grid_threads':>12s} {'wg':>4s} {'calls':>6s} {'avg_us':>9s} "
             f"{'p50_us':>8s} {'p90_us':>8s} {'min_us':>8s}"]
    for (k, grid, wg), v in sorted(groups.items()):
        v.sort()
        lines.append(f"{k:60s} {grid:12d} {wg:4d} {len(v):6d} {statistics.mean(v):9.2f} "
                     f"{v[len(v) // 2]:8.2f} {v[int(len(v) * 0.9)]:8.2f} {v[0]:8.2f}")
    return "\n".join(lines)


def summarize_counters(path: str) -> str:
    """Per-kernel, per-launch-shape mean counter values from a rocprofv3 counter CSV."""
    import collections
    import csv

    groups = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if "plr::" not in name and "direct_copy_kernel" not in name:
                continue
            short = name.split("(")[0].replace("void ", "")[:60]
            key = (short, int(r["Grid_Size"] if "Grid_Size" in r else r["Grid_Size_X"]), r["Counter_Name"])
            groups[key].append(float(r["Counter_Value"]))
    lines = [f"{'kernel':60s} {'grid_threads':>12s} {'counter':>12s} {'dispatches':>10s} {'mean':>16s}"]
    for (k, grid, c), v in sorted(groups.items()):
        lines.append(f"{k:60s} {grid:12d} {c:>12s} {len(v):10d} {statistics.mean(v):16.1f}")
    return "\n".join(lines)


# HBM traffic from the L2's memory-side request counters, each pass a run of its own
# (at most 4 TCC counters per pass): read requests by size, write requests by size, and
# the derived FETCH_SIZE / WRITE_SIZE beside them for comparison
TRAFFIC_PASSES = {
    "rd": "TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum TCC_EA0_RDREQ_sum",
    "wr": "TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum",
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
}
COUNTER_CMD = ("rocprofv3 --pmc {c} -f csv -d <dir>/{p} -o b -- python3 bench.py --steps 3 --warmup 1 "
               "--no-decode --no-cpu-baseline")
CALIB_CMD = "rocprofv3 --pmc {c} -f csv -d <dir>/cal_{p} -o c -- python3 bench.py --calibrate"
CALIB_KERNEL = "__amd_rocclr_copyBuffer"
# counters are taken per kernel; allgather and alltoall share the copy kernel and
# move the same bytes, so their dispatches are averaged together
OP_KERNELS = {"reduce": ("plr::k_reduce_direct", None), "allgather": ("plr::k_copy_direct", None),
              "alltoall": ("plr::k_copy_direct", None), "alltoallv": ("plr::k_copy_v_scatter", None)}


def _kernel_counters(path, name_part):
    """{counter: (mean over the kernel's dispatches, dispatches)} from a rocprofv3 counter CSV."""
    import csv

    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if name_part in r["Kernel_Name"]:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise ValueError(f"no dispatch of {name_part} in {path}")
    return {c: (statistics.mean(v), len(v)) for c, v in vals.items()}


def request_bytes(rd: dict, wr: dict):
    """(read bytes, write bytes) from the L2's memory-side request counts by size."""
    read = (32 * rd["TCC_EA0_RDREQ_32B_sum"][0] + 64 * rd["TCC_EA0_RDREQ_64B_sum"][0]
            + 128 * rd["TCC_EA0_RDREQ_128B_sum"][0])
    w64 = wr["TCC_EA0_WRREQ_64B_sum"][0]
    write = 64 * w64 + 32 * (wr["TCC_EA0_WRREQ_sum"][0] - w64)
    return read, write


def _pass_csv(d, name, prefix):
    return os.path.join(d, name, f"{prefix}_counter_collection.csv")


def write_counter_profiles(d, out_dir):
    """Per-op HBM traffic summaries from the counter passes under directory d (TRAFFIC_PASSES
    over the bench step in d/<pass>, over the calibration copy in d/cal_<pass>). Traffic is
    the read and write request counts times their sizes, with no scaling; FETCH_SIZE and
    WRITE_SIZE are reported beside it, and the calibration copy of 1 GiB (the HIP
    runtime's copy kernel) shows what each reads for a copy of known size."""
    cal = {p: _kernel_counters(_pass_csv(d, f"cal_{p}", "c"), CALIB_KERNEL) for p in TRAFFIC_PASSES}
    cal_r, cal_w = request_bytes(cal["rd"], cal["wr"])
    cal_fetch, cal_write = cal["fetch"]["FETCH_SIZE"][0] * 1024, cal["write"]["WRITE_SIZE"][0] * 1024
    cmds = [COUNTER_CMD.format(c=c, p=p) for p, c in TRAFFIC_PASSES.items()]
    cmds += [CALIB_CMD.format(c=c, p=p) for p, c in TRAFFIC_PASSES.items()]
    for op, (kname, _) in OP_KERNELS.items():
        k = {p: _kernel_counters(_pass_csv(d, p, "b"), kname) for p in TRAFFIC_PASSES}
        read, write = request_bytes(k["rd"], k["wr"])
        fetch, wsize = k["fetch"]["FETCH_SIZE"][0] * 1024, k["write"]["WRITE_SIZE"][0] * 1024
        traffic = read + write
        path = os.path.join(out_dir, f"{op}_counters.txt")
        with open(path, "w") as out:
            out.write(f"# HBM traffic per launch of {kname} ({op}) in the bench step, MI355X (gfx950)\n")
            out.write("# commands (one counter pass per run, <dir> any scratch directory):\n")
            for c in cmds:
                out.write(f"#   {c}\n")
            out.write("# then: python bench.py --counters-profile <dir>\n")
            out.write("# read bytes = 32 x RDREQ_32B + 64 x RDREQ_64B + 128 x RDREQ_128B; write bytes = 64 x WRREQ_64B\n"
                      "# + 32 x (WRREQ - WRREQ_64B) (TCC_EA0_* sums over all L2 channels of all XCDs).\n"
                      "# FETCH_SIZE counts every read request that is neither 32-byte nor a 'bubble' as 64 bytes;\n"
                      "# gfx950's reads here are 128-byte requests, so it reports half the bytes read.\n")
            out.write(f"kernel: {kname}\n")
            out.write(f"dispatches: {k['rd']['TCC_EA0_RDREQ_sum'][1]}\n")
            for p in ("rd", "wr"):
                for c, (m, _) in sorted(k[p].items()):
                    out.write(f"{c}: {m:.1f}\n")
            out.write(f"read_bytes_per_launch: {read:.0f}\nwrite_bytes_per_launch: {write:.0f}\n")
            out.write(f"fetch_size_bytes: {fetch:.0f}\nwrite_size_bytes: {wsize:.0f}\n")
            out.write(f"fetch_size_over_read_bytes: {fetch / read:.4f}\n")
            out.write(f"calibration_copy_1GiB_read_bytes: {cal_r:.0f}\ncalibration_copy_1GiB_write_bytes: {cal_w:.0f}\n")
            out.write(f"calibration_copy_1GiB_fetch_size_bytes: {cal_fetch:.0f}\n"
                      f"calibration_copy_1GiB_write_size_bytes: {cal_write:.0f}\n")
            out.write(f"traffic_bytes_per_launch: {traffic:.0f}\n")
            out.write(f"algorithmic_bytes_per_launch: {BYTES[op]}\n")
            out.write(f"traffic_over_algorithmic: {traffic / BYTES[op]:.4f}\n")
            out.write(f"source_hash: {source_hash(op)}\n")
        print(path, f"{traffic / BYTES[op]:.4f}")


# What bounds each streaming kernel: counter passes over one op run alone (bench.py --only)
BOUND_PASSES = {
    "lvl": "TCC_EA0_RDREQ_LEVEL_sum TCC_EA0_WRREQ_LEVEL_sum TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum "
           "TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum GRBM_GUI_ACTIVE",
    "req": "TCC_EA0_RDREQ_128B_sum TCC_EA0_WRREQ_64B_sum TCC_EA0_WRREQ_sum TCC_EA0_RDREQ_sum",
    "sq": "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_INST_ANY SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR GRBM_GUI_ACTIVE",
    "tcp": "TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum TCP_UTCL1_TRANSLATION_MISS_sum "
           "TCP_UTCL1_TRANSLATION_HIT_sum",
}
BOUND_OPS = {"reduce": "plr::k_reduce_direct", "allgather": "plr::k_copy_direct",
             "alltoallv": "plr::k_copy_v_scatter", "reduce_lds": "plr::k_reduce_lds",
             "allgather_lds": "plr::k_copy_lds", "allreduce_fused": "plr::k_allreduce_fused",
             "allreduce_cap3": "plr::k_allreduce_fused"}
BOUND_CMD = ("rocprofv3 --pmc {c} -f csv -d <dir>/{op}_{p} -o p -- python3 bench.py --only {op} --steps 5 "
             "--warmup 1")
XCDS = 8


def write_bound_profile(d, out_path):
    """Derived per-kernel figures from the BOUND_PASSES runs under d (d/<op>_<pass>):
    GPU cycles per XCD (GRBM_GUI_ACTIVE over the 8 XCDs), the mean number of read and
    write requests outstanding at the L2's memory interface (the _LEVEL sums over those
    cycles), the mean time a read request spends there (Little's law: outstanding /
    issue rate), the L1-to-L2 read latency, the share of cycles an L2 channel's DRAM
    request queue was full (credit stalls per channel), waves and their waiting."""
    rows = []
    for op, kname in BOUND_OPS.items():
        k = {}
        for p in BOUND_PASSES:
            k.update(_kernel_counters(_pass_csv(d, f"{op}_{p}", "p"), kname))
        v = {c: m for c, (m, _) in k.items()}
        cyc = v["GRBM_GUI_ACTIVE"] / XCDS
        chans = 16 * XCDS  # L2 channels
        rd_rate = v["TCC_EA0_RDREQ_sum"] / cyc
        rows.append((op, kname, {
            "cycles_per_xcd": cyc,
            "read_bytes": 128 * v["TCC_EA0_RDREQ_128B_sum"],
            "write_bytes": 64 * v["TCC_EA0_WRREQ_64B_sum"] + 32 * (v["TCC_EA0_WRREQ_sum"] - v["TCC_EA0_WRREQ_64B_sum"]),
            "reads_outstanding": v["TCC_EA0_RDREQ_LEVEL_sum"] / cyc,
            "writes_outstanding": v["TCC_EA0_WRREQ_LEVEL_sum"] / cyc,
            "read_requests_per_cycle": rd_rate,
            "read_residency_cycles": (v["TCC_EA0_RDREQ_LEVEL_sum"] / cyc) / rd_rate if rd_rate else 0.0,
            "l1_to_l2_read_latency_cycles": v["TCP_TCC_READ_REQ_LATENCY_sum"] / max(1.0, v["TCP_TCC_READ_REQ_sum"]),
            "dram_read_credit_stall_share": v["TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum"] / chans / cyc,
            "dram_write_credit_stall_share": v["TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum"] / chans / cyc,
            "waves": v["SQ_WAVES"],
            "wave_cycles_per_wave": v["SQ_WAVE_CYCLES"] / max(1.0, v["SQ_WAVES"]),
            "wait_share_of_wave_cycles": v["SQ_WAIT_INST_ANY"] / max(1.0, v["SQ_WAVE_CYCLES"]),
            "utcl1_miss_share": v["TCP_UTCL1_TRANSLATION_MISS_sum"] / max(
                1.0, v["TCP_UTCL1_TRANSLATION_MISS_sum"] + v["TCP_UTCL1_TRANSLATION_HIT_sum"]),
        }))
    with open(out_path, "w") as out:
        out.write("# What bounds the streaming kernels: rocprofv3 counters of each op run alone, MI355X (gfx950)\n")
        out.write("# commands (one pass per run; <op> in " + ", ".join(BOUND_OPS) + "):\n")
        for p, c in BOUND_PASSES.items():
            out.write(f"#   {BOUND_CMD.format(c=c, op='<op>', p=p)}\n")
        out.write("# then: python bench.py --bound-profile <dir>\n")
        for line in write_bound_profile.__doc__.strip().splitlines():
            out.write("# " + line.strip() + "\n")
        keys = list(rows[0][2])
        out.write(f"{'':34s}" + "".join(f"{op:>16s}" for op, _, _ in rows) + "\n")
        for key in keys:
            out.write(f"{key:34s}" + "".join(
                f"{r[key]:16.4f}" if r[key] < 10 else f"{r[key]:16.0f}" for _, _, r in rows) + "\n")
        for op, kname, _ in rows:
            out.write(f"# {op}: {kname}\n")
    print(open(out_path).read())


class TimingEvents:
    """HIP events for timing only, made with hipEventDisableSystemFence: recording one
    performs no system-scope cache writeback or invalidate, so it neither stalls the
    stream for several microseconds nor charges that stall to the kernels it brackets
    (torch's events do). Created and read through the HIP runtime that torch loaded."""

    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, torch):
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.hip = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so")
        self.made = []

    def create(self) -> int:
        h = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(self.FLAGS))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags: {rc}")
        self.made.append(h.value)
        return h.value

    def elapsed_ms(self, a: int, b: int) -> float:
        f = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime: {rc}")
        return f.value

    def record(self, e: int, stream: int) -> None:
        rc = self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord: {rc}")

    def destroy_all(self) -> None:
        for h in self.made:
            self.hip.hipEventDestroy(ctypes.c_void_p(h))
        self.made = []


def make_inputs(torch, synth, seed, dev):
    x = {}
    x["r_src"] = [synth.normal_t(seed, 3, w, R3 * C3, 0.5, device=dev) for w in range(W)]
    x["r_dst"] = torch.empty(R3 * C3, dtype=torch.bfloat16, device=dev)
    x["c_src"] = [synth.bits_t(seed, 4, s, B4, device=dev) for s in range(W)]
    x["ag_dst"] = torch.empty(W * B4, dtype=torch.uint8, device=dev)
    x["a2a_dst"] = torch.empty(W * B4, dtype=torch.uint8, device=dev)
    p = synth.zipf_weights(1.1, W)
    x["v_src"] = [synth.bits_t(seed, 6, s, R5 * RB5, device=dev) for s in range(W)]
    x["v_dest"] = [synth.categorical_t(seed, 5, s, R5, p, device=dev) for s in range(W)]
    x["v_dst"] = torch.empty(W * R5 * RB5, dtype=torch.uint8, device=dev)
    x["v_counts"] = torch.empty(W * W, dtype=torch.int64, device=dev)
    x["v_offsets"] = torch.empty(W * W, dtype=torch.int64, device=dev)
    return x


def host_inputs(torch, x):
    """The step's inputs as host numpy arrays (raw element bits), for the oracle."""
    import numpy as np

    def h(t):
        return t.view(torch.uint8).cpu().numpy()
    return {"r_src": [h(t).view(np.uint16) for t in x["r_src"]], "c_src": [h(t) for t in x["c_src"]],
            "v_src": [h(t) for t in x["v_src"]], "v_dest": [t.cpu().numpy() for t in x["v_dest"]]}


def run_bench(args):
    import torch

    import reduce_atom_amd as plr
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = make_inputs(torch, synth, args.seed, dev)
    L = {
        "reduce": plr.plr_layout_create("reduce", "bf16", W, R3 * C3 * 2, "packed", "packed"),
        "allgather": plr.plr_layout_create("copy", "bf16", W, B4, "packed", "packed"),
        "alltoall": plr.plr_layout_create("copy", "bf16", W, B4, "scattered", "transposed"),
    }
    ws = {k: torch.zeros(l.workspace_bytes, dtype=torch.uint8, device=dev) for k, l in L.items()}
    scratch = torch.zeros(plr.plr_copy_v_scratch_bytes(W, [R5] * W), dtype=torch.uint8, device=dev)

    def op(name):
        if name == "reduce":
            plr.plr_reduce(L[name], x["r_src"], x["r_dst"], ws[name])
        elif name == "allgather":
            plr.plr_copy(L[name], x["c_src"], x["ag_dst"], ws[name])
        elif name == "alltoall":
            plr.plr_copy(L[name], x["c_src"], x["a2a_dst"], ws[name])
        else:
            plr.plr_copy_v(x["v_src"], [R5] * W, x["v_dest"], RB5, x["v_dst"], x["v_counts"],
                           x["v_offsets"], scratch)

    ops = ["reduce", "allgather", "alltoall", "alltoallv"]

    def step(events=None):
        for name in ops:
            if name in L:
                plr.plr_notify(L[name], -1, ws[name])
            if events is not None:
                # the library records these around the op's datapath kernels (after a
                # notified call's check kernel), on the stream they run on: start and end
                # of the first dispatch and of the last (the same one for one kernel)
                plr.plr_set_timing_events_split(*events[name])
            op(name)
        if events is not None:
            plr.plr_set_timing_events_split()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # (1) the step as a whole: K steps back to back, nothing but the library's kernels
    t0 = time.perf_counter()
    for k in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # (2) the same K steps again, every op's datapath kernels carrying timing-only events:
    # the kernel-only duration that a kernel trace also reports. AllToAllV runs two
    # kernels, timed each on its own and summed (an event on the first dispatch delays
    # the second by about 4 us, which is not the op's time)
    E = TimingEvents(torch)
    ev = [{n: (E.create(), E.create(), E.create(), E.create()) for n in ops} for _ in range(args.steps)]

    def op_ms(n, e):
        if n == "alltoallv":
            return E.elapsed_ms(e[0], e[1]) + E.elapsed_ms(e[2], e[3])
        return E.elapsed_ms(e[0], e[3])
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    for name, l in L.items():
        rc = plr.plr_check(l, ws[name])
        if rc != plr.PLR_OK:
            raise RuntimeError(f"{name}: device error {plr.plr_strerror(rc)}")
    ms_per_step_events = (t3 - t2) * 1e3 / args.steps
    per_op_us = {n: statistics.mean(op_ms(n, e[n]) for e in ev) * 1e3 for n in ops}
    per_op_p50 = {n: statistics.median(op_ms(n, e[n]) for e in ev) * 1e3 for n in ops}
    E.destroy_all()
    step_bytes = sum(BYTES.values())
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # roofline of the dominant kernel: the one with the largest share of the step's time
    # (the copy kernel runs twice per step, for AllGather and AllToAll, with the same
    # bytes per launch; alltoallv is two kernels and is reported in per_op)
    launches = {"k_reduce_direct": ["reduce"], "k_copy_direct": ["allgather", "alltoall"]}
    dom_kernel = max(launches, key=lambda k: sum(per_op_us[n] for n in launches[k]))
    ops_k = launches[dom_kernel]
    avg_us = sum(per_op_us[n] for n in ops_k) / len(ops_k)
    achieved = sum(BYTES[n] for n in ops_k) / (sum(per_op_us[n] for n in ops_k) * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": counters_traffic(ops_k[0]),
                "kernel": dom_kernel, "op": "+".join(ops_k), "algorithmic_bytes": BYTES[ops_k[0]],
                "avg_us": round(avg_us, 2), "launches_per_step": len(ops_k)}
    per_op = {n: {"avg_us": round(per_op_us[n], 2), "p50_us": round(per_op_p50[n], 2),
                  "GB/s": round(BYTES[n] / (per_op_us[n] * 1e-6) / 1e9, 1),
                  "frac": round(BYTES[n] / (per_op_us[n] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
              for n in ops}
    per_op["target_frac"] = 0.8
    per_op["meets_target"] = {n: per_op[n]["frac"] >= 0.8 for n in ops}
    # the oracle's CPU baseline runs on these same input bytes, copied to the host
    host = None if args.no_cpu_baseline else host_inputs(torch, x)
    del x, ws, scratch
    torch.cuda.empty_cache()
    decode = run_decode(args, torch, plr, synth, dev) if not args.no_decode else None
    if decode is not None:
        decode = {"decode": decode, "local": run_local_reduce(args, torch, plr, synth, dev),
                  "producer": run_producer_kernel(args, torch, plr, synth, dev)}
    return value, ms_per_step, ms_per_step_events, roofline, per_op, decode, host


def graph_us_per_call(torch, once, iters, per_graph=50):
    """Mean microseconds per call of `once` with `per_graph` calls captured in one HIP graph
    and the graph replayed back to back (about `iters` calls in all), so that host-side call
    overhead does not starve the GPU. The captured launches are kernels only: no memory-set
    nodes."""
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for _ in range(per_graph):
                once()
    torch.cuda.current_stream().wait_stream(side)
    graph.replay()
    a0, b0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(1, iters // per_graph)
    torch.cuda.synchronize()
    a0.record()
    for _ in range(reps):
        graph.replay()
    b0.record()
    torch.cuda.synchronize()
    us = a0.elapsed_time(b0) * 1e3 / (per_graph * reps)
    del graph
    return us


def run_producer_kernel(args, torch, plr, synth, dev):
    """Producer kernels that announce their own chunks (tests/atom_kernels.hip, atom_produce:
    the producing kernel copies its input into the share, standing for any producing
    computation; section 3.2 and Figure 7), each followed by the library's consumer, per
    call in a replayed HIP graph, W = 8 x [T, 7168] bf16, every mode's result checked equal:
      ordered        plain stores, then the un-notified reduce (stream order alone, which
                     only a producer on the consumer's own GPU and stream can rely on);
      notify_kernel  plain stores, plr_notify (a separate release kernel), notified reduce;
      flags_fused    plain stores and each chunk's flag released by the producing kernel
                     (signal_flag), notified reduce;
      packets_fused  the producing kernel writes packets (store_packet), plr_reduce_packets."""
    path = os.path.join(ROOT, "tests", "libatom_kernels.so")
    if not os.path.exists(path):
        return "not built"
    lib = ctypes.CDLL(path)
    vp, sz, i, ull = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_ulonglong
    lib.atom_produce.argtypes = [i, i, ctypes.POINTER(vp), ctypes.POINTER(vp), sz, sz, vp, ull, vp]
    out = {}
    for T in (args.decode_t or DECODE_T):
        n = T * 7168
        share = 2 * n
        ins = [synth.normal_t(args.seed, 3, w, n, 1.0, device=dev) for w in range(W)]
        in_p = (vp * W)(*[t.data_ptr() for t in ins])
        dst = torch.empty(n, dtype=torch.bfloat16, device=dev)
        ref, res = None, {}
        for mode in ("ordered", "notify_kernel", "flags_fused", "packets_fused"):
            L = plr.plr_layout_create("reduce", "bf16", W, share, "packed", "packed")
            chunk = L.policy()["chunk_bytes"]
            if (share + chunk - 1) // chunk != L.nchunks:  # one producer workgroup per flag
                raise RuntimeError("producer chunks do not match the layout's flags")
            ws = torch.zeros(max(L.workspace_bytes, 256), dtype=torch.uint8, device=dev)
            nbytes = L.packet_bytes if mode == "packets_fused" else share
            outs = [torch.zeros(nbytes, dtype=torch.uint8, device=dev) for _ in range(W)]
            out_p = (vp * W)(*[t.data_ptr() for t in outs])
            pmode = {"ordered": 0, "notify_kernel": 0, "flags_fused": 1, "packets_fused": 2}[mode]

            def once():
                rc = lib.atom_produce(pmode, W, in_p, out_p, share, chunk, ws.data_ptr() + 256, L.epoch + 1,
                                      torch.cuda.current_stream().cuda_stream)
                if rc:
                    raise RuntimeError(f"atom_produce: {rc}")
                if mode == "ordered":
                    plr.plr_reduce(L, outs, dst)
                elif mode == "notify_kernel":
                    plr.plr_notify(L, -1, ws)
                    plr.plr_reduce(L, outs, dst, ws)
                elif mode == "flags_fused":
                    plr.plr_reduce(L, outs, dst, ws)
                else:
                    plr.plr_reduce_packets(L, outs, dst, ws)

            for _ in range(args.decode_warmup):
                once()
            torch.cuda.synchronize()
            if ref is None:
                ref = dst.clone()
            elif not torch.equal(dst, ref):
                raise RuntimeError(f"producer kernel {mode}: result differs from the ordered mode's")
            res[mode] = {"us_per_call_graph": round(graph_us_per_call(torch, once, args.decode_iters), 2)}
            if plr.plr_check(L, ws) != plr.PLR_OK:
                raise RuntimeError("producer kernel: device error")
        out[f"T={T}"] = res
    return out


def run_decode(args, torch, plr, synth, dev):
    out = {}
    for T in (args.decode_t or DECODE_T):
        n = T * 7168
        srcs = [synth.normal_t(args.seed, 2, w, n, 1.0, device=dev) for w in range(W)]
        dst = torch.empty(n, dtype=torch.bfloat16, device=dev)
        res = {}
        for mode in ("notify_off", "notify_on", "packets"):
            L = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed")
            ws = torch.zeros(max(L.workspace_bytes, 256), dtype=torch.uint8, device=dev) if mode != "notify_off" else None
            pk = [torch.zeros(L.packet_bytes, dtype=torch.uint8, device=dev) for _ in range(W)] \
                if mode == "packets" else None

            def produce():
                if pk is not None:
                    plr.plr_pack(L, -1, srcs, pk)
                elif ws is not None:
                    plr.plr_notify(L, -1, ws)

            def consume():
                if pk is not None:
                    plr.plr_reduce_packets(L, pk, dst, ws)
                else:
                    plr.plr_reduce(L, srcs, dst, ws)

            def once():
                produce()
                consume()

            for _ in range(args.decode_warmup):
                once()
            # (a) back to back on the GPU: 50 calls captured in one HIP graph, replayed
            per_call = graph_us_per_call(torch, once, args.decode_iters)
            # (b) a pair of timing-only events on every reduce kernel
            E = TimingEvents(torch)
            evs = [(E.create(), E.create()) for _ in range(args.decode_iters)]
            torch.cuda.synchronize()
            for a, b in evs:
                produce()
                plr.plr_set_timing_events(a, b)
                consume()
            plr.plr_set_timing_events()
            torch.cuda.synchronize()
            us = sorted(E.elapsed_ms(a, b) * 1e3 for a, b in evs)
            E.destroy_all()
            if ws is not None and plr.plr_check(L, ws) != plr.PLR_OK:
                raise RuntimeError("decode: device error")
            res[mode] = {"us_per_call_graph": round(per_call, 2),
                         "event_pair_p50_us": round(us[len(us) // 2], 2),
                         "event_pair_p90_us": round(us[int(len(us) * 0.9)], 2)}
        out[f"T={T}"] = res
    return out


DECODE_COLD_BYTES = 512 << 20  # the cold decode runs rotate over this much source memory
LOCAL_KEY = "local_8x1M"  # the local reduce's entry in the decode trace
CONSUMERS = ("k_reduce_direct", "k_reduce_packets")
PRODUCERS = ("k_notify", "k_pack")


def run_decode_trace_child(args):
    """Decode-size reduce calls for a kernel trace (run under rocprofv3 by
    run_decode_trace): for every T and mode (notify off, notify on, packets), warm (the
    same sources every call) and cold (each call's sources at another place of a
    512 MiB region, so that they are not in the L2 or the Infinity Cache), --decode-warmup
    calls and then --decode-iters calls, each one producer step (notify on: k_notify;
    packets: k_pack) and one consumer kernel. Then the local reduce of 8 x 1,048,576 bf16
    (uniform[-1, 1]) the same way, notify off, warm and cold (32 sets of 16 MiB). Prints
    the schedule as JSON."""
    import torch

    import reduce_atom_amd as plr
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    big = torch.empty(DECODE_COLD_BYTES, dtype=torch.uint8, device=dev)
    sched = []
    for T in (args.decode_t or DECODE_T):
        n = T * 7168
        nb = 2 * n
        srcs = [synth.normal_t(args.seed, 2, w, n, 1.0, device=dev) for w in range(W)]
        sets = DECODE_COLD_BYTES // (W * nb)
        cold = big[: sets * W * nb].view(sets, W, nb)
        cold.copy_(torch.stack([x.view(torch.uint8) for x in srcs]).unsqueeze(0).expand(sets, W, nb))
        cold_lists = [[cold[k, w] for w in range(W)] for k in range(min(sets, args.decode_warmup + args.decode_iters))]
        dst = torch.empty(n, dtype=torch.bfloat16, device=dev)
        for mode in ("notify_off", "notify_on", "packets"):
            L = plr.plr_layout_create("reduce", "bf16", W, nb, "packed", "packed")
            ws = torch.zeros(max(L.workspace_bytes, 256), dtype=torch.uint8, device=dev) if mode != "notify_off" else None
            pk = [torch.zeros(L.packet_bytes, dtype=torch.uint8, device=dev) for _ in range(W)] \
                if mode == "packets" else None
            for temp in ("warm", "cold"):
                for i in range(args.decode_warmup + args.decode_iters):
                    s_i = srcs if temp == "warm" else cold_lists[i % len(cold_lists)]
                    if pk is not None:
                        plr.plr_pack(L, -1, s_i, pk)
                        plr.plr_reduce_packets(L, pk, dst, ws)
                    else:
                        if ws is not None:
                            plr.plr_notify(L, -1, ws)
                        plr.plr_reduce(L, s_i, dst, ws)
                sched.append([T, mode, temp, args.decode_warmup, args.decode_iters])
            torch.cuda.synchronize()
            if ws is not None and plr.plr_check(L, ws) != plr.PLR_OK:
                raise RuntimeError(f"decode trace T={T} {mode}: device error")
        print(f"decode trace: T={T} done", file=sys.stderr, flush=True)
    n = 1 << 20
    srcs = [synth.uniform_pm1_t(args.seed, 1, w, n, device=dev) for w in range(W)]
    sets = DECODE_COLD_BYTES // (W * 2 * n)
    cold = big[: sets * W * 2 * n].view(sets, W, 2 * n)
    cold.copy_(torch.stack([x.view(torch.uint8) for x in srcs]).unsqueeze(0).expand(sets, W, 2 * n))
    cold_lists = [[cold[k, w] for w in range(W)] for k in range(sets)]
    dst = torch.empty(n, dtype=torch.bfloat16, device=dev)
    L = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed")
    for temp in ("warm", "cold"):
        for i in range(args.decode_warmup + args.decode_iters):
            plr.plr_reduce(L, srcs if temp == "warm" else cold_lists[i % sets], dst)
        sched.append([LOCAL_KEY, "notify_off", temp, args.decode_warmup, args.decode_iters])
    torch.cuda.synchronize()
    print("decode trace: local reduce done", file=sys.stderr, flush=True)
    print(json.dumps({"decode_trace_schedule": sched}), flush=True)


def _pct(v, q):
    return v[min(len(v) - 1, int(len(v) * q))]


def parse_decode_trace(path, sched):
    """Per (T, mode, warm / cold) statistics of the consumer kernel's traced duration from
    a rocprofv3 kernel-trace CSV, walking the dispatches in start order along the child's
    schedule [T, mode, temp, warmup calls, timed calls]: each call has one consumer
    dispatch, and one producer dispatch unless the mode is notify_off."""
    import csv

    cons, prod = [], []
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            t0 = int(row["Start_Timestamp"])
            us = (int(row["End_Timestamp"]) - t0) / 1000.0
            if any(k in name for k in CONSUMERS):
                cons.append((t0, us))
            elif any(k in name for k in PRODUCERS):
                prod.append((t0, us))
    cons.sort()
    prod.sort()
    out, ci, pi = {}, 0, 0
    for T, mode, temp, nw, ni in sched:
        c = sorted(us for _, us in cons[ci + nw: ci + nw + ni])
        ci += nw + ni
        if len(c) != ni:
            return {"error": f"trace holds {len(cons)} consumer dispatches, fewer than the schedule"}
        row = {"p50_us": round(_pct(c, 0.5), 2), "p90_us": round(_pct(c, 0.9), 2),
               "mean_us": round(statistics.mean(c), 2), "min_us": round(c[0], 2), "calls": len(c)}
        if mode != "notify_off":
            p = sorted(us for _, us in prod[pi + nw: pi + nw + ni])
            pi += nw + ni
            row["producer_p50_us"] = round(_pct(p, 0.5), 2) if p else None
        out.setdefault(T if T == LOCAL_KEY else f"T={T}", {}).setdefault(mode, {})[temp] = row
    if ci != len(cons) or pi != len(prod):
        return {"error": f"trace holds {len(cons)} consumer and {len(prod)} producer dispatches, "
                         f"the schedule {ci} and {pi}"}
    out["source"] = ("rocprofv3 kernel trace: consumer kernel duration per call (k_reduce_direct; packets: "
                     "k_reduce_packets), after the warmup calls; producer: k_notify / k_pack; "
                     f"{LOCAL_KEY}: the local reduce of 8 x 1,048,576 bf16, notify off")
    return out


def summarize_decode(path: str) -> str:
    """The decode-size latency rows of a bench JSON line (the last line of the file): the
    kernel-trace p50 / p90 of the consumer kernel per T, mode and warm / cold, the
    producer kernel's p50, and the per-call time in replayed graphs."""
    with open(path) as f:
        line = [x for x in f.read().splitlines() if x.startswith("{")][-1]
    full = json.loads(line)
    dec = full["decode_reduce_us"]
    kt = dec["kernel_trace"]
    out = [f"{'T':>4s} {'mode':11s} {'temp':5s} {'p50_us':>7s} {'p90_us':>7s} {'mean_us':>8s} {'min_us':>7s} "
           f"{'calls':>6s} {'producer_p50_us':>16s} {'graph_us_per_call':>18s}"]
    for T in (k for k in kt if k.startswith("T=")):
        for mode, temps in kt[T].items():
            for temp, r in temps.items():
                prod = r.get("producer_p50_us")
                graph = dec[T][mode]["us_per_call_graph"] if temp == "warm" else None
                out.append(f"{T[2:]:>4s} {mode:11s} {temp:5s} {r['p50_us']:7.2f} {r['p90_us']:7.2f} "
                           f"{r['mean_us']:8.2f} {r['min_us']:7.2f} {r['calls']:6d} "
                           f"{'' if prod is None else f'{prod:.2f}':>16s} {'' if graph is None else f'{graph:.2f}':>18s}")
    local = (full.get("local_reduce_8x1M_bf16") or {}).get("kernel_trace")
    if local:
        out.append("")
        out.append("local reduce, 8 x 1,048,576 bf16 (18,874,368 bytes), notify off")
        out.append(f"{'temp':5s} {'p50_us':>7s} {'p90_us':>7s} {'mean_us':>8s} {'min_us':>7s} {'calls':>6s} "
                   f"{'GB/s_at_p50':>12s}")
        for temp, r in local.items():
            out.append(f"{temp:5s} {r['p50_us']:7.2f} {r['p90_us']:7.2f} {r['mean_us']:8.2f} {r['min_us']:7.2f} "
                       f"{r['calls']:6d} {r['GB/s_at_p50']:12.1f}")
    return "\n".join(out)


def summarize_sweep(path: str) -> str:
    """Tables of a --collective or --v-sweep JSON output: time per call, HBM GB/s and (for
    the collectives) the pages' algbw, one row per size."""
    with open(path) as f:
        line = [x for x in f.read().splitlines() if x.startswith("{")][-1]
    d = json.loads(line)
    out = []
    if "collective_sweep" in d:
        cs = d["collective_sweep"]
        names = list(cs)
        sizes = [r["bytes"] for r in cs[names[0]]]
        for title, key, fmt in (("time per call, us", "us", "{:10.2f}"),
                                ("HBM GB/s (algorithmic bytes / time)", "hbm_GB/s", "{:10.1f}"),
                                ("algbw GB/s (page-convention bytes / time)", "algbw_GB/s", "{:10.1f}")):
            out.append(title)
            out.append(f"{'S_bytes':>12s}" + "".join(f"{n:>10s}" for n in names))
            for i, size in enumerate(sizes):
                out.append(f"{size:12d}" + "".join(fmt.format(cs[n][i][key]) for n in names))
            out.append("")
    else:
        out.append(f"{'T_bytes':>12s} {'largest_part':>12s} {'agv_us':>9s} {'agv_GB/s':>9s} {'rsv0_us':>9s} "
                   f"{'rsv0_GB/s':>9s}")
        for r in d["v_sweep"]:
            out.append(f"{r['T']:12d} {r['largest_part']:12d} {r['allgatherv_us']:9.2f} {r['allgatherv_GB/s']:9.1f} "
                       f"{r['reducescatterv_rank0_us']:9.2f} {r['reducescatterv_rank0_GB/s']:9.1f}")
    return "\n".join(out)


def run_decode_trace(args):
    """Kernel-trace latency of the decode-size reduce: this script's
    --decode-trace-child under `rocprofv3 --kernel-trace` in a child process (started
    before this process touches the GPU), then p50 / p90 of the consumer kernel's traced
    duration (k_reduce_direct, or k_reduce_packets for packets) per T, mode and warm /
    cold, with the producer kernel's p50 beside it."""
    import shutil
    import subprocess
    import tempfile

    prof = shutil.which("rocprofv3")
    if prof is None:
        return {"error": "rocprofv3 not found"}
    d = tempfile.mkdtemp(prefix="plr_decode_trace_")
    cmd = [prof, "--kernel-trace", "--output-format", "csv", "-d", d, "-o", "dec", "--", sys.executable,
           os.path.abspath(__file__), "--decode-trace-child", "--decode-iters", str(args.decode_iters),
           "--decode-warmup", str(args.decode_warmup), "--seed", str(args.seed)]
    if args.decode_t:
        cmd += ["--decode-t", ",".join(str(t) for t in args.decode_t)]
    try:
        r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=600)
        sched = None
        for line in r.stdout.splitlines():
            if line.startswith('{"decode_trace_schedule"'):
                sched = json.loads(line)["decode_trace_schedule"]
        path = os.path.join(d, "dec_kernel_trace.csv")
        if sched is None or not os.path.exists(path):
            return {"error": f"trace run ended with status {r.returncode} without its schedule or trace"}
        return parse_decode_trace(path, sched)
    except subprocess.TimeoutExpired:
        return {"error": "trace run timed out"}
    finally:
        shutil.rmtree(d, ignore_errors=True)


def _time_calls(torch, plr, fn, n=10, warm=3):
    """Mean datapath-kernel time of n calls, each carrying timing-only events."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    E = TimingEvents(torch)
    evs = [(E.create(), E.create()) for _ in range(n)]
    for a, b in evs:
        plr.plr_set_timing_events(a, b)
        fn()
    plr.plr_set_timing_events()
    torch.cuda.synchronize()
    us = statistics.mean(E.elapsed_ms(a, b) for a, b in evs) * 1e3
    E.destroy_all()
    return us


def run_next(args):
    """Rows beyond the step (measured beside it, not part of `value`): the AllReduce of
    W=8 contributions of [8192, 7168] bf16 into 8 outputs, fused and composed; and the
    variable-length collectives of appendix C.4 over 8 ranks with Zipf(s = 0.125)
    partitions of a total T: AllGatherV (8 contributions -> T bytes) and the largest
    ReduceScatterV share (rank 0: 8 contributions of T bytes, bf16, N(0, 1)), at
    T = 1 GiB (bandwidth) and T = 2 MiB (the size of the pages' largest gain); the
    LDS-staged pipeline beside the direct path at the step's reduce and AllGather; the
    HIP runtime's own device-to-device copy of the same 512 MiB; and the Atom user
    kernels."""
    import torch

    import reduce_atom_amd as plr
    import synth

    dev = torch.device("cuda:0")
    out = {}
    for T in (1 << 30, 2 << 20):
        parts = synth.zipf_split(T, W)
        tag = "1GiB" if T == 1 << 30 else "2MiB"
        srcs = [synth.bits_t(args.seed, 7, w, parts[w], device=dev) for w in range(W)]
        dst = torch.empty(T, dtype=torch.uint8, device=dev)
        L = plr.plr_layout_create("copy", "bf16", W, T, "packed", "packed", part_bytes=parts)
        us = _time_calls(torch, plr, lambda: plr.plr_copy(L, srcs, dst))
        algo = 2 * T
        out[f"allgatherv_{tag}"] = {"avg_us": round(us, 2), "GB/s": round(algo / (us * 1e-6) / 1e9, 1),
                                    "algorithmic_bytes": algo, "parts": parts}
        del srcs, dst
        srcs = [synth.normal_t(args.seed, 8, w, T // 2, 1.0, device=dev) for w in range(W)]
        dst = torch.empty(parts[0], dtype=torch.uint8, device=dev)
        L = plr.plr_layout_create("reduce", "bf16", W, T, "scattered", "packed", rank=0, part_bytes=parts)
        us = _time_calls(torch, plr, lambda: plr.plr_reduce(L, srcs, dst))
        algo = (W + 1) * parts[0]
        out[f"reducescatterv_rank0_{tag}"] = {"avg_us": round(us, 2), "GB/s": round(algo / (us * 1e-6) / 1e9, 1),
                                              "algorithmic_bytes": algo}
        del srcs, dst
        torch.cuda.empty_cache()
    srcs = [synth.normal_t(args.seed, 3, w, R3 * C3, 0.5, device=dev) for w in range(W)]
    dsts = [torch.empty(R3 * C3, dtype=torch.bfloat16, device=dev) for _ in range(W)]
    algo = 2 * W * R3 * C3 * 2  # W contributions read, W outputs written
    # the fused kernel at the policy's launch (8 workgroups per CU) and at 3 per CU, the
    # layout option that speeds it on separately allocated buffers such as these
    for name, path, cap in (("allreduce_fused", plr.PLR_PATH_DIRECT, 0), ("allreduce_cap3", plr.PLR_PATH_DIRECT, 3),
                            ("allreduce_composed", plr.PLR_PATH_COMPOSED, 0)):
        L = plr.plr_layout_create("allreduce", "bf16", W, R3 * C3 * 2, "scattered", "scattered", datapath=path,
                                  wgs_per_cu=cap)
        ws = torch.zeros(max(L.workspace_bytes, 256), dtype=torch.uint8, device=dev)
        us = _time_calls(torch, plr, lambda: plr.plr_allreduce(L, srcs, dsts, ws))
        if plr.plr_check(L, ws) != plr.PLR_OK:
            raise RuntimeError(f"{name}: device error")
        out[name] = {"avg_us": round(us, 2), "GB/s": round(algo / (us * 1e-6) / 1e9, 1),
                     "algorithmic_bytes": algo}
    del dsts
    # the LDS-staged pipeline (PLR_PATH_LDS) at the step's reduce and AllGather shapes,
    # notified as in the step, beside the direct path the policy uses
    rdst = torch.empty(R3 * C3, dtype=torch.bfloat16, device=dev)
    csrc = [synth.bits_t(args.seed, 4, s, B4, device=dev) for s in range(W)]
    cdst = torch.empty(W * B4, dtype=torch.uint8, device=dev)
    for name, make, call, algo in (
            ("reduce", lambda p: plr.plr_layout_create("reduce", "bf16", W, R3 * C3 * 2, "packed", "packed", datapath=p),
             lambda L, ws: plr.plr_reduce(L, srcs, rdst, ws), BYTES["reduce"]),
            ("allgather", lambda p: plr.plr_layout_create("copy", "bf16", W, B4, "packed", "packed", datapath=p),
             lambda L, ws: plr.plr_copy(L, csrc, cdst, ws), BYTES["allgather"])):
        for tag, path in (("lds", plr.PLR_PATH_LDS), ("direct", plr.PLR_PATH_DIRECT)):
            L = make(path)
            ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device=dev)

            def notified(L=L, ws=ws):
                plr.plr_notify(L, -1, ws)
                call(L, ws)
            us = _time_calls(torch, plr, notified)
            if plr.plr_check(L, ws) != plr.PLR_OK:
                raise RuntimeError(f"{name} {tag}: device error")
            out[f"{name}_{tag}_path"] = {"avg_us": round(us, 2), "GB/s": round(algo / (us * 1e-6) / 1e9, 1),
                                          "algorithmic_bytes": algo}
    # the HIP runtime's own device-to-device copy (torch's copy_ of one contiguous
    # buffer: hipMemcpyAsync) of the step AllGather's 512 MiB, as an anchor for what a
    # plain copy reaches on this machine; events on the stream the copy runs on
    E = TimingEvents(torch)
    flat = torch.cat([c.view(-1) for c in csrc])
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        cdst.copy_(flat)
    torch.cuda.synchronize()
    evs = [(E.create(), E.create()) for _ in range(10)]
    for a, b in evs:
        E.record(a, st)
        cdst.copy_(flat)
        E.record(b, st)
    torch.cuda.synchronize()
    us = statistics.mean(E.elapsed_ms(a, b) for a, b in evs) * 1e3
    E.destroy_all()
    if not torch.equal(cdst, flat):
        raise RuntimeError("runtime copy: wrong result")
    out["runtime_copy_512MiB"] = {"avg_us": round(us, 2), "GB/s": round(BYTES["allgather"] / (us * 1e-6) / 1e9, 1),
                                  "algorithmic_bytes": BYTES["allgather"]}
    del rdst, csrc, cdst, flat
    out.update(run_atom_user_kernels(torch, srcs))
    del srcs
    torch.cuda.empty_cache()
    return out


def run_local_reduce(args, torch, plr, synth, dev):
    """The local reduce of 8 contributions of 1,048,576 bf16 (uniform[-1, 1]) into one
    share, 18 MiB of traffic per call: warm (the same buffers back to back, L2 and the
    256 MB Infinity Cache hold them) and cold (rotating among 40 buffer sets, 720 MiB,
    so that every call's inputs have left the caches). Kernel-only time per call from
    timing-only events, median of 50 after 10 warmup calls."""
    n = 1 << 20
    sets = 40
    bufs = [[synth.uniform_pm1_t(args.seed, 1, w, n, device=dev) if k == 0 else None for w in range(W)]
            for k in range(sets)]
    for k in range(1, sets):  # the same values in every set, different memory
        bufs[k] = [b.clone() for b in bufs[0]]
    dst = torch.empty(n, dtype=torch.bfloat16, device=dev)
    L = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed")
    E = TimingEvents(torch)
    out = {}
    for mode in ("warm", "cold"):
        calls = [0] * 60 if mode == "warm" else [k % sets for k in range(60)]
        evs = [(E.create(), E.create()) for _ in calls]
        torch.cuda.synchronize()
        for (a, b), k in zip(evs, calls):
            plr.plr_set_timing_events(a, b)
            plr.plr_reduce(L, bufs[k], dst)
        plr.plr_set_timing_events()
        torch.cuda.synchronize()
        us = sorted(E.elapsed_ms(a, b) * 1e3 for a, b in evs[10:])
        p50 = us[len(us) // 2]
        out[mode] = {"p50_us": round(p50, 2), "GB/s_at_p50": round(9 * 2 * n / (p50 * 1e-6) / 1e9, 1)}
    E.destroy_all()
    return out


def run_v_sweep(args):
    """AllGatherV and the rank-0 ReduceScatterV share over 8 ranks with the Zipf
    (s = 0.125) split of a total T, for T = 1 KiB .. 1 GiB (appendix C.4's sweep):
    kernel-only time per call (timing-only events, median of 20 after 5 warmup calls)
    and the algorithmic GB/s at that time. Sources are allocated once at the largest T."""
    import torch

    import reduce_atom_amd as plr
    import synth

    dev = torch.device("cuda:0")
    Tmax = 1 << 30
    E = TimingEvents(torch)
    stream = torch.cuda.current_stream().cuda_stream

    def median_us(fn, n=20):
        for _ in range(5):
            fn()
        evs = [(E.create(), E.create()) for _ in range(n)]
        torch.cuda.synchronize()
        for a, b in evs:
            plr.plr_set_timing_events(a, b)
            fn()
        plr.plr_set_timing_events()
        torch.cuda.synchronize()
        t = sorted(E.elapsed_ms(a, b) * 1e3 for a, b in evs)
        return t[len(t) // 2]

    rows = []
    big = synth.zipf_split(Tmax, W)
    g_src = [synth.bits_t(args.seed, 7, w, big[w], device=dev) for w in range(W)]
    g_dst = torch.empty(Tmax, dtype=torch.uint8, device=dev)
    r_src = [synth.normal_t(args.seed, 8, w, Tmax // 2, 1.0, device=dev) for w in range(W)]
    r_dst = torch.empty(big[0], dtype=torch.uint8, device=dev)
    T = 1024
    while T <= Tmax:
        parts = synth.zipf_split(T, W)
        L = plr.plr_layout_create("copy", "bf16", W, T, "packed", "packed", part_bytes=parts)
        ag = median_us(lambda: plr.plr_copy(L, g_src, g_dst))
        R = plr.plr_layout_create("reduce", "bf16", W, T, "scattered", "packed", rank=0, part_bytes=parts)
        rs = median_us(lambda: plr.plr_reduce(R, r_src, r_dst))
        rows.append({"T": T, "largest_part": parts[0],
                     "allgatherv_us": round(ag, 2), "allgatherv_GB/s": round(2 * T / ag / 1e3, 1),
                     "reducescatterv_rank0_us": round(rs, 2),
                     "reducescatterv_rank0_GB/s": round((W + 1) * parts[0] / rs / 1e3, 1)})
        T *= 2
    E.destroy_all()
    del stream
    return rows


COLLECTIVES = ("ar", "a2a", "a2av", "ag", "agv", "rs", "rsv")


def run_collective_sweep(args):
    """The pages' per-collective microbenchmarks (testAR, testA2A, testA2AV, testAG,
    testAGV, testRS, testRSV: minimum and maximum bytes, graph launches, runs, warmup,
    seed) on one GPU's share of W = 8 ranks, sizes doubling from min to max. Size
    convention of the pages' benchmarks: the output size for AllGather(V), the per-rank
    input size for the others. Per size: `graph_launches` un-notified calls captured in
    one HIP graph, `warmup` untimed replays, then `runs` replays each bracketed by
    timing-only events; the time per call is the median replay over graph_launches.
    algbw = page-convention bytes / time (the pages' figure); hbm = the share's
    algorithmic HBM bytes (read + written) / time.
      ar   AllReduce, fused: W sources of S bytes -> W outputs       hbm 2*W*S
      a2a  AllToAll: W sources of S bytes (W tiles) -> W*S           hbm 2*W*S
      a2av AllToAllV: W sources of S // row_bytes rows (row_bytes 14,336, or 256 when
           S < 14,336), Zipf(1.1) destinations                    hbm 2*W*rows*row_bytes + 4*W*rows
      ag   AllGather: W sources of S / W bytes -> S                  hbm 2*S
      agv  AllGatherV: Zipf(s = 0.125) split of S -> S               hbm 2*S
      rs   ReduceScatter share of rank 0: W x S / W bf16 -> S / W    hbm (W+1)*S/W
      rsv  ReduceScatterV share of rank 0 (Zipf split of S)          hbm (W+1)*part_0"""
    import torch

    import reduce_atom_amd as plr
    import synth

    dev = torch.device("cuda:0")
    names = COLLECTIVES if args.collective == "all" else (args.collective,)
    E = TimingEvents(torch)
    out = {}
    for name in names:
        smax = args.max_bytes
        S_list = []
        S = args.min_bytes
        while S <= smax:
            S_list.append(S)
            S *= 2
        # buffers at the largest size; smaller sizes use their leading bytes
        if name in ("ar", "a2a", "rs", "a2av"):
            srcs = [synth.bits_t(args.seed, 11, w, smax, device=dev) if name != "rs"
                    else synth.normal_t(args.seed, 12, w, smax // 2, 1.0, device=dev).view(torch.uint8)
                    for w in range(W)]
        elif name == "ag":
            srcs = [synth.bits_t(args.seed, 13, w, smax // W, device=dev) for w in range(W)]
        elif name == "agv":
            srcs = [synth.bits_t(args.seed, 14, w, p, device=dev) for w, p in enumerate(synth.zipf_split(smax, W))]
        else:  # rsv
            srcs = [synth.normal_t(args.seed, 15, w, smax // 2, 1.0, device=dev).view(torch.uint8) for w in range(W)]
        if name == "ar":
            dsts = [torch.empty(smax, dtype=torch.uint8, device=dev) for _ in range(W)]
        elif name in ("a2a", "a2av"):
            dst = torch.empty(W * smax, dtype=torch.uint8, device=dev)
        elif name in ("ag", "agv"):
            dst = torch.empty(smax, dtype=torch.uint8, device=dev)
        else:
            dst = torch.empty(smax, dtype=torch.uint8, device=dev)
        if name == "a2av":
            zp = synth.zipf_weights(1.1, W)
            rmax = max(smax // 14336, smax // 256)
            dests = [synth.categorical_t(args.seed, 16, w, rmax, zp, device=dev) for w in range(W)]
            counts = torch.empty(W * W, dtype=torch.int64, device=dev)
            offsets = torch.empty(W * W, dtype=torch.int64, device=dev)
            scratch = torch.zeros(plr.plr_copy_v_scratch_bytes(W, [rmax] * W), dtype=torch.uint8, device=dev)
        rows_out = []
        for S in S_list:
            if name == "ar":
                L = plr.plr_layout_create("allreduce", "bf16", W, S, "scattered", "scattered")
                call = lambda: plr.plr_allreduce(L, srcs, dsts)  # noqa: E731
                page, hbm = S, 2 * W * S
            elif name == "a2a":
                L = plr.plr_layout_create("copy", "bf16", W, S, "scattered", "transposed")
                call = lambda: plr.plr_copy(L, srcs, dst)  # noqa: E731
                page, hbm = S, 2 * W * S
            elif name == "a2av":
                rb = 14336 if S >= 14336 else 256
                rows = S // rb
                call = lambda: plr.plr_copy_v(srcs, [rows] * W, dests, rb, dst, counts, offsets, scratch)  # noqa: E731
                page, hbm = rows * rb, 2 * W * rows * rb + 4 * W * rows
            elif name == "ag":
                L = plr.plr_layout_create("copy", "bf16", W, S // W, "packed", "packed")
                call = lambda: plr.plr_copy(L, srcs, dst)  # noqa: E731
                page, hbm = S, 2 * S
            elif name == "agv":
                parts = synth.zipf_split(S, W)
                L = plr.plr_layout_create("copy", "bf16", W, S, "packed", "packed", part_bytes=parts)
                call = lambda: plr.plr_copy(L, srcs, dst)  # noqa: E731
                page, hbm = S, 2 * S
            elif name == "rs":
                L = plr.plr_layout_create("reduce", "bf16", W, S, "scattered", "packed", rank=0)
                call = lambda: plr.plr_reduce(L, srcs, dst)  # noqa: E731
                page, hbm = S, (W + 1) * S // W
            else:
                parts = synth.zipf_split(S, W)
                L = plr.plr_layout_create("reduce", "bf16", W, S, "scattered", "packed", rank=0, part_bytes=parts)
                call = lambda: plr.plr_reduce(L, srcs, dst)  # noqa: E731
                page, hbm = S, (W + 1) * parts[0]
            call()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                with torch.cuda.graph(graph, stream=side):
                    for _ in range(args.graph_launches):
                        call()
            torch.cuda.current_stream().wait_stream(side)
            for _ in range(args.warmup):
                graph.replay()
            stream = torch.cuda.current_stream().cuda_stream
            evs = [(E.create(), E.create()) for _ in range(args.runs)]
            torch.cuda.synchronize()
            for a, b in evs:
                E.record(a, stream)
                graph.replay()
                E.record(b, stream)
            torch.cuda.synchronize()
            t = sorted(E.elapsed_ms(a, b) * 1e3 / args.graph_launches for a, b in evs)
            us = t[len(t) // 2]
            del graph
            rows_out.append({"bytes": S, "page_bytes": page, "us": round(us, 2),
                             "algbw_GB/s": round(page / us / 1e3, 1), "hbm_GB/s": round(hbm / us / 1e3, 1)})
        out[name] = rows_out
        print(f"collective sweep: {name} done ({len(rows_out)} sizes)", file=sys.stderr, flush=True)
        del srcs
        dst = dsts = None
        torch.cuda.empty_cache()
    E.destroy_all()
    return out


def run_atom_user_kernels(torch, srcs):
    """User kernels written on the device-callable Atom (include/plr_atom.h; built by
    build() into tests/libatom_kernels.so), timed with events around single launches:
    the reduce of the 8 prefill contributions fused with a residual add (one more
    contribution read, so 10 x 117 MB of traffic), 2 KiB per 128-thread workgroup,
    and a 512 MiB copy in 2 KiB workgroup slices (the README's device-side sample)."""
    path = os.path.join(ROOT, "tests", "libatom_kernels.so")
    if not os.path.exists(path):
        return {"atom_user_kernels": "not built"}
    lib = ctypes.CDLL(path)
    vp, sz, i, u = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint
    lib.atom_block_reduce.argtypes = [i, i, ctypes.POINTER(vp), vp, vp, sz, u, i, vp]
    lib.atom_block_copy.argtypes = [vp, vp, sz, u, i, vp]
    E = TimingEvents(torch)
    stream = torch.cuda.current_stream().cuda_stream

    def timed(fn, n=10):
        for _ in range(3):
            fn()
        evs = [(E.create(), E.create()) for _ in range(n)]
        torch.cuda.synchronize()
        for a, b in evs:
            E.record(a, stream)
            fn()
            E.record(b, stream)
        torch.cuda.synchronize()
        return statistics.mean(E.elapsed_ms(a, b) for a, b in evs) * 1e3

    out = {}
    share = R3 * C3 * 2
    res = torch.empty(R3 * C3, dtype=torch.bfloat16, device=srcs[0].device).normal_()
    dst = torch.empty_like(res)
    ptrs = (vp * W)(*[s.data_ptr() for s in srcs])
    per, nblk = 2048, share // 2048

    def red():
        rc = lib.atom_block_reduce(0, W, ptrs, res.data_ptr(), dst.data_ptr(), per, nblk, 1, stream)
        if rc:
            raise RuntimeError(f"atom_block_reduce: {rc}")

    us = timed(red)
    algo = (W + 2) * share
    out["atom_reduce_residual"] = {"avg_us": round(us, 2), "GB/s": round(algo / (us * 1e-6) / 1e9, 1),
                                   "algorithmic_bytes": algo}
    del res, dst
    n = W * B4
    a = torch.empty(n, dtype=torch.uint8, device=srcs[0].device).fill_(1)
    b = torch.empty_like(a)

    def cp():
        rc = lib.atom_block_copy(b.data_ptr(), a.data_ptr(), 2048, n // 2048, 128, stream)
        if rc:
            raise RuntimeError(f"atom_block_copy: {rc}")

    us = timed(cp)
    out["atom_block_copy"] = {"avg_us": round(us, 2), "GB/s": round(2 * n / (us * 1e-6) / 1e9, 1),
                              "algorithmic_bytes": 2 * n}
    E.destroy_all()
    return out


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo, with its family, model and stepping
    numbers (virtual machines often report a generic name)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's block is enough
                k, _, v = line.partition(":")
                fields[k.strip()] = v.strip()
    except OSError:
        pass
    name = fields.get("model name", "unknown")
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


ONLY_OPS = ("reduce", "allgather", "alltoall", "alltoallv", "reduce_lds", "allgather_lds", "allreduce_fused",
            "allreduce_cap3", "allreduce_composed")


def run_only(args):
    """One op of the step (or one row beside it) alone, --warmup + --steps calls, notified
    as in the step where it is notified there, and nothing else on the GPU: a short
    program for rocprofv3 counter passes on one kernel."""
    import torch

    import reduce_atom_amd as plr
    import synth

    dev = torch.device("cuda:0")
    op = args.only
    lds = plr.PLR_PATH_LDS if op.endswith("_lds") else 0
    if op.startswith("reduce"):
        srcs = [synth.normal_t(args.seed, 3, w, R3 * C3, 0.5, device=dev) for w in range(W)]
        dst = torch.empty(R3 * C3, dtype=torch.bfloat16, device=dev)
        L = plr.plr_layout_create("reduce", "bf16", W, R3 * C3 * 2, "packed", "packed", datapath=lds)
        ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device=dev)

        def call():
            plr.plr_notify(L, -1, ws)
            plr.plr_reduce(L, srcs, dst, ws)
    elif op.startswith("allgather") or op == "alltoall":
        srcs = [synth.bits_t(args.seed, 4, s, B4, device=dev) for s in range(W)]
        dst = torch.empty(W * B4, dtype=torch.uint8, device=dev)
        kinds = ("scattered", "transposed") if op == "alltoall" else ("packed", "packed")
        L = plr.plr_layout_create("copy", "bf16", W, B4, *kinds, datapath=lds)
        ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device=dev)

        def call():
            plr.plr_notify(L, -1, ws)
            plr.plr_copy(L, srcs, dst, ws)
    elif op == "alltoallv":
        p = synth.zipf_weights(1.1, W)
        srcs = [synth.bits_t(args.seed, 6, s, R5 * RB5, device=dev) for s in range(W)]
        dest = [synth.categorical_t(args.seed, 5, s, R5, p, device=dev) for s in range(W)]
        dst = torch.empty(W * R5 * RB5, dtype=torch.uint8, device=dev)
        counts = torch.empty(W * W, dtype=torch.int64, device=dev)
        offsets = torch.empty(W * W, dtype=torch.int64, device=dev)
        scratch = torch.zeros(plr.plr_copy_v_scratch_bytes(W, [R5] * W), dtype=torch.uint8, device=dev)
        L, ws = None, None

        def call():
            plr.plr_copy_v(srcs, [R5] * W, dest, RB5, dst, counts, offsets, scratch)
    else:
        path = plr.PLR_PATH_COMPOSED if op == "allreduce_composed" else plr.PLR_PATH_DIRECT
        srcs = [synth.normal_t(args.seed, 3, w, R3 * C3, 0.5, device=dev) for w in range(W)]
        dsts = [torch.empty(R3 * C3, dtype=torch.bfloat16, device=dev) for _ in range(W)]
        L = plr.plr_layout_create("allreduce", "bf16", W, R3 * C3 * 2, "scattered", "scattered", datapath=path,
                                  wgs_per_cu=3 if op == "allreduce_cap3" else 0)
        ws = torch.zeros(max(L.workspace_bytes, 256), dtype=torch.uint8, device=dev)

        def call():
            plr.plr_allreduce(L, srcs, dsts, ws)
    for _ in range(args.warmup + args.steps):
        call()
    torch.cuda.synchronize()
    if ws is not None and plr.plr_check(L, ws) != plr.PLR_OK:
        raise RuntimeError(f"{op}: device error")
    print(json.dumps({"only": op, "calls": args.warmup + args.steps}), flush=True)


def run_cpu_baseline(args, host):
    """The oracle, as it stands, on this host's CPU, on the same input bytes as the GPU
    step: on all the cores this process may use (the oracle's threaded form, at most 16
    threads) over the whole step, and single-threaded over a fraction of every op
    (--cpu-fraction) to bound the run time; median of --cpu-reps runs after one warmup
    run each. GB/s from the same algorithmic byte counts as the GPU figures."""
    import oracle
    import synth

    f = args.cpu_fraction
    rr = max(1, int(R3 * f))
    bb = max(16 * W, int(B4 * f) // (16 * W) * (16 * W))
    rv = max(1, int(R5 * f))
    full_bytes = sum(BYTES.values())
    part_bytes = (W + 1) * rr * C3 * 2 + 2 * (2 * W * bb) + 2 * W * rv * RB5 + W * rv * 4
    red_part = [a[: rr * C3] for a in host["r_src"]]
    cps_part = [a[:bb] for a in host["c_src"]]
    vs_part = [a[: rv * RB5] for a in host["v_src"]]
    vd_part = [a[:rv] for a in host["v_dest"]]

    op_times = {}  # (threads, op) -> seconds of each timed run

    def step(threads, red, cps, vs, vd, record=False):
        for name, fn in (("reduce", lambda: oracle.reduce("bf16", red, threads=threads)),
                         ("allgather", lambda: oracle.copy_layout("packed", "packed", cps, threads=threads)),
                         ("alltoall", lambda: oracle.copy_layout("scattered", "transposed", cps, threads=threads)),
                         ("alltoallv", lambda: oracle.copy_v(vs, vd, RB5, threads=threads))):
            t = time.perf_counter()
            fn()
            if record:
                op_times.setdefault((threads, name), []).append(time.perf_counter() - t)

    def timed(fn):
        fn(False)  # warmup
        times = []
        for _ in range(args.cpu_reps):
            t = time.perf_counter()
            fn(True)
            times.append(time.perf_counter() - t)
        return statistics.median(times)

    cores = oracle.default_threads()
    t_all = timed(lambda rec: step(cores, host["r_src"], host["c_src"], host["v_src"], host["v_dest"], rec))
    t_one = timed(lambda rec: step(1, red_part, cps_part, vs_part, vd_part, rec))
    part = {"reduce": (W + 1) * rr * C3 * 2, "allgather": 2 * W * bb, "alltoall": 2 * W * bb,
            "alltoallv": 2 * W * rv * RB5 + W * rv * 4}
    per_op = {n: {"GB/s_all_cores": round(BYTES[n] / statistics.median(op_times[(cores, n)]) / 1e9, 4),
                  "GB/s_one_core": round(part[n] / statistics.median(op_times[(1, n)]) / 1e9, 4)}
              for n in BYTES}
    # the two configs outside the step: the local reduce (8 x 1,048,576 bf16) and the
    # largest decode share (8 x [64, 7168] bf16), median of --cpu-reps calls each
    for name, srcs in (("local_reduce_8x1M", [synth.uniform_pm1_np(args.seed, 1, w, 1 << 20) for w in range(W)]),
                       ("decode_T64", [synth.normal_np(args.seed, 2, w, 64 * 7168, 1.0) for w in range(W)])):
        nbytes = (W + 1) * srcs[0].nbytes
        row = {}
        for tag, th in (("all_cores", cores), ("one_core", 1)):
            oracle.reduce("bf16", srcs, threads=th)
            ts = []
            for _ in range(args.cpu_reps):
                t = time.perf_counter()
                oracle.reduce("bf16", srcs, threads=th)
                ts.append(time.perf_counter() - t)
            tm = statistics.median(ts)
            row[f"GB/s_{tag}"] = round(nbytes / tm / 1e9, 4)
            row[f"us_{tag}"] = round(tm * 1e6, 1)
        per_op[name] = row
    one = {"value": round(part_bytes / t_one / 1e9, 4), "unit": "GB/s", "cores": 1,
           "sample": (f"fraction {f} of every op of the step (reduce {rr} of {R3} rows, allgather/alltoall "
                      f"{bb} of {B4} bytes per source, alltoallv {rv} of {R5} rows per source); median of "
                      f"{args.cpu_reps} runs of {t_one:.2f} s after one warmup run"),
           "seconds": round(t_one, 3)}
    return {"value": round(full_bytes / t_all / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": (f"the whole step (all four ops, the GPU step's own input bytes) on {cores} threads; "
                       f"median of {args.cpu_reps} runs of {t_all:.2f} s after one warmup run"),
            "seconds": round(t_all, 3), "single_core": one, "per_op": per_op,
            "host": {"cpu_model": cpu_model(), "hardware_threads": oracle.hardware_threads(),
                     "threads_available": len(os.sched_getaffinity(0))}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--decode-iters", type=int, default=1000)
    ap.add_argument("--decode-warmup", type=int, default=100)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode-size latency runs (for profiling them), printed as JSON")
    ap.add_argument("--decode-t", type=lambda v: [int(x) for x in v.split(",")], default=None,
                    help="decode token counts T (comma separated; default 1,8,32,64)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-trace", action="store_true",
                    help="skip the kernel-trace run of the decode-size reduce (rocprofv3 child process)")
    ap.add_argument("--decode-trace-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--only", choices=ONLY_OPS,
                    help="run one op alone (--warmup + --steps calls, no timing), for counter passes")
    ap.add_argument("--v-sweep", action="store_true",
                    help="only the AllGatherV / ReduceScatterV sweep over T = 1 KiB .. 1 GiB, as JSON")
    ap.add_argument("--collective", choices=COLLECTIVES + ("all",),
                    help="only the per-collective size sweep (the pages' testAR ... testRSV), as JSON")
    ap.add_argument("--min-bytes", type=int, default=1 << 10)
    ap.add_argument("--max-bytes", type=int, default=1 << 30)
    ap.add_argument("--graph-launches", type=int, default=10)
    ap.add_argument("--runs", type=int, default=20)
    ap.add_argument("--cpu-fraction", type=float, default=0.25,
                    help="fraction of every op the single-threaded oracle baseline runs on")
    ap.add_argument("--cpu-reps", type=int, default=5)
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="print per-kernel durations of a rocprofv3 kernel-trace CSV and exit")
    ap.add_argument("--summarize-sweep", metavar="JSON",
                    help="print the tables of a --collective / --v-sweep JSON output and exit")
    ap.add_argument("--summarize-decode", metavar="JSON",
                    help="print the decode latency table of a bench JSON line and exit")
    ap.add_argument("--summarize-counters", metavar="CSV",
                    help="print per-kernel mean counters of a rocprofv3 counter CSV and exit")
    ap.add_argument("--counters-profile", metavar="DIR",
                    help="directory of the traffic counter passes (TRAFFIC_PASSES): write "
                         "profiles/<op>_counters.txt and exit")
    ap.add_argument("--bound-profile", metavar="DIR",
                    help="directory of the bound counter passes (BOUND_PASSES): write "
                         "profiles/bounds_counters.txt and exit")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run torch's plain device copy of 1 GiB five times (the reference "
                         "for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0 or args.runs < 1 or args.graph_launches < 1:
        sys.exit("--steps, --runs and --graph-launches must be at least 1, --warmup at least 0")
    if args.gpus != 1:
        sys.exit(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this datapath holds the W "
                 "contributions of one GPU's share in that GPU's memory and uses no second GPU.")

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.counters_profile:
        write_counter_profiles(args.counters_profile, os.path.join(ROOT, "profiles"))
        return
    if args.bound_profile:
        write_bound_profile(args.bound_profile, os.path.join(ROOT, "profiles", "bounds_counters.txt"))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return
    if args.summarize_sweep:
        print(summarize_sweep(args.summarize_sweep))
        return
    if args.summarize_decode:
        print(summarize_decode(args.summarize_decode))
        return
    if args.calibrate:
        import torch

        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate": "torch copy_", "bytes_read": 1 << 30, "bytes_written": 1 << 30,
                          "launches": 5}), flush=True)
        return
    if args.v_sweep:
        print(json.dumps({"v_sweep": run_v_sweep(args)}), flush=True)
        return
    if args.collective:
        lo, hi = args.min_bytes, args.max_bytes
        if lo < 16 * W * 8 or lo & (lo - 1) or hi < lo or hi & (hi - 1):
            sys.exit("--min-bytes and --max-bytes must be powers of two, at least 1024")
        print(json.dumps({"collective_sweep": run_collective_sweep(args), "graph_launches": args.graph_launches,
                          "runs": args.runs, "warmup": args.warmup, "seed": args.seed}), flush=True)
        return
    if args.decode_trace_child:
        run_decode_trace_child(args)
        return
    if args.only:
        run_only(args)
        return
    # before this process touches the GPU: the decode kernel trace runs in a child
    trace = None if (args.no_decode or args.no_decode_trace) else run_decode_trace(args)
    if args.decode_only:
        import torch

        import reduce_atom_amd as plr
        import synth

        dec = run_decode(args, torch, plr, synth, torch.device("cuda:0"))
        print(json.dumps({"decode_reduce_us": {"kernel_trace": trace, **dec}}), flush=True)
        return
    value, ms, ms_events, roofline, per_op, small, host = run_bench(args)
    decode = small["decode"] if small else None
    local = small["local"] if small else None
    producer = small["producer"] if small else None
    nxt = None if args.no_decode else run_next(args)
    cpu = None if host is None else run_cpu_baseline(args, host)
    del host
    if trace is not None and LOCAL_KEY in trace:
        lt = trace.pop(LOCAL_KEY)["notify_off"]
        for temp in lt:
            lt[temp]["GB/s_at_p50"] = round(9 * 2 * (1 << 20) / (lt[temp]["p50_us"] * 1e-6) / 1e9, 1)
        local = {"kernel_trace": lt, **(local or {})}
    if decode is not None and trace is not None:
        decode = {"kernel_trace": trace, **decode}
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "notified datapath step, W=8: reduce 8x[8192,7168] bf16 N(0,0.5); "
                               "allgather 8x64MiB; alltoall 8x(8x8MiB); alltoallv 8x4096 rows x "
                               "7168 bf16, Zipf(1.1) destinations",
                   "world": W, "notify": True, "seed": args.seed, "step_bytes": sum(BYTES.values())},
        "roofline": roofline, "cpu_baseline": cpu, "per_op": per_op,
        "ms_per_step_with_op_events": round(ms_events, 4), "decode_reduce_us": decode,
        "local_reduce_8x1M_bf16": local, "decode_producer_kernel_us": producer,
        "beyond_step": nxt,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
