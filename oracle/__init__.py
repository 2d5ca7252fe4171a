"""The oracle: a plain, slow, obviously correct CPU implementation of the datapath.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The library in
``reduce_atom_amd/`` never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, one element at a time; threaded
variants split the same per-element code over host threads, for comparing full-size
outputs in seconds and for timing the oracle on every core). This module
marshals numpy arrays into it and holds the oracle's own reading of the layouts
(Purlin paper, section 3.1 "Layouts": a collective is a naming of an input and an
output layout plus a copy or a reduction; the layout kinds are packed, scattered
and transposed). The readings used here:

- packed: a rank's region is one contiguous block of ``bytes_per_src`` bytes;
- scattered: a rank's region is W equal slices, slice j belonging to rank j;
- transposed: a W x W grid of slices in which output slice (d, s) is input
  slice (s, d).

Reduce shares: a packed contribution is reduced whole (offset 0 in every source);
a scattered contribution gives rank ``r`` its slice ``r`` of every source.
Copies: packed -> packed is AllGather (source s lands at s * bytes_per_src);
scattered -> transposed is AllToAll; scattered -> scattered is the gather half of
a composed AllReduce (slice s of source s lands at slice s of the output).

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
things other than itself (library conversions, closed forms, hand-derived
vectors under ``tests/golden/``, brute force, invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PLR_ORACLE_LIB names another build of oracle.c to load instead: the mutation tests plant
# a mistake in a copy of the source and check that the pins fail against that copy's build
_SO = os.environ.get("PLR_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

DTYPES = {"bf16": 0, "f16": 1, "f32": 2}
ELEM_BYTES = {"bf16": 2, "f16": 2, "f32": 4}
PACKED, SCATTERED, TRANSPOSED = "packed", "scattered", "transposed"

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
          "-Wall", "-Wextra", "-Werror"]


def build(out: str = _SO, src: str = _SRC) -> str:
    """Compile oracle.c (or another copy of it) with gcc (plain scalar C, no contraction,
    no fast math)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_widen.argtypes = [i32, vp, vp, i64]
        L.oracle_narrow.argtypes = [i32, vp, vp, i64]
        L.oracle_add_f32.argtypes = [ctypes.c_float, ctypes.c_float]
        L.oracle_add_f32.restype = ctypes.c_float
        L.oracle_reduce.argtypes = [i32, i32, vp, vp, vp, i64]
        L.oracle_reduce.restype = i32
        L.oracle_copy.argtypes = [i32, vp, vp, vp, vp, vp, vp]
        L.oracle_copy.restype = i32
        L.oracle_copy_v.argtypes = [i32, vp, vp, vp, i64, vp, vp, vp]
        L.oracle_copy_v.restype = i64
        L.oracle_reduce_mt.argtypes = [i32, i32, vp, vp, vp, i64, i32]
        L.oracle_reduce_mt.restype = i32
        L.oracle_copy_mt.argtypes = [i32, vp, vp, vp, vp, vp, vp, i32]
        L.oracle_copy_mt.restype = i32
        L.oracle_copy_v_mt.argtypes = [i32, vp, vp, vp, i64, vp, vp, vp, i32]
        L.oracle_copy_v_mt.restype = i64
        L.oracle_hardware_threads.argtypes = []
        L.oracle_hardware_threads.restype = i32
        _lib = L
    return _lib


def hardware_threads() -> int:
    """Logical CPUs online on this host (sysconf, as std::thread::hardware_concurrency)."""
    return lib().oracle_hardware_threads()


def default_threads() -> int:
    """Threads the threaded variants use by default: the CPUs this process may run on,
    at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _ptr_array(arrs):
    return (ctypes.c_void_p * len(arrs))(*[_ptr(a) for a in arrs])


def _raw(a, dtype):
    """View element data as the raw storage type the C code reads."""
    a = np.ascontiguousarray(a)
    if dtype == "f32":
        return a.view(np.float32)
    return a.view(np.uint16)


# ------------------------------------------------------------------ formats
def widen(dtype: str, bits: np.ndarray) -> np.ndarray:
    """Element bits (uint16 for bf16/f16, float32 for f32) -> exact float32 values."""
    src = _raw(bits, dtype)
    out = np.empty(src.size, dtype=np.float32)
    lib().oracle_widen(DTYPES[dtype], _ptr(src), _ptr(out), src.size)
    return out.reshape(src.shape)


def narrow(dtype: str, x: np.ndarray) -> np.ndarray:
    """float32 values -> element bits, round to nearest, ties to even."""
    src = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(src.size, dtype=np.float32 if dtype == "f32" else np.uint16)
    lib().oracle_narrow(DTYPES[dtype], _ptr(src), _ptr(out), src.size)
    return out.reshape(src.shape)


def add_f32(a: float, b: float) -> float:
    return lib().oracle_add_f32(a, b)


# ------------------------------------------------------------------ layouts
def reduce_share(in_kind: str, world: int, rank: int, elems_per_src: int):
    """(element offset of the share in every source, share length in elements)."""
    if in_kind == PACKED:
        return [0] * world, elems_per_src
    if in_kind == SCATTERED:
        if elems_per_src % world:
            raise ValueError("scattered contribution not divisible by W")
        n = elems_per_src // world
        return [rank * n] * world, n
    raise ValueError(in_kind)


def copy_segments(in_kind: str, out_kind: str, world: int, bytes_per_src: int):
    """Segments (src, src_off, dst_off, len) in bytes, and the output size."""
    W, B = world, bytes_per_src
    if in_kind == PACKED and out_kind == PACKED:  # AllGather: concatenation by rank
        return [(s, 0, s * B, B) for s in range(W)], W * B
    if B % W:
        raise ValueError("scattered contribution not divisible by W")
    t = B // W
    if in_kind == SCATTERED and out_kind == TRANSPOSED:  # AllToAll
        segs = []
        for s in range(W):
            for d in range(W):
                segs.append((s, d * t, (d * W + s) * t, t))
        return segs, W * W * t
    if in_kind == SCATTERED and out_kind == SCATTERED:  # gather half of AllReduce
        return [(s, s * t, s * t, t) for s in range(W)], W * t
    raise ValueError((in_kind, out_kind))


# ------------------------------------------------------------------ reduce
def reduce(dtype: str, srcs, src_off=None, n=None, threads: int = 1) -> np.ndarray:
    """Rank-order fp32 reduction of W sources into one share (element bits out).
    threads > 1 splits the elements over that many host threads (same results)."""
    raws = [_raw(s, dtype).reshape(-1) for s in srcs]
    W = len(raws)
    if src_off is None:
        src_off = [0] * W
    if n is None:
        n = raws[0].size
    for w in range(W):
        if src_off[w] < 0 or src_off[w] + n > raws[w].size:
            raise ValueError("share out of bounds")
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    offs = np.asarray(src_off, dtype=np.int64)
    if threads > 1:
        rc = lib().oracle_reduce_mt(DTYPES[dtype], W, _ptr_array(raws), _ptr(offs), _ptr(out), n, threads)
    else:
        rc = lib().oracle_reduce(DTYPES[dtype], W, _ptr_array(raws), _ptr(offs), _ptr(out), n)
    if rc:
        raise ValueError("oracle_reduce rejected its arguments")
    return out


def reduce_layout(dtype: str, in_kind: str, rank: int, srcs, threads: int = 1) -> np.ndarray:
    W = len(srcs)
    offs, n = reduce_share(in_kind, W, rank, _raw(srcs[0], dtype).size)
    return reduce(dtype, srcs, offs, n, threads)


def allreduce(dtype: str, srcs, threads: int = 1):
    """AllReduce of W contributions (Purlin paper, section 2.1: every rank ends with the
    reduction of all contributions): W outputs, each the rank-order reduction of the
    W sources. Written from that definition; the composition ReduceScatter then
    AllGather (section 3.1) is checked against it in the tests."""
    out = reduce(dtype, srcs, threads=threads)
    return [out.copy() for _ in srcs]


def pack(data: np.ndarray, epoch: int) -> np.ndarray:
    """Latency-path packets (Purlin paper, section 3.2 and Figure 7: payload and
    notification combined in one atomic packet, doubling the data volume). Reading:
    an 8-byte packet per 4-byte payload word, the word in the low half and the low 32
    bits of the epoch in the high half (little-endian), so that one 8-byte atomic
    carries both. Returns uint64 packets."""
    words = np.ascontiguousarray(data).reshape(-1).view(np.uint32).astype(np.uint64)
    return words | (np.uint64(epoch & 0xFFFFFFFF) << np.uint64(32))


def unpack(packets: np.ndarray, epoch: int):
    """(payload bytes, mask of packets whose stamp equals the epoch)."""
    p = np.ascontiguousarray(packets).view(np.uint64)
    ok = (p >> np.uint64(32)) == np.uint64(epoch & 0xFFFFFFFF)
    return (p & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.uint8), ok


# ------------------------------------------------------------------ copy
def copy(srcs, segments, dst_bytes: int, fill: int = 0, threads: int = 1) -> np.ndarray:
    """Apply byte segments (src, src_off, dst_off, len) to a fresh output buffer.
    threads > 1 splits every segment over that many host threads (same bytes)."""
    raws = [np.ascontiguousarray(s).reshape(-1).view(np.uint8) for s in srcs]
    out = np.full(dst_bytes, fill, dtype=np.uint8)
    for (s, so, do, ln) in segments:
        if so + ln > raws[s].size or do + ln > dst_bytes:
            raise ValueError("segment out of bounds")
    k = len(segments)
    seg_src = np.array([g[0] for g in segments], dtype=np.int32)
    so = np.array([g[1] for g in segments], dtype=np.int64)
    do = np.array([g[2] for g in segments], dtype=np.int64)
    ln = np.array([g[3] for g in segments], dtype=np.int64)
    if threads > 1:
        lib().oracle_copy_mt(k, _ptr_array(raws), _ptr(seg_src), _ptr(so), _ptr(do), _ptr(ln), _ptr(out),
                             threads)
    else:
        lib().oracle_copy(k, _ptr_array(raws), _ptr(seg_src), _ptr(so), _ptr(do), _ptr(ln), _ptr(out))
    return out


def copy_layout(in_kind: str, out_kind: str, srcs, threads: int = 1) -> np.ndarray:
    B = np.ascontiguousarray(srcs[0]).nbytes
    segs, total = copy_segments(in_kind, out_kind, len(srcs), B)
    return copy(srcs, segs, total, threads=threads)


# ------------------------------------------------------------------ variable length
def part_offsets(parts):
    """Byte offset of every partition: the exclusive prefix sum of the sizes (appendix
    C.4 and section 4: partition sizes are given at run time, offsets are prefix sums)."""
    offs, run = [], 0
    for p in parts:
        offs.append(run)
        run += int(p)
    return offs


def allgather_v(srcs, parts, threads: int = 1) -> np.ndarray:
    """AllGatherV (section 2.1 and appendix C.4: a contribution of its own size per
    rank; every rank receives all of them in rank order): source w contributes its
    first parts[w] bytes, placed at the sum of the sizes before it."""
    offs = part_offsets(parts)
    segs = [(w, 0, offs[w], int(parts[w])) for w in range(len(srcs))]
    return copy(srcs, segs, sum(int(p) for p in parts), threads=threads)


def reduce_scatter_v(dtype: str, srcs, parts, rank: int, threads: int = 1) -> np.ndarray:
    """ReduceScatterV share of `rank` (appendix C.4: the rank's assigned partition is
    its output): every source holds all partitions back to back; the share is the
    rank-order reduction of partition `rank` of every source."""
    eb = ELEM_BYTES[dtype]
    off = part_offsets(parts)[rank]
    if off % eb or int(parts[rank]) % eb:
        raise ValueError("partition not a whole number of elements")
    W = len(srcs)
    return reduce(dtype, srcs, [off // eb] * W, int(parts[rank]) // eb, threads)


# ------------------------------------------------------------------ copy_v
def copy_v(srcs, dests, row_bytes: int, threads: int = 1):
    """Variable-length AllToAll packing. srcs[s]: rows of source s (any dtype, C order);
    dests[s]: int32 destination per row. Returns (out bytes, counts[s][d], offsets[d][s]).
    threads > 1 moves the rows on that many host threads (same bytes)."""
    W = len(srcs)
    raws = [np.ascontiguousarray(s).reshape(-1).view(np.uint8) for s in srcs]
    ds = [np.ascontiguousarray(d, dtype=np.int32).reshape(-1) for d in dests]
    rows = np.array([d.size for d in ds], dtype=np.int64)
    for s in range(W):
        if raws[s].size < rows[s] * row_bytes:
            raise ValueError("source smaller than its rows")
    total = int(rows.sum())
    out = np.zeros(total * row_bytes, dtype=np.uint8)
    counts = np.zeros((W, W), dtype=np.int64)
    offsets = np.zeros((W, W), dtype=np.int64)
    if threads > 1:
        got = lib().oracle_copy_v_mt(W, _ptr_array(raws), _ptr(rows), _ptr_array(ds), row_bytes,
                                     _ptr(out), _ptr(counts), _ptr(offsets), threads)
    else:
        got = lib().oracle_copy_v(W, _ptr_array(raws), _ptr(rows), _ptr_array(ds), row_bytes,
                                  _ptr(out), _ptr(counts), _ptr(offsets))
    if got < 0:
        raise ValueError("destination out of range")
    assert got == total
    return out, counts, offsets
