"""Pins of the oracle's variable-length collectives (AllGatherV, ReduceScatterV) and of
the benchmark's Zipf partition (Purlin paper, appendix C.4)."""
import numpy as np
import pytest

import oracle
import synth
from conftest import golden_lines


def test_zipf_split_golden():
    for line in golden_lines("zipf_split.txt"):
        head, sizes = line.split(":")
        total, n, s = head.split()
        got = synth.zipf_split(int(total), int(n), float(s))
        assert got == [int(v) for v in sizes.split()], line


@pytest.mark.parametrize("total", [1024, 2048, 4096, 8192, 65536, 1 << 20, 37 * 1024, 1 << 30])
def test_zipf_split_properties(total):
    parts = synth.zipf_split(total)
    assert sum(parts) == total  # splits preserve the total
    assert all(p % 16 == 0 and p > 0 for p in parts)
    assert all(parts[r] >= parts[r + 1] for r in range(7))
    if total >= 4096:
        # within one granule per rank of the real-valued Zipf share
        w = synth.zipf_weights(0.125, 8)
        assert all(abs(parts[r] - total * w[r]) < 2 * 16 for r in range(8))
    else:
        assert len(set(parts)) == 1


def test_part_offsets_is_exclusive_scan():
    assert oracle.part_offsets([]) == []
    assert oracle.part_offsets([5]) == [0]
    assert oracle.part_offsets([16, 0, 32, 48]) == [0, 16, 16, 48]
    p = synth.zipf_split(1 << 20)
    assert oracle.part_offsets(p) == list(np.concatenate([[0], np.cumsum(p)[:-1]]))


def test_allgather_v_is_concatenation():
    parts = [48, 0, 16, 160, 32]
    srcs = [synth.bits_np(3, 9, w, max(p, 16)) for w, p in enumerate(parts)]
    got = oracle.allgather_v(srcs, parts)
    ref = np.concatenate([s[:p] for s, p in zip(srcs, parts)])
    assert got.dtype == np.uint8 and np.array_equal(got, ref)
    # one rank: the identity on its contribution
    assert np.array_equal(oracle.allgather_v([srcs[3]], [160]), srcs[3][:160])
    # equal sizes: the fixed-length AllGather of the same bytes
    eq = [synth.bits_np(4, 9, w, 64) for w in range(4)]
    assert np.array_equal(oracle.allgather_v(eq, [64] * 4), oracle.copy_layout("packed", "packed", eq))


def test_reduce_scatter_v_worked_example():
    """W = 3 sources of 48 bf16 elements, element i of source w = (w+1)(i+1) (small
    integers, exact in bf16); partitions of 32, 16 and 48 bytes = 16, 8 and 24 elements.
    Rank 1's share is elements 16..23 of every source: (1+2+3)(i+1) = 6(i+1) for
    i = 16..23, i.e. 102, 108, ..., 144; rank 2's is 6(i+1) for i = 24..47 (even numbers
    up to 288, exact in bf16, whose spacing is 2 between 256 and 512)."""
    W, n = 3, 48
    vals = [np.array([(w + 1) * (i + 1) for i in range(n)], np.float32) for w in range(W)]
    srcs = [oracle.narrow("bf16", v) for v in vals]
    parts = [32, 16, 48]
    r1 = oracle.widen("bf16", oracle.reduce_scatter_v("bf16", srcs, parts, 1))
    assert list(r1) == [102, 108, 114, 120, 126, 132, 138, 144]
    r2 = oracle.widen("bf16", oracle.reduce_scatter_v("bf16", srcs, parts, 2))
    assert list(r2) == [6 * (i + 1) for i in range(24, 48)]
    r0 = oracle.widen("bf16", oracle.reduce_scatter_v("bf16", srcs, parts, 0))
    assert list(r0) == [6 * (i + 1) for i in range(16)]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_reduce_scatter_v_shares_tile_the_full_reduce(dtype):
    """The W shares, in rank order, are the reduction of the whole contributions (the
    reduction is elementwise, so cutting it by partition changes nothing), whatever
    the partition, empty partitions included."""
    W, total = 5, 2048
    eb = oracle.ELEM_BYTES[dtype]
    srcs = [synth.normal_np(5, 9, w, total // eb, dtype=dtype) for w in range(W)]
    full = oracle.reduce(dtype, srcs)
    for parts in ([total // W // 16 * 16] * (W - 1) + [total - (W - 1) * (total // W // 16 * 16)],
                  [0, 1024, 0, 512, 512], [2048, 0, 0, 0, 0]):
        got = np.concatenate([oracle.reduce_scatter_v(dtype, srcs, parts, r) for r in range(W)])
        assert np.array_equal(got.view(np.uint8), full.view(np.uint8)), parts
        for r in range(W):
            assert oracle.reduce_scatter_v(dtype, srcs, parts, r).nbytes == parts[r]
