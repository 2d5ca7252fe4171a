"""The oracle's variable-length AllToAll packing, pinned to a hand-worked example,
numpy's histogram / cumulative sum / stable sort, and special cases."""
import numpy as np
import pytest

import synth
from conftest import golden_lines


def _tagged_rows(W, rows, row_bytes):
    """Rows whose first 8 bytes encode (source, row index); the rest is random bits."""
    out = []
    for s in range(W):
        r = synth.bits_np(0, 5, 100 + s, rows[s] * row_bytes).reshape(rows[s], row_bytes).copy()
        tag = (np.uint64(s) << np.uint64(32)) | np.arange(rows[s], dtype=np.uint64)
        r[:, :8] = tag.view(np.uint8).reshape(rows[s], 8)
        out.append(r)
    return out


def _tags(out, row_bytes):
    t = out.reshape(-1, row_bytes)[:, :8].copy().view(np.uint64).reshape(-1)
    return [(int(x >> np.uint64(32)), int(x & np.uint64(0xFFFFFFFF))) for x in t]


def test_golden_small(oracle_mod):
    lines = list(golden_lines("copy_v_small.txt"))
    W = int(lines[0].split()[1])
    dests = [np.array([int(v) for v in l.split()[2:]], np.int32) for l in lines[1:1 + W]]
    counts = np.array([int(v) for v in lines[1 + W].split()[1:]]).reshape(W, W)
    offsets = np.array([int(v) for v in lines[2 + W].split()[1:]]).reshape(W, W)
    order = [tuple(int(v) for v in t.split(":")) for t in lines[3 + W].split()[1:]]
    rows = _tagged_rows(W, [d.size for d in dests], 16)
    out, c, o = oracle_mod.copy_v(rows, dests, 16)
    assert np.array_equal(c, counts) and np.array_equal(o, offsets)
    assert _tags(out, 16) == order


@pytest.mark.parametrize("W,rows_each,seed", [(2, 7, 0), (3, 50, 1), (8, 300, 2), (5, 1, 3)])
def test_against_numpy_stable_sort(oracle_mod, W, rows_each, seed):
    rb = 32
    rows = [rows_each + (s * 3) % 5 for s in range(W)]
    p = synth.zipf_weights(1.1, W)
    dests = [synth.categorical_np(seed, 5, s, rows[s], p) for s in range(W)]
    srcs = _tagged_rows(W, rows, rb)
    out, counts, offsets = oracle_mod.copy_v(srcs, dests, rb)
    # counts: histogram per source
    assert np.array_equal(counts, np.stack([np.bincount(d, minlength=W) for d in dests]))
    # offsets: exclusive scan in (destination, source) order
    flat = counts.T.reshape(-1)
    excl = np.concatenate([[0], np.cumsum(flat)[:-1]]).reshape(W, W)
    assert np.array_equal(offsets, excl)
    # rows: all rows in (source, row) order, stably sorted by destination
    allrows = np.concatenate(srcs)
    alld = np.concatenate(dests)
    ref = allrows[np.argsort(alld, kind="stable")].reshape(-1)
    assert np.array_equal(out, ref)
    assert counts.sum() == sum(rows)


def test_all_to_destination_zero_is_concatenation(oracle_mod):
    W = 4
    srcs = _tagged_rows(W, [10] * W, 48)
    out, counts, _ = oracle_mod.copy_v(srcs, [np.zeros(10, np.int32)] * W, 48)
    assert np.array_equal(out, np.concatenate(srcs).reshape(-1))
    assert (counts[:, 0] == 10).all() and (counts[:, 1:] == 0).all()


def test_round_robin_destinations_balance(oracle_mod):
    W, R = 8, 4096
    srcs = _tagged_rows(W, [R] * W, 16)
    dests = [(np.arange(R) % W).astype(np.int32)] * W
    _, counts, _ = oracle_mod.copy_v(srcs, dests, 16)
    assert (counts == R // W).all()


def test_single_source_identity(oracle_mod):
    srcs = _tagged_rows(1, [33], 64)
    out, counts, offsets = oracle_mod.copy_v(srcs, [np.zeros(33, np.int32)], 64)
    assert np.array_equal(out, srcs[0].reshape(-1)) and counts[0, 0] == 33 and offsets[0, 0] == 0


def test_empty_sources(oracle_mod):
    srcs = _tagged_rows(3, [0, 4, 0], 16)
    dests = [np.zeros(0, np.int32), np.array([2, 0, 2, 1], np.int32), np.zeros(0, np.int32)]
    out, counts, offsets = oracle_mod.copy_v(srcs, dests, 16)
    assert _tags(out, 16) == [(1, 1), (1, 3), (1, 0), (1, 2)]
    assert counts.sum() == 4


def test_bad_destination_rejected(oracle_mod):
    srcs = _tagged_rows(2, [2, 2], 16)
    with pytest.raises(ValueError):
        oracle_mod.copy_v(srcs, [np.array([0, 2], np.int32), np.array([0, 1], np.int32)], 16)
