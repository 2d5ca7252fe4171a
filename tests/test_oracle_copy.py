"""The oracle's layout copies, pinned to hand-derived segments and to numpy
concatenation / transposition; random-bit payloads carry NaN/inf/subnormal patterns,
so any float path in a copy would show."""
import numpy as np
import pytest

import synth
from conftest import golden_lines


def test_golden_segments(oracle_mod):
    for line in golden_lines("layout_segments.txt"):
        ik, ok, *segs = line.split()
        want = [tuple(int(v) for v in s.split(":")) for s in segs]
        got, _ = oracle_mod.copy_segments(ik, ok, 2, 32)
        assert sorted(got) == sorted(want), line


def _srcs(W, B, seed=0):
    return [synth.bits_np(seed, 4, s, B) for s in range(W)]


@pytest.mark.parametrize("W", [1, 2, 3, 8])
def test_allgather_is_concatenation(oracle_mod, W):
    srcs = _srcs(W, 256)
    assert np.array_equal(oracle_mod.copy_layout("packed", "packed", srcs), np.concatenate(srcs))


@pytest.mark.parametrize("W", [1, 2, 4, 8])
def test_alltoall_is_transpose(oracle_mod, W):
    t = 48
    srcs = _srcs(W, W * t, seed=1)
    out = oracle_mod.copy_layout("scattered", "transposed", srcs)
    grid = np.stack(srcs).reshape(W, W, t)          # [src][dst][t]
    assert np.array_equal(out, grid.transpose(1, 0, 2).reshape(-1))
    # involution: applying it to the output blocks again gives the input back
    back = oracle_mod.copy_layout("scattered", "transposed", list(out.reshape(W, W * t)))
    assert np.array_equal(back, np.concatenate(srcs))


@pytest.mark.parametrize("W", [1, 2, 5, 8])
def test_allreduce_gather_half(oracle_mod, W):
    t = 32
    srcs = _srcs(W, W * t, seed=2)
    out = oracle_mod.copy_layout("scattered", "scattered", srcs)
    assert np.array_equal(out, np.concatenate([srcs[s][s * t:(s + 1) * t] for s in range(W)]))


def test_copy_preserves_nan_payloads(oracle_mod):
    specials = np.array([0x7F800001, 0xFFC01234, 0x7FBFFFFF, 0x00000001, 0x80000000],
                        dtype=np.uint32).view(np.uint8)
    srcs = [np.tile(specials, 4), np.tile(specials[::-1].copy(), 4)]
    out = oracle_mod.copy_layout("packed", "packed", srcs)
    assert out.tobytes() == srcs[0].tobytes() + srcs[1].tobytes()


def test_segment_bounds_checked(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.copy([np.zeros(16, np.uint8)], [(0, 0, 0, 32)], 32)
