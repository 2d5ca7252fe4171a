"""The oracle's latency-path packet encoding, pinned to hand-built packets and to the
round-trip and stamp invariants."""
import numpy as np

import synth
from conftest import golden_lines


def test_golden_packets(oracle_mod):
    for line in golden_lines("packets_small.txt"):
        lhs, rhs = line.split("->")
        epoch, *words = lhs.split()
        data = np.array([int(w, 16) for w in words], dtype=np.uint32)
        want = np.array([int(p, 16) for p in rhs.split()], dtype=np.uint64)
        assert np.array_equal(oracle_mod.pack(data, int(epoch)), want), line


def test_round_trip_and_stamp(oracle_mod):
    data = synth.bits_np(0, 9, 0, 4096)
    p = oracle_mod.pack(data, 12345)
    assert p.nbytes == 2 * data.nbytes  # the doubled volume
    back, ok = oracle_mod.unpack(p, 12345)
    assert ok.all() and np.array_equal(back, data)
    _, ok2 = oracle_mod.unpack(p, 12346)
    assert not ok2.any()
