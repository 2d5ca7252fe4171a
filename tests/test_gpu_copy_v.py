"""Parity of plr_copy_v (HIP, through the C ABI) with the oracle: output rows, counts
and offsets bitwise."""
import numpy as np
import pytest
import torch

import synth
from conftest import golden_lines
from plrtest import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def plr():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import reduce_atom_amd

    return reduce_atom_amd


def _run(plr, srcs_np, dests_np, row_bytes):
    W = len(srcs_np)
    rows = [int(d.size) for d in dests_np]
    srcs = [to_dev(s) for s in srcs_np]
    dests = [torch.from_numpy(np.ascontiguousarray(d, dtype=np.int32).copy()).cuda()
             if d.size else torch.zeros(4, dtype=torch.int32, device="cuda") for d in dests_np]
    total = sum(rows)
    dst = torch.full((max(total * row_bytes, 16),), 0x77, dtype=torch.uint8, device="cuda")
    counts = torch.full((W * W,), -1, dtype=torch.int64, device="cuda")
    offsets = torch.full((W * W,), -1, dtype=torch.int64, device="cuda")
    scratch = torch.zeros(plr.plr_copy_v_scratch_bytes(W, rows), dtype=torch.uint8, device="cuda")
    plr.plr_copy_v(srcs, rows, dests, row_bytes, dst, counts, offsets, scratch)
    torch.cuda.synchronize()
    return (dst.cpu().numpy()[:total * row_bytes], counts.cpu().numpy().reshape(W, W),
            offsets.cpu().numpy().reshape(W, W))


def _check(plr, oracle_mod, srcs, dests, rb):
    out, c, o = _run(plr, srcs, dests, rb)
    ref, rc, ro = oracle_mod.copy_v(srcs, dests, rb)
    assert np.array_equal(c, rc)
    assert np.array_equal(o, ro)
    assert np.array_equal(out, ref)


def test_golden_small(plr, oracle_mod):
    lines = list(golden_lines("copy_v_small.txt"))
    W = int(lines[0].split()[1])
    dests = [np.array([int(v) for v in l.split()[2:]], np.int32) for l in lines[1:1 + W]]
    srcs = [synth.bits_np(0, 5, s, d.size * 32) for s, d in enumerate(dests)]
    out, c, o = _run(plr, srcs, dests, 32)
    assert np.array_equal(c.reshape(-1), [int(v) for v in lines[1 + W].split()[1:]])
    assert np.array_equal(o.reshape(-1), [int(v) for v in lines[2 + W].split()[1:]])
    order = [tuple(int(v) for v in t.split(":")) for t in lines[3 + W].split()[1:]]
    rows = out.reshape(-1, 32)
    for k, (s, i) in enumerate(order):
        assert np.array_equal(rows[k], srcs[s].reshape(-1, 32)[i])


@pytest.mark.parametrize("W,rows_each,rb", [(1, 100, 16), (2, 7, 48), (3, 513, 32), (8, 300, 14336),
                                            (16, 40, 64), (5, 0, 16)])
def test_random_zipf(plr, oracle_mod, W, rows_each, rb):
    rows = [rows_each + (s * 7) % 3 if rows_each else (s % 2) * 5 for s in range(W)]
    p = synth.zipf_weights(1.1, W)
    dests = [synth.categorical_np(W, 5, s, rows[s], p) for s in range(W)]
    srcs = [synth.bits_np(W, 6, s, max(rows[s], 1) * rb) for s in range(W)]
    _check(plr, oracle_mod, srcs, dests, rb)


def test_many_tiles_per_source(plr, oracle_mod):
    """More rows per source than one rank-kernel tile (4096), uneven across sources."""
    W, rb = 4, 16
    rows = [10000, 4096, 4097, 1]
    dests = [synth.categorical_np(9, 5, s, rows[s], synth.zipf_weights(1.1, W)) for s in range(W)]
    srcs = [synth.bits_np(9, 6, s, rows[s] * rb) for s in range(W)]
    _check(plr, oracle_mod, srcs, dests, rb)


@pytest.mark.parametrize("rb", [2064, 6160, 4096])
def test_row_tiles_ragged(plr, oracle_mod, rb):
    """Rows that are not a whole number of the scatter's 2 KiB tiles (a last tile of one
    vector, or of 2 KiB + 16 bytes), and rows of exactly two tiles."""
    W = 3
    rows = [37, 0, 21]
    p = synth.zipf_weights(1.1, W)
    dests = [synth.categorical_np(13, 5, s, rows[s], p) for s in range(W)]
    srcs = [synth.bits_np(13, 6, s, max(rows[s], 1) * rb) for s in range(W)]
    _check(plr, oracle_mod, srcs, dests, rb)


def test_many_segments(plr, oracle_mod):
    """More segment counts (1024-row segments x W) than the last rank workgroup stages in
    LDS (8192): W=16 with 36,000 rows per source gives 576 segments, 9216 counts."""
    W, R, rb = 16, 36000, 16
    p = synth.zipf_weights(1.1, W)
    dests = [synth.categorical_np(14, 5, s, R + s, p) for s in range(W)]
    srcs = [synth.bits_np(14, 6, s, (R + s) * rb) for s in range(W)]
    _check(plr, oracle_mod, srcs, dests, rb)


def test_special_destinations(plr, oracle_mod):
    W, R, rb = 8, 1000, 32
    srcs = [synth.bits_np(11, 6, s, R * rb) for s in range(W)]
    _check(plr, oracle_mod, srcs, [np.zeros(R, np.int32)] * W, rb)
    _check(plr, oracle_mod, srcs, [(np.arange(R) % W).astype(np.int32)] * W, rb)
    _check(plr, oracle_mod, srcs, [np.full(R, W - 1, np.int32)] * W, rb)


def test_config5_moe_dispatch(plr, oracle_mod):
    """8 sources x 4096 rows of 7168 bf16, destinations from Zipf(1.1) weights; the
    whole output, counts and offsets."""
    W, R, rb = 8, 4096, 7168 * 2
    p = synth.zipf_weights(1.1, W)
    dests = [synth.categorical_np(0, 5, s, R, p) for s in range(W)]
    srcs = [synth.bits_np(0, 6, s, R * rb) for s in range(W)]
    _check(plr, oracle_mod, srcs, dests, rb)


def test_scratch_reused_across_calls(plr, oracle_mod):
    """The scratch header (the finished-workgroup ticket) returns to zero after every
    call, so one zeroed scratch serves many calls with different row counts."""
    W, rb = 4, 32
    p = synth.zipf_weights(1.1, W)
    scratch = torch.zeros(plr.plr_copy_v_scratch_bytes(W, [3000] * W), dtype=torch.uint8, device="cuda")
    for k, rows_each in enumerate([3000, 17, 1000, 0, 2999]):
        rows = [rows_each] * W
        dests_np = [synth.categorical_np(k, 5, s, rows_each, p) for s in range(W)]
        srcs_np = [synth.bits_np(k, 6, s, max(rows_each, 1) * rb) for s in range(W)]
        srcs = [to_dev(s) for s in srcs_np]
        dests = [torch.from_numpy(d.copy()).cuda() if d.size else torch.zeros(4, dtype=torch.int32, device="cuda")
                 for d in dests_np]
        total = sum(rows)
        dst = torch.zeros(max(total * rb, 16), dtype=torch.uint8, device="cuda")
        counts = torch.empty(W * W, dtype=torch.int64, device="cuda")
        offsets = torch.empty(W * W, dtype=torch.int64, device="cuda")
        plr.plr_copy_v(srcs, rows, dests, rb, dst, counts, offsets, scratch)
        torch.cuda.synchronize()
        ref, rc, ro = oracle_mod.copy_v(srcs_np, dests_np, rb)
        assert np.array_equal(counts.cpu().numpy().reshape(W, W), rc)
        assert np.array_equal(offsets.cpu().numpy().reshape(W, W), ro)
        assert np.array_equal(dst.cpu().numpy()[:total * rb], ref)
        assert int(scratch[:4].view(torch.int32).item()) == 0


@pytest.mark.parametrize("W", [1, 8, 16])
def test_all_sources_empty(plr, oracle_mod, W):
    """No rows anywhere: counts and offsets come back zero and nothing is moved."""
    srcs = [np.zeros(16, np.uint8) for _ in range(W)]
    dests = [np.zeros(0, np.int32) for _ in range(W)]
    out, c, o = _run(plr, srcs, dests, 16)
    assert out.size == 0 and not c.any() and not o.any()


@pytest.mark.parametrize("W,rows", [(8, [1024] * 8), (8, [1025] + [1024] * 7), (4, [4096] * 4),
                                    (4, [4096] * 3 + [4097]), (2, [1, 0]), (16, [3] * 4 + [0] * 12),
                                    (8, [4096] * 8), (8, [4097] + [4096] * 7), (16, [1024] * 16),
                                    (16, [1025] + [1024] * 15), (3, [40000, 0, 3]), (8, [8192] * 8),
                                    (8, [8193] + [8192] * 7), (16, [2048] * 16), (16, [2049] + [2048] * 15)])
def test_small_and_ticket_forms(plr, oracle_mod, W, rows):
    """Both sides of each switch between the small forms (at most 64 segment counts, one
    per lane; at most 256, four per lane: the scatter derives the output rows from the
    counts) and the ticket form (the last rank workgroup scans them), and the ticket form
    at 512 segment counts and beyond."""
    p = synth.zipf_weights(1.1, W)
    dests = [synth.categorical_np(W, 9, s, rows[s], p) for s in range(W)]
    srcs = [synth.bits_np(W, 10, s, max(rows[s], 1) * 64) for s in range(W)]
    _check(plr, oracle_mod, srcs, dests, 64)


@pytest.mark.parametrize("rb", [16, 1008, 1024, 1040, 2048, 2064, 5 * 1024 + 48])
def test_row_sizes_both_scatter_shapes(plr, oracle_mod, rb):
    """Both sides of the scatter's shape switch (rows of at most 1 KiB: 1 KiB tiles of 64
    lanes in runs of 4; larger: 2 KiB tiles of 128 lanes in runs of 2), with ragged last
    tiles in each."""
    W, rows = 8, [300, 0, 129, 1025, 64, 1, 700, 333]
    p = synth.zipf_weights(1.1, W)
    dests = [synth.categorical_np(W, 11, s, rows[s], p) for s in range(W)]
    srcs = [synth.bits_np(W, 12, s, max(rows[s], 1) * rb) for s in range(W)]
    _check(plr, oracle_mod, srcs, dests, rb)
