"""The notification protocol (stage / notify / consume) on one GPU: a consumer never
reads a chunk before its flag, a withheld flag ends in PLR_ETIMEOUT (no hang), and
epochs keep working across many calls without resetting the workspace."""
import numpy as np
import pytest
import torch

import synth
from plrtest import assert_same, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def plr():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import reduce_atom_amd

    return reduce_atom_amd


MODES = {"chunks": 1, "check": 2}


def _diag(L, ws, op):
    """(ready word, late counter, check-time mirror of every flag) of a workspace."""
    words = ws.view(torch.int64).cpu().numpy()
    nflags = L.nchunks if op == "copy" else L.world * L.nchunks
    return int(words[1]), int(words[2]), words[32 + nflags: 32 + 2 * nflags]


def _until_waited(plr, L, ws, op, mode, produce_late, consume, check, produce_early=None, missing=None,
                  attempts=8):
    """The delayed-producer scenario: the producer's work (poison, a sleep, the real data,
    its notify) is queued on one fresh stream and the consumer's call on another, so the
    consumer reaches the flags before they are set and must wait. Whether two streams run
    concurrently is up to how HIP maps them to hardware queues, so the scenario is run on
    new stream pairs until the workspace shows that the consumer waited (its late counter
    grew; in check mode the check also found the flags missing: ready word 0, mirror 0 for
    `missing`); every attempt's output is checked. Returns the attempts taken."""
    for attempt in range(1, attempts + 1):
        torch.cuda.synchronize()
        before = _diag(L, ws, op)[1]
        if produce_early is not None:
            produce_early()
            torch.cuda.synchronize()
        producer, consumer = torch.cuda.Stream(), torch.cuda.Stream()
        with torch.cuda.stream(producer):  # queued first: a consumer queued first on a
            produce_late()                 # hardware queue it shares could only time out
        with torch.cuda.stream(consumer):
            consume()
        torch.cuda.synchronize()
        assert plr.plr_check(L, ws, consumer) == plr.PLR_OK
        check()
        ready, late, mirror = _diag(L, ws, op)
        if late > before:
            if mode == "check":
                assert ready == 0, ready
                assert (mirror == 0).any()
                if missing is not None:
                    assert (mirror[missing] == 0).all()
            return attempt
    pytest.fail(f"the consumer never had to wait in {attempts} attempts: the streams never overlapped")


def _poison_then_real(plr, L, ws, srcs, real, poison, notify_srcs):
    def produce():
        for x in srcs:
            x.fill_(poison)
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(20_000_000)
        for x, r in zip(srcs, real):
            x.copy_(r)
        for w in notify_srcs:
            plr.plr_notify(L, w, ws)
    return produce


@pytest.mark.parametrize("mode", list(MODES))
def test_many_calls_without_reset(plr, oracle_mod, mode):
    W, n = 4, 8192
    srcs_np = [synth.normal_np(1, 2, w, n) for w in range(W)]
    ref = oracle_mod.reduce("bf16", srcs_np)
    srcs = [to_dev(s) for s in srcs_np]
    L = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed", chunk_bytes=2048,
                              notify_mode=MODES[mode])
    ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(2 * n, dtype=torch.uint8, device="cuda")
    for i in range(1000):
        for w in range(W):
            plr.plr_notify(L, w, ws)
        plr.plr_reduce(L, srcs, dst, ws)
    assert plr.plr_check(L, ws) == plr.PLR_OK
    assert L.epoch == 1000
    assert_same("bf16", dst.cpu().numpy().view(np.uint16), ref)
    flags = ws[256:256 + 8 * W * L.nchunks].view(torch.int64).cpu().numpy()
    assert (flags == 1000).all()
    ready, late, _ = _diag(L, ws, "reduce")
    assert late == 0  # every flag was set before its call: no wait ever polled
    if mode == "check":
        assert ready == 1000


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("op", ["reduce", "copy"])
def test_withheld_notify_times_out(plr, op, mode):
    W, nbytes = 4, 16384
    srcs = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(W)]
    kinds = ("packed", "packed")
    L = plr.plr_layout_create(op, "bf16", W, nbytes, *kinds, chunk_bytes=4096, spin_limit=2000,
                              notify_mode=MODES[mode])
    ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(L.dst_bytes, dtype=torch.uint8, device="cuda")
    for w in range(W - 1):  # the last source never notifies
        plr.plr_notify(L, w, ws)
    (plr.plr_reduce if op == "reduce" else plr.plr_copy)(L, srcs, dst, ws)
    assert plr.plr_check(L, ws) == plr.PLR_ETIMEOUT
    assert plr.plr_check(L, ws) == plr.PLR_OK  # read-and-clear
    # the next epoch works once every source notifies
    plr.plr_notify(L, -1, ws)
    (plr.plr_reduce if op == "reduce" else plr.plr_copy)(L, srcs, dst, ws)
    assert plr.plr_check(L, ws) == plr.PLR_OK


@pytest.mark.parametrize("mode", list(MODES))
def test_delayed_producer_on_another_stream(plr, oracle_mod, mode):
    """The producer writes poison, sleeps, writes the real data and notifies, all on its
    own stream; the consumer is queued right after on another stream, so it reaches the
    flags long before they are set and must wait for them; its output must be the
    reduction of the real data, never of the poison. The workspace's diagnostics prove
    that the wait happened (the late counter grew; in check mode the check found the
    flags missing). The producer is queued first: a consumer queued first on a hardware
    queue it shares with the producer could only time out."""
    W, n = 8, 1 << 16
    real_np = [synth.normal_np(2, 2, w, n) for w in range(W)]
    ref = oracle_mod.reduce("bf16", real_np)
    real = [to_dev(s) for s in real_np]
    srcs = [torch.empty_like(r) for r in real]
    L = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed", chunk_bytes=4096,
                              workgroups=4, block=64, spin_limit=1 << 22, notify_mode=MODES[mode])
    ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(2 * n, dtype=torch.uint8, device="cuda")
    _until_waited(plr, L, ws, "reduce", mode,
                  produce_late=_poison_then_real(plr, L, ws, srcs, real, 0xFF, [-1]),  # NaN poison
                  consume=lambda: plr.plr_reduce(L, srcs, dst, ws),
                  check=lambda: assert_same("bf16", dst.cpu().numpy().view(np.uint16), ref))


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("op", ["reduce", "copy"])
def test_tiles_crossing_chunks(plr, oracle_mod, op, mode):
    """Few workgroups striding over many tiles, several tiles per chunk and ragged
    ends on both levels: every chunk's flags are waited for exactly when needed."""
    W, nbytes = 4, 37 * 1024 + 48
    if op == "reduce":
        srcs_np = [synth.normal_np(3, 2, w, nbytes // 2) for w in range(W)]
        ref = oracle_mod.reduce("bf16", srcs_np)
        L = plr.plr_layout_create("reduce", "bf16", W, nbytes, "packed", "packed", tile_bytes=1024,
                                  chunk_bytes=4096, workgroups=3, block=64, notify_mode=MODES[mode])
    else:
        nbytes = 16 * W * 150
        srcs_np = [synth.bits_np(3, 4, s, nbytes) for s in range(W)]
        ref = oracle_mod.copy_layout("scattered", "transposed", srcs_np).view(np.uint16)
        L = plr.plr_layout_create("copy", "bf16", W, nbytes, "scattered", "transposed", tile_bytes=256,
                                  chunk_bytes=1024, workgroups=5, block=64, notify_mode=MODES[mode])
    srcs = [to_dev(s) for s in srcs_np]
    ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(L.dst_bytes, dtype=torch.uint8, device="cuda")
    for epoch in range(1, 4):
        for w in range(W):
            plr.plr_notify(L, w, ws)
        (plr.plr_reduce if op == "reduce" else plr.plr_copy)(L, srcs, dst, ws)
        assert plr.plr_check(L, ws) == plr.PLR_OK
        if op == "copy":  # copies are bitwise, NaN payloads included
            assert np.array_equal(dst.cpu().numpy().view(np.uint16), ref), f"epoch {epoch}"
        else:
            assert_same("bf16", dst.cpu().numpy().view(np.uint16), ref, f"epoch {epoch}")


@pytest.mark.parametrize("op", ["reduce", "copy"])
def test_check_mode_partial_arrival(plr, oracle_mod, op):
    """Check mode where half the sources are notified before the call and half by a
    delayed producer on a second stream: the check finds the late sources' flags missing
    (and only those) and the consumer takes the per-chunk path and waits for them, which
    the workspace's diagnostics confirm."""
    W, nbytes = 4, 64 * 1024
    real_np = [synth.bits_np(7, 4, s, nbytes) for s in range(W)]
    if op == "reduce":
        real_np = [synth.normal_np(7, 2, w, nbytes // 2) for w in range(W)]
        ref = oracle_mod.reduce("bf16", real_np)
    else:
        ref = oracle_mod.copy_layout("packed", "packed", real_np).view(np.uint16)
    real = [to_dev(s) for s in real_np]
    srcs = [torch.empty_like(r) for r in real]
    L = plr.plr_layout_create(op, "bf16", W, nbytes, "packed", "packed", chunk_bytes=8192,
                              workgroups=4, block=64, spin_limit=1 << 22, notify_mode=MODES["check"])
    ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(L.dst_bytes, dtype=torch.uint8, device="cuda")

    def early():  # sources 0 and 1: written and announced before the call
        for x, r in zip(srcs[:2], real[:2]):
            x.copy_(r)
        for w in range(2):
            plr.plr_notify(L, w, ws)

    def check():
        if op == "copy":
            assert np.array_equal(dst.cpu().numpy().view(np.uint16), ref)
        else:
            assert_same("bf16", dst.cpu().numpy().view(np.uint16), ref)

    nflags = L.nchunks if op == "copy" else W * L.nchunks
    consume = (lambda: plr.plr_reduce(L, srcs, dst, ws)) if op == "reduce" else (lambda: plr.plr_copy(L, srcs, dst, ws))
    # the late sources (2 and 3) own the second half of the flags: missing at check time,
    # while the early ones had arrived
    _until_waited(plr, L, ws, op, "check", produce_early=early,
                  produce_late=_poison_then_real(plr, L, ws, srcs[2:], real[2:], 0xFF, range(2, W)),
                  consume=consume, check=check, missing=np.arange(nflags // 2, nflags))
    assert (_diag(L, ws, op)[2][: nflags // 2] == L.epoch).all()


def test_check_mode_many_flags(plr, oracle_mod):
    """More flags (16,384) than the check's lanes hold in one round of loads (8,192): the
    check's outcome, the ready word and the mirror cover every flag; a flag still missing in the
    second round sends the consumer to wait and, withheld, to PLR_ETIMEOUT."""
    W, nbytes = 8, 1 << 20
    srcs_np = [synth.bits_np(8, 4, s, nbytes) for s in range(W)]
    ref = oracle_mod.copy_layout("packed", "packed", srcs_np).view(np.uint16)
    srcs = [to_dev(s) for s in srcs_np]
    L = plr.plr_layout_create("copy", "bf16", W, nbytes, "packed", "packed", tile_bytes=512, chunk_bytes=512,
                              spin_limit=2000, notify_mode=MODES["check"])
    nflags = L.nchunks  # copy: one flag per chunk of every segment
    assert nflags == 16384
    ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(L.dst_bytes, dtype=torch.uint8, device="cuda")
    plr.plr_notify(L, -1, ws)
    plr.plr_copy(L, srcs, dst, ws)
    assert plr.plr_check(L, ws) == plr.PLR_OK
    assert np.array_equal(dst.cpu().numpy(), ref.view(np.uint8))
    words = ws.view(torch.int64).cpu().numpy()
    assert words[1] == 1  # ready: every flag had arrived at epoch 1
    mirror = words[32 + nflags: 32 + 2 * nflags]
    assert (mirror == 1).all()
    # epoch 2: the last source (flags 14,336.. in the check's second round) withholds
    for w in range(W - 1):
        plr.plr_notify(L, w, ws)
    plr.plr_copy(L, srcs, dst, ws)
    assert plr.plr_check(L, ws) == plr.PLR_ETIMEOUT
    words = ws.view(torch.int64).cpu().numpy()
    assert words[1] == 0
    mirror = words[32 + nflags: 32 + 2 * nflags]
    own = nflags // W  # the last source's flags: the last of W equal ranges
    assert (mirror[:nflags - own] == 2).all() and (mirror[nflags - own:] == 0).all()


@pytest.mark.parametrize("mode", list(MODES))
def test_allgatherv_cut_tiles_wait_for_both_chunks(plr, oracle_mod, mode):
    """AllGatherV with partitions that start inside 128-byte lines of the output: its
    tiles are cut on the output's lines, so most of them span two notification chunks
    (chunks stay whole tiles from the segment start) and wait for both. A delayed
    producer on another stream, as above; the output must be the real data."""
    W = 4
    parts = [16112, 13248, 16 * 1234 + 96, 16 * 555]  # later partitions start 112, 48, 48 B into a line
    real_np = [synth.bits_np(9, 7, w, parts[w]) for w in range(W)]
    ref = oracle_mod.allgather_v(real_np, parts)
    real = [to_dev(s) for s in real_np]
    srcs = [torch.empty_like(r) for r in real]
    T = sum(parts)
    L = plr.plr_layout_create("copy", "bf16", W, T, "packed", "packed", part_bytes=parts, tile_bytes=1024,
                              chunk_bytes=2048, workgroups=3, block=64, spin_limit=1 << 22,
                              notify_mode=MODES[mode])
    assert L.ntiles > sum((p + 1023) // 1024 for p in parts)  # the cut added tiles
    ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(T, dtype=torch.uint8, device="cuda")
    _until_waited(plr, L, ws, "copy", mode,
                  produce_late=_poison_then_real(plr, L, ws, srcs, real, 0xA5, [-1]),
                  consume=lambda: plr.plr_copy(L, srcs, dst, ws),
                  check=lambda: np.testing.assert_array_equal(dst.cpu().numpy(), ref))
