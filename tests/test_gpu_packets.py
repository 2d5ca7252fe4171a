"""Latency-path packets on one GPU: the producer's packets are bit-identical to the
oracle's encoding, the consumer's reduction is bit-identical to the oracle's, a source
whose packets still carry an older epoch is never consumed (PLR_ETIMEOUT instead), and
packet buffers work across many epochs without being reset."""
import numpy as np
import pytest
import torch

import synth
from plrtest import NP_RAW, assert_same, to_dev

pytestmark = pytest.mark.gpu

EB = {"bf16": 2, "f16": 2, "f32": 4}


@pytest.fixture(scope="module")
def plr():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import reduce_atom_amd

    return reduce_atom_amd


def _setup(plr, dtype, W, nbytes, in_kind="packed", rank=0, **kw):
    L = plr.plr_layout_create("reduce", dtype, W, nbytes, in_kind, "packed", rank=rank, **kw)
    pk = [torch.zeros(L.packet_bytes, dtype=torch.uint8, device="cuda") for _ in range(W)]
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    dst = torch.empty(max(L.dst_bytes, 16), dtype=torch.uint8, device="cuda")
    return L, pk, ws, dst


def _srcs_bits(dtype, W, nbytes, seed):
    return [synth.normal_np(seed, 2, w, nbytes // EB[dtype], dtype=dtype) for w in range(W)]


@pytest.mark.parametrize("W", [1, 2, 3, 8])
def test_pack_matches_oracle_encoding(plr, oracle_mod, W):
    nbytes = 16 * W * 37
    srcs_np = [synth.bits_np(11, 1, w, nbytes) for w in range(W)]
    srcs = [to_dev(s) for s in srcs_np]
    L, pk, ws, dst = _setup(plr, "bf16", W, nbytes, "scattered", rank=W - 1)
    share = nbytes // W
    for epoch in (1, 2):
        if epoch == 1:
            for w in range(W):
                plr.plr_pack(L, w, srcs, pk)
        else:
            plr.plr_pack(L, -1, srcs, pk)  # every source in one launch
        torch.cuda.synchronize()
        nw = share // 4  # packets per slot; epoch e uses slot e & 1
        for w in range(W):
            want = oracle_mod.pack(srcs_np[w][(W - 1) * share:], epoch)[:nw]
            got = pk[w].cpu().numpy().view(np.uint64)[(epoch & 1) * nw:(epoch & 1) * nw + nw]
            assert np.array_equal(got, want), (epoch, w)
        plr.plr_reduce_packets(L, pk, dst, ws)
        assert plr.plr_check(L, ws) == plr.PLR_OK


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("W", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 262144 + 16 * 7])
def test_reduce_packets_parity(plr, oracle_mod, dtype, W, nbytes):
    srcs_np = _srcs_bits(dtype, W, nbytes, 12 + W)
    ref = oracle_mod.reduce(dtype, srcs_np)
    srcs = [to_dev(s) for s in srcs_np]
    L, pk, ws, dst = _setup(plr, dtype, W, nbytes)
    for w in range(W):
        plr.plr_pack(L, w, srcs, pk)
    plr.plr_reduce_packets(L, pk, dst, ws)
    assert plr.plr_check(L, ws) == plr.PLR_OK
    assert L.epoch == 1
    assert_same(dtype, dst[:nbytes].cpu().numpy().view(NP_RAW[dtype]), ref)


@pytest.mark.parametrize("W", [2, 8])
def test_reduce_packets_scattered_share(plr, oracle_mod, W):
    nbytes = 16 * W * 1000
    srcs_np = [synth.normal_np(13, 2, w, nbytes // 2) for w in range(W)]
    srcs = [to_dev(s) for s in srcs_np]
    for rank in (0, W - 1):
        ref = oracle_mod.reduce_layout("bf16", "scattered", rank, srcs_np)
        L, pk, ws, dst = _setup(plr, "bf16", W, nbytes, "scattered", rank=rank)
        for w in range(W):
            plr.plr_pack(L, w, srcs, pk)
        plr.plr_reduce_packets(L, pk, dst, ws)
        assert plr.plr_check(L, ws) == plr.PLR_OK
        assert_same("bf16", dst.cpu().numpy().view(np.uint16), ref, f"rank {rank}")


def test_special_values(plr, oracle_mod):
    """Infinities, NaNs, signed zeros, overflow and denormals go through the payload
    words untouched and reduce as the oracle does."""
    W, n = 4, 4096
    specials = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0x7F7F, 0xFF7F, 0x0001, 0x8001,
                         0x3F80, 0xBF80, 0x4B80, 0xCB80], dtype=np.uint16)
    srcs_np = []
    for w in range(W):
        idx = synth.categorical_np(14, 1, w, n, np.ones(specials.size) / specials.size)
        srcs_np.append(specials[idx])
    ref = oracle_mod.reduce("bf16", srcs_np)
    srcs = [to_dev(s) for s in srcs_np]
    L, pk, ws, dst = _setup(plr, "bf16", W, 2 * n)
    for w in range(W):
        plr.plr_pack(L, w, srcs, pk)
    plr.plr_reduce_packets(L, pk, dst, ws)
    assert plr.plr_check(L, ws) == plr.PLR_OK
    assert_same("bf16", dst.cpu().numpy().view(np.uint16), ref)


def test_many_epochs_without_reset(plr, oracle_mod):
    W, n = 4, 8192
    a_np = [synth.normal_np(15, 2, w, n) for w in range(W)]
    b_np = [synth.normal_np(15, 3, w, n) for w in range(W)]
    a, b = [to_dev(s) for s in a_np], [to_dev(s) for s in b_np]
    ra, rb = oracle_mod.reduce("bf16", a_np), oracle_mod.reduce("bf16", b_np)
    L, pk, ws, dst = _setup(plr, "bf16", W, 2 * n)
    for i in range(1, 501):
        srcs = a if i % 2 else b
        for w in range(W):
            plr.plr_pack(L, w, srcs, pk)
        plr.plr_reduce_packets(L, pk, dst, ws)
        if i in (1, 2, 499, 500):
            assert_same("bf16", dst.cpu().numpy().view(np.uint16), ra if i % 2 else rb, f"call {i}")
    assert plr.plr_check(L, ws) == plr.PLR_OK
    assert L.epoch == 500
    stamps = (pk[0].cpu().numpy().view(np.uint64) >> np.uint64(32)).reshape(2, -1)
    assert (stamps[0] == 500).all() and (stamps[1] == 499).all()  # slot = epoch parity


def test_stale_packets_time_out(plr, oracle_mod):
    """After epoch 1 every packet buffer holds epoch-1 packets of poison data; in epoch 2
    the last source never packs, so its packets keep the old stamp: the consumer must
    time out rather than reduce them, and epoch 3 works once every source packs."""
    W, n = 4, 8192
    real_np = [synth.normal_np(16, 2, w, n) for w in range(W)]
    real = [to_dev(s) for s in real_np]
    poison = [torch.full((2 * n,), 0xFF, dtype=torch.uint8, device="cuda") for _ in range(W)]
    L, pk, ws, dst = _setup(plr, "bf16", W, 2 * n, spin_limit=2000)
    for w in range(W):
        plr.plr_pack(L, w, poison, pk)
    plr.plr_reduce_packets(L, pk, dst, ws)
    assert plr.plr_check(L, ws) == plr.PLR_OK
    for w in range(W - 1):
        plr.plr_pack(L, w, real, pk)
    plr.plr_reduce_packets(L, pk, dst, ws)
    assert plr.plr_check(L, ws) == plr.PLR_ETIMEOUT
    assert plr.plr_check(L, ws) == plr.PLR_OK  # read-and-clear
    for w in range(W):
        plr.plr_pack(L, w, real, pk)
    plr.plr_reduce_packets(L, pk, dst, ws)
    assert plr.plr_check(L, ws) == plr.PLR_OK
    assert_same("bf16", dst.cpu().numpy().view(np.uint16), oracle_mod.reduce("bf16", real_np))


def test_delayed_producer_on_another_stream(plr, oracle_mod):
    """The producer writes poison, sleeps, writes the real data and packs it on its own
    stream; the consumer is queued right after on another stream. Where the streams run
    concurrently the consumer finds old or missing stamps and keeps polling; its output
    must be the reduction of the real data. (The producer is queued first, as a consumer
    queued first on a hardware queue it shares with the producer could only time out.)"""
    W, n = 8, 1 << 16
    real_np = [synth.normal_np(17, 2, w, n) for w in range(W)]
    ref = oracle_mod.reduce("bf16", real_np)
    real = [to_dev(s) for s in real_np]
    srcs = [torch.empty_like(r) for r in real]
    L, pk, ws, dst = _setup(plr, "bf16", W, 2 * n, spin_limit=1 << 22)
    torch.cuda.synchronize()
    producer, consumer = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(producer):
        for s in srcs:
            s.fill_(0xFF)
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(20_000_000)
        for s, r in zip(srcs, real):
            s.copy_(r)
        for w in range(W):
            plr.plr_pack(L, w, srcs, pk)
    with torch.cuda.stream(consumer):
        plr.plr_reduce_packets(L, pk, dst, ws)
    torch.cuda.synchronize()
    assert plr.plr_check(L, ws, consumer) == plr.PLR_OK
    assert_same("bf16", dst.cpu().numpy().view(np.uint16), ref)


def test_producer_one_epoch_ahead(plr, oracle_mod):
    """The producer packs epoch 2 while the consumer of epoch 1 may not have read its
    packets yet (the consumer's stream is held by a sleep; the producer's is not): the two
    epochs use the two slots of the packet buffers (epoch parity), so both reductions are
    the oracle's. With one slot the second pack would overwrite the first epoch's packets
    and the first consumer would see the wrong stamp."""
    W, n = 8, 1 << 14
    a_np = [synth.normal_np(18, 2, w, n) for w in range(W)]
    b_np = [synth.normal_np(18, 3, w, n) for w in range(W)]
    a, b = [to_dev(s) for s in a_np], [to_dev(s) for s in b_np]
    L, pk, ws, dst1 = _setup(plr, "bf16", W, 2 * n, spin_limit=1 << 22)
    dst2 = torch.empty_like(dst1)
    torch.cuda.synchronize()
    producer, consumer = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(consumer):
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(20_000_000)
    with torch.cuda.stream(producer):
        plr.plr_pack(L, -1, a, pk)  # epoch 1 (slot 1)
    ev = torch.cuda.Event()
    ev.record(producer)
    with torch.cuda.stream(consumer):
        consumer.wait_event(ev)
        plr.plr_reduce_packets(L, pk, dst1, ws)  # epoch 1
    with torch.cuda.stream(producer):
        plr.plr_pack(L, -1, b, pk)  # epoch 2 (slot 0), possibly before the epoch-1 consumer ran
    with torch.cuda.stream(consumer):
        plr.plr_reduce_packets(L, pk, dst2, ws)  # epoch 2
    torch.cuda.synchronize()
    assert plr.plr_check(L, ws, consumer) == plr.PLR_OK
    assert_same("bf16", dst1.cpu().numpy().view(np.uint16), oracle_mod.reduce("bf16", a_np), "epoch 1")
    assert_same("bf16", dst2.cpu().numpy().view(np.uint16), oracle_mod.reduce("bf16", b_np), "epoch 2")
