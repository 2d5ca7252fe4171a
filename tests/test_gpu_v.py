"""Parity of the variable-length collectives (HIP, through the C ABI) with the oracle:
AllGatherV bitwise, ReduceScatterV bitwise (NaN as a class), un-notified and notified,
with the benchmark's Zipf partitions (appendix C.4), empty and 16-byte partitions,
ragged tiles and a per-source producer."""
import numpy as np
import pytest
import torch

import synth
from plrtest import assert_same, empty_dev, from_dev, to_dev

pytestmark = pytest.mark.gpu

MODES = {"chunks": 1, "check": 2}


@pytest.fixture(scope="module")
def plr():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import reduce_atom_amd

    return reduce_atom_amd


PART_SETS = {
    "zipf_8k": (8, synth.zipf_split(8192, 8)),
    "zipf_1m": (8, synth.zipf_split(1 << 20, 8)),
    "uniform_1k": (8, synth.zipf_split(1024, 8)),
    "empty_and_tiny": (5, [0, 16, 4096 + 48, 0, 32]),
    "one_rank": (1, [3 * 2048 + 16]),
    "w16_ragged": (16, [16 * (7 * k + 3) for k in range(16)]),
}


def _agv(plr, L, srcs_np, notify=None):
    srcs = [to_dev(s) for s in srcs_np]
    dst = empty_dev(max(L.dst_bytes, 16), fill=0x5A)
    ws = None
    if notify is not None:
        ws = torch.zeros(max(L.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
        for w in notify:
            plr.plr_notify(L, w, ws)
    plr.plr_copy(L, srcs, dst, ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert plr.plr_check(L, ws) == plr.PLR_OK
    return from_dev(dst)[:L.dst_bytes]


@pytest.mark.parametrize("name", list(PART_SETS))
def test_allgather_v(plr, oracle_mod, name):
    W, parts = PART_SETS[name]
    T = sum(parts)
    srcs = [synth.bits_np(31, 7, w, max(p, 16)) for w, p in enumerate(parts)]
    ref = oracle_mod.allgather_v(srcs, parts)
    for kw in (dict(), dict(tile_bytes=256, chunk_bytes=1024), dict(tile_bytes=1024, workgroups=3, block=64,
                                                                    unroll=2)):
        L = plr.plr_layout_create("copy", "bf16", W, T, "packed", "packed", part_bytes=parts, **kw)
        assert np.array_equal(_agv(plr, L, srcs), ref), (name, kw)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("name", ["zipf_1m", "empty_and_tiny", "w16_ragged"])
def test_allgather_v_notified_per_source(plr, oracle_mod, name, mode):
    """Every source notifies only its own flags (a source with an empty contribution
    has none); the consumer waits for each segment's own chunks."""
    W, parts = PART_SETS[name]
    T = sum(parts)
    srcs = [synth.bits_np(32, 7, w, max(p, 16)) for w, p in enumerate(parts)]
    ref = oracle_mod.allgather_v(srcs, parts)
    L = plr.plr_layout_create("copy", "bf16", W, T, "packed", "packed", part_bytes=parts, tile_bytes=512,
                              chunk_bytes=2048, notify_mode=MODES[mode])
    for epoch in range(3):
        assert np.array_equal(_agv(plr, L, srcs, notify=range(W)), ref), (name, mode, epoch)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("name", ["zipf_8k", "zipf_1m", "empty_and_tiny", "w16_ragged"])
def test_reduce_scatter_v(plr, oracle_mod, name, dtype):
    W, parts = PART_SETS[name]
    T = sum(parts)
    eb = oracle_mod.ELEM_BYTES[dtype]
    srcs_np = [synth.normal_np(33, 7, w, T // eb, dtype=dtype) for w in range(W)]
    srcs = [to_dev(s) for s in srcs_np]
    for r in range(W):
        ref = oracle_mod.reduce_scatter_v(dtype, srcs_np, parts, r)
        L = plr.plr_layout_create("reduce", dtype, W, T, "scattered", "packed", rank=r, part_bytes=parts)
        dst = empty_dev(max(parts[r], 16), fill=0x5A)
        plr.plr_reduce(L, srcs, dst)
        torch.cuda.synchronize()
        assert_same(dtype, from_dev(dst)[:parts[r]], ref.view(np.uint8), f"{name} rank {r}")


@pytest.mark.parametrize("mode", list(MODES))
def test_reduce_scatter_v_notified(plr, oracle_mod, mode):
    W = 8
    parts = synth.zipf_split(1 << 21, W)
    T = sum(parts)
    srcs_np = [synth.normal_np(34, 7, w, T // 2) for w in range(W)]
    srcs = [to_dev(s) for s in srcs_np]
    for r in (0, 7):
        ref = oracle_mod.reduce_scatter_v("bf16", srcs_np, parts, r)
        L = plr.plr_layout_create("reduce", "bf16", W, T, "scattered", "packed", rank=r, part_bytes=parts,
                                  chunk_bytes=16384, notify_mode=MODES[mode])
        ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device="cuda")
        dst = empty_dev(parts[r], fill=0x5A)
        for epoch in range(2):
            for w in range(W):
                plr.plr_notify(L, w, ws)
            plr.plr_reduce(L, srcs, dst, ws)
            assert plr.plr_check(L, ws) == plr.PLR_OK
            assert_same("bf16", from_dev(dst), ref.view(np.uint8), f"rank {r} epoch {epoch}")


def test_allgather_v_1gib_full(plr, oracle_mod):
    """The bench's AllGatherV: 8 contributions of the Zipf(s = 0.125) split of T = 1 GiB,
    default policy; the whole 1 GiB output against the oracle."""
    W, T = 8, 1 << 30
    parts = synth.zipf_split(T, W)
    srcs = [synth.bits_t(0, 7, w, parts[w], device="cuda") for w in range(W)]
    L = plr.plr_layout_create("copy", "bf16", W, T, "packed", "packed", part_bytes=parts)
    dst = torch.full((T,), 0x5A, dtype=torch.uint8, device="cuda")
    plr.plr_copy(L, srcs, dst)
    torch.cuda.synchronize()
    ref = oracle_mod.allgather_v([s.cpu().numpy() for s in srcs], parts)
    assert np.array_equal(dst.cpu().numpy(), ref)


def test_reduce_scatter_v_1gib_full(plr, oracle_mod):
    """The bench's ReduceScatterV share: rank 0 of the Zipf split of T = 1 GiB over 8
    contributions of T bytes bf16, N(0, 1), default policy; the whole share (157,859,568
    bytes) against the oracle's reduction of partition 0 of every source."""
    W, T = 8, 1 << 30
    parts = synth.zipf_split(T, W)
    srcs = [synth.normal_t(0, 8, w, T // 2, 1.0, device="cuda") for w in range(W)]
    L = plr.plr_layout_create("reduce", "bf16", W, T, "scattered", "packed", rank=0, part_bytes=parts)
    n = parts[0] // 2
    dst = torch.full((n,), float("nan"), dtype=torch.bfloat16, device="cuda")
    plr.plr_reduce(L, srcs, dst)
    torch.cuda.synchronize()
    got = dst.view(torch.int16).cpu().numpy().view(np.uint16)
    host = [s[:n].view(torch.int16).cpu().numpy().view(np.uint16) for s in srcs]  # partition 0 starts at 0
    assert_same("bf16", got, oracle_mod.reduce("bf16", host, threads=oracle_mod.default_threads()))
