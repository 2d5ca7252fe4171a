"""Parity of plr_copy (HIP, through the C ABI) with the oracle: bitwise."""
import numpy as np
import pytest
import torch

import synth
from plrtest import empty_dev, from_dev, to_dev

pytestmark = pytest.mark.gpu

PAIRS = {"allgather": ("packed", "packed"), "alltoall": ("scattered", "transposed"),
         "ar_gather": ("scattered", "scattered")}


@pytest.fixture(scope="module")
def plr():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import reduce_atom_amd

    return reduce_atom_amd


def _run(plr, L, srcs_np, workspace=False):
    srcs = [to_dev(s) for s in srcs_np]
    dst = empty_dev(L.dst_bytes, fill=0x5A)
    ws = None
    if workspace:
        ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device="cuda")
        plr.plr_notify(L, -1, ws)
    plr.plr_copy(L, srcs, dst, ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert plr.plr_check(L, ws) == plr.PLR_OK
    return from_dev(dst)[:L.dst_bytes]


@pytest.mark.parametrize("kind", list(PAIRS))
@pytest.mark.parametrize("W", [1, 2, 3, 8, 9, 16])
def test_small_ragged(plr, oracle_mod, kind, W):
    B = 16 * W * 37  # not a multiple of the chunk: ragged last chunk in every segment
    srcs = [synth.bits_np(1, 4, s, B) for s in range(W)]
    ref = oracle_mod.copy_layout(*PAIRS[kind], srcs)
    for kw in (dict(), dict(chunk_bytes=64), dict(chunk_bytes=256, workgroups=3, block=64, unroll=2)):
        L = plr.plr_layout_create("copy", "bf16", W, B, *PAIRS[kind], **kw)
        assert np.array_equal(_run(plr, L, srcs), ref), (kind, W, kw)


@pytest.mark.parametrize("kind", list(PAIRS))
def test_notified(plr, oracle_mod, kind):
    W, B = 8, 8 * 1024 * 16
    srcs = [synth.bits_np(2, 4, s, B) for s in range(W)]
    ref = oracle_mod.copy_layout(*PAIRS[kind], srcs)
    L = plr.plr_layout_create("copy", "bf16", W, B, *PAIRS[kind], chunk_bytes=4096)
    assert np.array_equal(_run(plr, L, srcs, workspace=True), ref)


def _sizes_around_run_switch(plr, kind, W=8):
    """Per-source sizes whose layouts have just under 4096 tiles, exactly 4096 and just
    over (all but the exact one with a ragged last tile)."""
    q = 16 * W
    lay = lambda B: plr.plr_layout_create("copy", "bf16", W, B, *PAIRS[kind])
    exact = (1 << 20) * 4096 // lay(1 << 20).ntiles
    assert lay(exact).ntiles == 4096, (kind, exact, lay(exact).ntiles)
    below = exact - q
    while lay(below).ntiles >= 4096:
        below -= q
    return [below - q, exact, exact + q]


@pytest.mark.parametrize("kind", list(PAIRS))
def test_policy_run_boundary(plr, oracle_mod, kind):
    """Copies of 4096 tiles or more run two 2 KiB tiles per workgroup: both sides of the
    switch, un-notified and notified."""
    W = 8
    for B in _sizes_around_run_switch(plr, kind, W):
        srcs = [synth.bits_np(7, 4, s, B) for s in range(W)]
        ref = oracle_mod.copy_layout(*PAIRS[kind], srcs)
        L = plr.plr_layout_create("copy", "bf16", W, B, *PAIRS[kind])
        assert np.array_equal(_run(plr, L, srcs), ref), (kind, B, L.ntiles)
        assert np.array_equal(_run(plr, L, srcs, workspace=True), ref), (kind, B, L.ntiles)


def test_explicit_offsets(plr, oracle_mod):
    W, B = 4, 4096
    srcs = [synth.bits_np(3, 4, s, 2 * B) for s in range(W)]
    in_off = [0, 16, B, 2 * B - B]
    out_off = [3 * B, 0, 2 * B, B]  # a permuted AllGather
    segs = [(s, in_off[s], out_off[s], B) for s in range(W)]
    ref = oracle_mod.copy(srcs, segs, W * B)
    L = plr.plr_layout_create("copy", "bf16", W, B, "packed", "packed", in_offsets=in_off,
                              out_offsets=out_off, chunk_bytes=1024)
    assert sorted(L.segments()) == sorted(segs)
    assert np.array_equal(_run(plr, L, srcs), ref)


def test_nan_payloads_preserved(plr):
    pat = np.array([0x7F800001, 0xFFC01234, 0x7FBFFFFF, 0x00000001], dtype=np.uint32)
    srcs = [np.tile(pat, 64).view(np.uint8), np.tile(pat[::-1].copy(), 64).view(np.uint8)]
    L = plr.plr_layout_create("copy", "f32", 2, srcs[0].nbytes, "packed", "packed")
    assert _run(plr, L, srcs).tobytes() == srcs[0].tobytes() + srcs[1].tobytes()


@pytest.mark.parametrize("notified", [False, True])
@pytest.mark.parametrize("kind", ["allgather", "alltoall"])
def test_config4_full(plr, oracle_mod, kind, notified):
    """8 sources of 64 MiB of random bits; AllGather into 512 MiB, AllToAll of 8 MiB
    tiles; the whole output compared with the oracle, default policy, un-notified and in
    the bench's launch configuration (notified, check mode: runs of 2 tiles)."""
    W, B = 8, 64 << 20
    srcs = [synth.bits_t(0, 4, s, B, device="cuda") for s in range(W)]
    L = plr.plr_layout_create("copy", "bf16", W, B, *PAIRS[kind])
    dst = torch.full((L.dst_bytes,), 0x5A, dtype=torch.uint8, device="cuda")
    ws = None
    if notified:
        ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device="cuda")
        plr.plr_notify(L, -1, ws)
    plr.plr_copy(L, srcs, dst, ws)
    torch.cuda.synchronize()
    if notified:
        assert plr.plr_check(L, ws) == plr.PLR_OK
    ref = oracle_mod.copy_layout(*PAIRS[kind], [s.cpu().numpy() for s in srcs])
    assert np.array_equal(dst.cpu().numpy(), ref)


def test_alltoall_twice_is_identity(plr):
    W, B = 8, 16 * 8 * 1000
    srcs = [synth.bits_t(4, 4, s, B, device="cuda") for s in range(W)]
    L = plr.plr_layout_create("copy", "bf16", W, B, "scattered", "transposed")
    mid = torch.empty(W * B, dtype=torch.uint8, device="cuda")
    plr.plr_copy(L, srcs, mid)
    back = torch.empty(W * B, dtype=torch.uint8, device="cuda")
    plr.plr_copy(L, list(mid.view(W, B)), back)
    assert torch.equal(back, torch.cat(srcs))
