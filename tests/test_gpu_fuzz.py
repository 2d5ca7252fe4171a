"""Seeded random configurations of the whole boundary against the oracle: op and layout
kind (reduce share, AllGather, AllToAll, AllReduce gather, AllGatherV, ReduceScatterV),
W, element type, ragged sizes, policy overrides (tile, chunk, block, unroll, grid,
XCD order, datapath) and notification (none, per-chunk waits, check first). Most cases
are small, one in ten has thousands of tiles; a failure prints its configuration."""
import os

import numpy as np
import pytest
import torch

import synth
from plrtest import assert_same, empty_dev, from_dev, to_dev

pytestmark = pytest.mark.gpu

# PLR_FUZZ_SCALE multiplies every seed count (a longer campaign; the default is 1)
SCALE = int(os.environ.get("PLR_FUZZ_SCALE", "1"))
KINDS = ["reduce_packed", "reduce_scattered", "allgather", "alltoall", "ar_gather", "agv", "rsv"]
EB = {"bf16": 2, "f16": 2, "f32": 4}


@pytest.fixture(scope="module")
def plr():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import reduce_atom_amd

    return reduce_atom_amd


def _draw(rng):
    kind = KINDS[rng.integers(len(KINDS))]
    W = int(rng.choice([1, 2, 3, 4, 5, 8, 11, 16]))
    dtype = ["bf16", "f16", "f32"][rng.integers(3)]
    pol = {}
    if rng.random() < 0.7:
        pol["tile_bytes"] = int(rng.choice([256, 1024, 2048, 4096, 8192, 65536]))
    if rng.random() < 0.5:
        pol["chunk_bytes"] = int(rng.choice([512, 4096, 16384, 262144]))
    if rng.random() < 0.5:
        pol["block"] = int(rng.choice([64, 128, 256, 512]))
    if rng.random() < 0.4:
        pol["unroll"] = int(rng.choice([1, 2, 4]))
    if rng.random() < 0.3:
        pol["workgroups"] = int(rng.integers(1, 65))
    if rng.random() < 0.3:
        pol["xcd_order"] = int(rng.integers(1, 3))
    if rng.random() < 0.2 and kind not in ("agv",):
        pol["datapath"] = 2  # the LDS-staged pipeline
        pol["block"] = 256
        pol["tile_bytes"] = 4096 * int(rng.integers(1, 4))
        pol.pop("chunk_bytes", None)
    if rng.random() < 0.25:  # resident workgroups per CU (LDS reservation at launch)
        pol["wgs_per_cu"] = int(rng.choice([-1, 3, 4, 5, 8, 16]))
    notify = ["none", "chunks", "check"][rng.integers(3)]
    if notify != "none":
        pol["notify_mode"] = 1 if notify == "chunks" else 2
    return kind, W, dtype, pol, notify


def _sizes(rng, kind, W):
    if kind in ("agv", "rsv"):
        parts = [16 * int(rng.integers(0, 700)) for _ in range(W)]
        if sum(parts) == 0:
            parts[0] = 16
        return sum(parts), parts
    large = rng.random() < 0.1  # now and then thousands of tiles (copies: runs of 2)
    per = 16 * int(rng.integers(1, 131072 if large else 3000))
    if kind in ("reduce_scattered", "alltoall", "ar_gather"):
        per = 16 * W * int(rng.integers(1, 16384 // W if large else 300))
    return per, None


@pytest.mark.parametrize("seed", range(200 * SCALE))
def test_fuzz(plr, oracle_mod, seed):
    rng = np.random.default_rng(1000 + seed)
    kind, W, dtype, pol, notify = _draw(rng)
    B, parts = _sizes(rng, kind, W)
    rank = int(rng.integers(W))
    what = f"seed={seed} kind={kind} W={W} dtype={dtype} B={B} parts={parts} rank={rank} pol={pol} notify={notify}"
    print(what, flush=True)
    eb = EB[dtype]
    if kind.startswith("reduce") or kind == "rsv":
        srcs_np = [synth.normal_np(seed, 10, w, B // eb, 1.0, dtype) for w in range(W)]
        if kind == "reduce_packed":
            L = plr.plr_layout_create("reduce", dtype, W, B, "packed", "packed", **pol)
            ref = oracle_mod.reduce_layout(dtype, "packed", 0, srcs_np)
        elif kind == "reduce_scattered":
            L = plr.plr_layout_create("reduce", dtype, W, B, "scattered", "packed", rank=rank, **pol)
            ref = oracle_mod.reduce_layout(dtype, "scattered", rank, srcs_np)
        else:
            L = plr.plr_layout_create("reduce", dtype, W, B, "scattered", "packed", rank=rank, part_bytes=parts,
                                      **pol)
            ref = oracle_mod.reduce_scatter_v(dtype, srcs_np, parts, rank)
        call = plr.plr_reduce
    else:
        if kind == "agv":
            srcs_np = [synth.bits_np(seed, 11, w, max(parts[w], 16)) for w in range(W)]
            L = plr.plr_layout_create("copy", dtype, W, B, "packed", "packed", part_bytes=parts, **pol)
            ref = oracle_mod.allgather_v(srcs_np, parts)
        else:
            pair = {"allgather": ("packed", "packed"), "alltoall": ("scattered", "transposed"),
                    "ar_gather": ("scattered", "scattered")}[kind]
            srcs_np = [synth.bits_np(seed, 11, w, B) for w in range(W)]
            L = plr.plr_layout_create("copy", dtype, W, B, *pair, **pol)
            ref = oracle_mod.copy_layout(*pair, srcs_np)
        call = plr.plr_copy
    srcs = [to_dev(s) for s in srcs_np]
    dst = empty_dev(L.dst_bytes, fill=0x5A)
    ws = None
    for epoch in range(2 if notify != "none" else 1):
        if notify != "none":
            if ws is None:
                ws = torch.zeros(max(L.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
            for w in rng.permutation(W):
                plr.plr_notify(L, int(w), ws)
        call(L, srcs, dst, ws)
        torch.cuda.synchronize()
        if ws is not None:
            assert plr.plr_check(L, ws) == plr.PLR_OK, what
        got = from_dev(dst)[:L.dst_bytes]
        if call is plr.plr_copy:
            assert np.array_equal(got, ref.view(np.uint8)), what
        else:
            assert_same(dtype, got, ref.view(np.uint8), what)
    if notify != "none":  # the same layout un-notified (its own launch shape where the policy gives one)
        dst2 = empty_dev(L.dst_bytes, fill=0xA5)
        call(L, srcs, dst2)
        torch.cuda.synchronize()
        got = from_dev(dst2)[:L.dst_bytes]
        if call is plr.plr_copy:
            assert np.array_equal(got, ref.view(np.uint8)), what + " un-notified"
        else:
            assert_same(dtype, got, ref.view(np.uint8), what + " un-notified")


@pytest.mark.parametrize("seed", range(40 * SCALE))
def test_fuzz_decode_shares(plr, oracle_mod, seed):
    """Reduce shares of at most 2 MiB per source with the policy's own launch shapes:
    notified calls and un-notified ones launch differently over 512 KiB per source, and
    both must give the oracle's bits, ragged ends included."""
    rng = np.random.default_rng(5000 + seed)
    W = int(rng.choice([1, 2, 3, 5, 8, 13, 16]))
    dtype = ["bf16", "f16", "f32"][rng.integers(3)]
    B = 16 * int(rng.integers(1, 131073))  # up to 2 MiB per source
    pol = {"workgroups": int(rng.integers(1, 300))} if rng.random() < 0.2 else {}
    what = f"seed={seed} W={W} dtype={dtype} B={B} pol={pol}"
    print(what, flush=True)
    srcs_np = [synth.normal_np(seed, 12, w, B // EB[dtype], 1.0, dtype) for w in range(W)]
    ref = oracle_mod.reduce(dtype, srcs_np)
    srcs = [to_dev(x) for x in srcs_np]
    L = plr.plr_layout_create("reduce", dtype, W, B, "packed", "packed", **pol)
    p = L.policy()
    assert (p["plain_tile_bytes"], p["plain_block"]) == ((min(4096, B), 256) if not pol or "workgroups" in pol
                                                         else (p["tile_bytes"], p["block"])), what
    ws = torch.zeros(max(L.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
    for notified in (False, True, False):
        dst = empty_dev(B, fill=0x5A)
        if notified:
            plr.plr_notify(L, -1, ws)
        plr.plr_reduce(L, srcs, dst, ws if notified else None)
        torch.cuda.synchronize()
        assert_same(dtype, from_dev(dst)[:B], ref.view(np.uint8), f"{what} notified={notified}")
    assert plr.plr_check(L, ws) == plr.PLR_OK, what


@pytest.mark.parametrize("seed", range(40 * SCALE))
def test_fuzz_copy_v(plr, oracle_mod, seed):
    """Variable-length AllToAll: random W, rows per source (empty ones included), row
    sizes (16 B to 20 KiB, ragged against the 2 KiB scatter tile) and destination skews."""
    rng = np.random.default_rng(5000 + seed)
    W = int(rng.choice([1, 2, 3, 5, 8, 13, 16]))
    rows = [int(rng.integers(0, 2500)) if rng.random() < 0.85 else 0 for _ in range(W)]
    rb = 16 * int(rng.choice([1, 3, 64, 128, 129, 896, 1280]))
    s = float(rng.choice([0.0, 0.5, 1.1, 3.0]))
    p = synth.zipf_weights(s, W)
    what = f"seed={seed} W={W} rows={rows} rb={rb} zipf={s}"
    print(what, flush=True)
    dests = [synth.categorical_np(seed, 12, w, rows[w], p) for w in range(W)]
    srcs_np = [synth.bits_np(seed, 13, w, max(rows[w], 1) * rb) for w in range(W)]
    srcs = [to_dev(x) for x in srcs_np]
    dd = [torch.from_numpy(d.copy()).cuda() if d.size else torch.zeros(4, dtype=torch.int32, device="cuda")
          for d in dests]
    total = sum(rows)
    dst = empty_dev(max(total * rb, 16), fill=0x5A)
    counts = torch.full((W * W,), -1, dtype=torch.int64, device="cuda")
    offsets = torch.full((W * W,), -1, dtype=torch.int64, device="cuda")
    scratch = torch.zeros(plr.plr_copy_v_scratch_bytes(W, rows), dtype=torch.uint8, device="cuda")
    plr.plr_copy_v(srcs, rows, dd, rb, dst, counts, offsets, scratch)
    torch.cuda.synchronize()
    ref, rc, ro = oracle_mod.copy_v(srcs_np, dests, rb)
    assert np.array_equal(counts.cpu().numpy().reshape(W, W), rc), what
    assert np.array_equal(offsets.cpu().numpy().reshape(W, W), ro), what
    assert np.array_equal(from_dev(dst)[:total * rb], ref), what


@pytest.mark.parametrize("seed", range(30 * SCALE))
def test_fuzz_allreduce(plr, oracle_mod, seed):
    """AllReduce into W outputs, fused and composed, random W, element type, size and tile."""
    rng = np.random.default_rng(7000 + seed)
    W = int(rng.choice([1, 2, 3, 4, 8, 16]))
    dtype = ["bf16", "f16", "f32"][rng.integers(3)]
    B = 16 * W * int(rng.integers(1, 400))
    path = [plr.PLR_PATH_DIRECT, plr.PLR_PATH_COMPOSED][rng.integers(2)]
    pol = {}
    if rng.random() < 0.6:
        pol["tile_bytes"] = int(rng.choice([256, 1024, 4096, 65536]))
    if rng.random() < 0.4:
        pol["block"] = int(rng.choice([64, 128, 256, 512]))
    what = f"seed={seed} W={W} dtype={dtype} B={B} path={path} pol={pol}"
    print(what, flush=True)
    eb = EB[dtype]
    srcs_np = [synth.normal_np(seed, 14, w, B // eb, 1.0, dtype) for w in range(W)]
    ref = oracle_mod.allreduce(dtype, srcs_np)
    if path == plr.PLR_PATH_COMPOSED and "tile_bytes" in pol:
        # composed calls must fit one round of workgroups (ntiles + 16 <= 256 CUs)
        slice_ = B // W
        tps = -(-slice_ // min(pol["tile_bytes"], slice_))
        if W * tps + 16 > 256:
            with pytest.raises(plr.PlrError) as e:
                plr.plr_layout_create("allreduce", dtype, W, B, "scattered", "scattered", datapath=path, **pol)
            assert e.value.code == plr.PLR_EUNSUPPORTED, what
            return
    L = plr.plr_layout_create("allreduce", dtype, W, B, "scattered", "scattered", datapath=path, **pol)
    ws = torch.zeros(max(L.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
    srcs = [to_dev(x) for x in srcs_np]
    dsts = [empty_dev(B, fill=0x5A) for _ in range(W)]
    for epoch in range(2):
        plr.plr_allreduce(L, srcs, dsts, ws)
        torch.cuda.synchronize()
        assert plr.plr_check(L, ws) == plr.PLR_OK, what
        for w in range(W):
            assert_same(dtype, from_dev(dsts[w])[:B], ref[w].view(np.uint8), f"{what} output {w} epoch {epoch}")
