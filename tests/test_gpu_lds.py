"""Parity of the LDS-staged datapath (PLR_PATH_LDS) with the oracle: the same results
as the direct path, bit for bit, for ragged sizes, long per-workgroup runs (the LDS ring
wraps many times), and notified calls."""
import numpy as np
import pytest
import torch

import synth
from plrtest import NP_RAW, assert_same, empty_dev, from_dev, to_dev

pytestmark = pytest.mark.gpu
EB = {"bf16": 2, "f16": 2, "f32": 4}
KINDS = {"allgather": ("packed", "packed"), "alltoall": ("scattered", "transposed"),
         "ar_gather": ("scattered", "scattered")}


@pytest.fixture(scope="module")
def plr():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import reduce_atom_amd

    return reduce_atom_amd


def _notified(plr, L, fn, srcs, dst):
    ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        plr.plr_notify(L, -1, ws)
        fn(L, srcs, dst, ws)
    assert plr.plr_check(L, ws) == plr.PLR_OK


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("W", [1, 2, 3, 5, 8, 16])
def test_reduce_lds(plr, oracle_mod, dtype, W):
    nbytes = 37 * 4096 + 48  # 38 slabs, the last one ragged
    n = nbytes // EB[dtype]
    raw = NP_RAW[dtype]
    srcs_np = [synth.normal_np(W, 8, w, n, 1.0, dtype) for w in range(W)]
    srcs_np[0][::17] = np.array([0x7FC0 if dtype == "bf16" else (0x7E00 if dtype == "f16" else 0x7FC00000)],
                                dtype=raw).view(srcs_np[0].dtype)[0]
    ref = oracle_mod.reduce(dtype, srcs_np)
    srcs = [to_dev(s) for s in srcs_np]
    for kw in (dict(), dict(workgroups=3), dict(workgroups=2, chunk_bytes=8192, notify=True),
               dict(tile_bytes=8192, workgroups=5, notify=True)):
        kw = dict(kw)
        notify = kw.pop("notify", False)
        L = plr.plr_layout_create("reduce", dtype, W, nbytes, "packed", "packed",
                                  datapath=plr.PLR_PATH_LDS, **kw)
        dst = empty_dev(nbytes, fill=0xA5)
        if notify:
            _notified(plr, L, plr.plr_reduce, srcs, dst)
        else:
            plr.plr_reduce(L, srcs, dst)
        torch.cuda.synchronize()
        assert_same(dtype, from_dev(dst)[:nbytes].view(raw), ref, f"{dtype} W={W} {kw} notify={notify}")


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("W", [1, 2, 3, 8, 9, 16])
def test_copy_lds(plr, oracle_mod, kind, W):
    B = 16 * W * 300  # segments not a multiple of 4 KiB: ragged slabs
    srcs_np = [synth.bits_np(W, 4, s, B) for s in range(W)]
    ref = oracle_mod.copy_layout(*KINDS[kind], srcs_np)
    srcs = [to_dev(s) for s in srcs_np]
    for kw in (dict(), dict(tile_bytes=4096, workgroups=3), dict(workgroups=4, chunk_bytes=4096, notify=True)):
        kw = dict(kw)
        notify = kw.pop("notify", False)
        L = plr.plr_layout_create("copy", "bf16", W, B, *KINDS[kind], datapath=plr.PLR_PATH_LDS, **kw)
        dst = empty_dev(L.dst_bytes, fill=0x5A)
        if notify:
            _notified(plr, L, plr.plr_copy, srcs, dst)
        else:
            plr.plr_copy(L, srcs, dst)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(dst)[:L.dst_bytes], ref), (kind, W, kw, notify)


def test_reduce_lds_prefill_share_full(plr, oracle_mod):
    """The prefill share (8 x [8192, 7168] bf16) on the LDS-staged path: every element
    against the oracle."""
    W, R, C = 8, 8192, 7168
    srcs = [synth.normal_t(0, 3, w, R * C, 0.5, device="cuda") for w in range(W)]
    dst = torch.full((R * C,), float("nan"), dtype=torch.bfloat16, device="cuda")
    L = plr.plr_layout_create("reduce", "bf16", W, R * C * 2, "packed", "packed", datapath=plr.PLR_PATH_LDS)
    plr.plr_reduce(L, srcs, dst)
    torch.cuda.synchronize()
    got = dst.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle_mod.reduce("bf16", [s.view(torch.int16).cpu().numpy().view(np.uint16) for s in srcs],
                            threads=oracle_mod.default_threads())
    assert_same("bf16", got, ref)


def test_copy_lds_alltoall_full(plr, oracle_mod):
    W, B = 8, 64 << 20
    srcs = [synth.bits_t(0, 4, s, B, device="cuda") for s in range(W)]
    L = plr.plr_layout_create("copy", "bf16", W, B, "scattered", "transposed", datapath=plr.PLR_PATH_LDS)
    dst = torch.empty(L.dst_bytes, dtype=torch.uint8, device="cuda")
    plr.plr_copy(L, srcs, dst)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), oracle_mod.copy_layout("scattered", "transposed",
                                                                     [s.cpu().numpy() for s in srcs]))
