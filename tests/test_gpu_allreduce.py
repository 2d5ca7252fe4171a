"""Parity of plr_allreduce (fused and composed datapaths, through the C ABI) with the
oracle: every one of the W outputs equals the rank-order reduction, bit for bit."""
import numpy as np
import pytest
import torch

import synth
from plrtest import NP_RAW, assert_same, empty_dev, from_dev, to_dev

pytestmark = pytest.mark.gpu
EB = {"bf16": 2, "f16": 2, "f32": 4}
PATHS = {"fused": 1, "composed": 3}


@pytest.fixture(scope="module")
def plr():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import reduce_atom_amd

    return reduce_atom_amd


def _run(plr, L, srcs, nbytes, W, calls=1):
    dsts = [empty_dev(nbytes, fill=0x3C) for _ in range(W)]
    ws = torch.zeros(max(L.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
    for _ in range(calls):
        plr.plr_allreduce(L, srcs, dsts, ws)
    torch.cuda.synchronize()
    assert plr.plr_check(L, ws) == plr.PLR_OK
    return dsts


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("W", [1, 2, 3, 8, 16])
def test_allreduce_small(plr, oracle_mod, path, dtype, W):
    nbytes = 16 * W * 211  # slices of 211 vectors: ragged against every tile size
    n = nbytes // EB[dtype]
    srcs_np = [synth.normal_np(W, 10, w, n, 1.0, dtype) for w in range(W)]
    refs = oracle_mod.allreduce(dtype, srcs_np)
    srcs = [to_dev(s) for s in srcs_np]
    for tile in (0, 256, 1024):
        L = plr.plr_layout_create("allreduce", dtype, W, nbytes, "scattered", "scattered",
                                  datapath=PATHS[path], tile_bytes=tile)
        dsts = _run(plr, L, srcs, nbytes, W, calls=2)
        for w in range(W):
            assert_same(dtype, from_dev(dsts[w])[:nbytes].view(NP_RAW[dtype]), refs[w], f"{path} W={W} t={tile} out {w}")


@pytest.mark.parametrize("path", list(PATHS))
def test_allreduce_prefill_share_full(plr, oracle_mod, path):
    """8 contributions of [8192, 7168] bf16 N(0, 0.5) into 8 outputs, default tiles (and,
    fused, the policy's 8 resident workgroups per CU): output 0 whole against the oracle,
    outputs 1..7 bitwise equal to output 0."""
    W, R, C = 8, 8192, 7168
    srcs = [synth.normal_t(0, 3, w, R * C, 0.5, device="cuda") for w in range(W)]
    dsts = [torch.full((R * C,), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    L = plr.plr_layout_create("allreduce", "bf16", W, R * C * 2, "scattered", "scattered", datapath=PATHS[path])
    assert L.policy()["wgs_per_cu"] == (8 if PATHS[path] == plr.PLR_PATH_DIRECT else 0)
    ws = torch.zeros(max(L.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
    plr.plr_allreduce(L, srcs, dsts, ws)
    torch.cuda.synchronize()
    assert plr.plr_check(L, ws) == plr.PLR_OK
    ref = oracle_mod.reduce("bf16", [s.view(torch.int16).cpu().numpy().view(np.uint16) for s in srcs],
                            threads=oracle_mod.default_threads())
    assert_same("bf16", dsts[0].view(torch.int16).cpu().numpy().view(np.uint16), ref, "out 0")
    for w in range(1, W):
        assert torch.equal(dsts[w].view(torch.int16), dsts[0].view(torch.int16)), f"out {w}"
