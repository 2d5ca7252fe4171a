"""The datapath captured in a HIP graph: every replay, with the inputs changed by eager
work in between, matches the oracle (no memory-set nodes are recorded: the library's
calls are kernel launches only)."""
import numpy as np
import pytest
import torch

import synth
from plrtest import assert_same

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def plr():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import reduce_atom_amd

    return reduce_atom_amd


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def test_graph_replays_follow_inputs(plr, oracle_mod):
    W, n, B, R, rb = 8, 64 * 1024, 256 * 1024, 200, 256
    rsrc = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    rdst = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    Lr = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed")
    csrc = [torch.empty(B, dtype=torch.uint8, device="cuda") for _ in range(W)]
    Lc = plr.plr_layout_create("copy", "bf16", W, B, "scattered", "transposed")
    cdst = torch.empty(Lc.dst_bytes, dtype=torch.uint8, device="cuda")
    vsrc = [torch.empty(R * rb, dtype=torch.uint8, device="cuda") for _ in range(W)]
    vdest = [torch.empty(R, dtype=torch.int32, device="cuda") for _ in range(W)]
    vdst = torch.empty(W * R * rb, dtype=torch.uint8, device="cuda")
    cnt = torch.empty(W * W, dtype=torch.int64, device="cuda")
    off = torch.empty(W * W, dtype=torch.int64, device="cuda")
    scr = torch.zeros(plr.plr_copy_v_scratch_bytes(W, [R] * W), dtype=torch.uint8, device="cuda")
    La = plr.plr_layout_create("allreduce", "bf16", W, 2 * n, "scattered", "scattered")
    adst = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(W)]

    def calls():
        plr.plr_reduce(Lr, rsrc, rdst)
        plr.plr_copy(Lc, csrc, cdst)
        plr.plr_copy_v(vsrc, [R] * W, vdest, rb, vdst, cnt, off, scr)
        plr.plr_allreduce(La, rsrc, adst)

    g = _capture(calls)
    p = synth.zipf_weights(1.1, W)
    for replay in range(3):
        r_np = [synth.normal_np(replay, 2, w, n) for w in range(W)]
        c_np = [synth.bits_np(replay, 4, s, B) for s in range(W)]
        v_np = [synth.bits_np(replay, 6, s, R * rb) for s in range(W)]
        d_np = [synth.categorical_np(replay, 5, s, R, p) for s in range(W)]
        for t, a in zip(rsrc, r_np):  # eager work between replays
            t.copy_(torch.from_numpy(a.view(np.int16)).view(torch.bfloat16))
        for t, a in zip(csrc, c_np):
            t.copy_(torch.from_numpy(a))
        for t, a in zip(vsrc, v_np):
            t.copy_(torch.from_numpy(a))
        for t, a in zip(vdest, d_np):
            t.copy_(torch.from_numpy(a))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle_mod.reduce("bf16", r_np)
        assert_same("bf16", rdst.view(torch.int16).cpu().numpy().view(np.uint16), ref, f"reduce {replay}")
        for w in range(W):
            assert_same("bf16", adst[w].view(torch.int16).cpu().numpy().view(np.uint16), ref, f"allreduce {replay}")
        assert np.array_equal(cdst.cpu().numpy(), oracle_mod.copy_layout("scattered", "transposed", c_np))
        vref, vc, vo = oracle_mod.copy_v(v_np, d_np, rb)
        assert np.array_equal(vdst.cpu().numpy(), vref)
        assert np.array_equal(cnt.cpu().numpy().reshape(W, W), vc)
        assert np.array_equal(off.cpu().numpy().reshape(W, W), vo)
