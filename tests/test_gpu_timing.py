"""plr_set_timing_events: the caller's event pair brackets a call's datapath kernels
(not the check kernel of a notified call) and leaves the results unchanged."""
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


def _pair():
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def test_timed_reduce_and_copy_v(plr, oracle_mod):
    W, n = 8, 1 << 20
    srcs_np = [synth.normal_np(21, 2, w, n) for w in range(W)]
    ref = oracle_mod.reduce("bf16", srcs_np)
    srcs = [to_dev(s) for s in srcs_np]
    L = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed")
    ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(2 * n, dtype=torch.uint8, device="cuda")
    times = []
    for notified in (False, True):
        a, b = _pair()
        plr.plr_set_timing_events(a, b)
        if notified:
            plr.plr_notify(L, -1, ws)
        plr.plr_reduce(L, srcs, dst, ws if notified else None)
        plr.plr_set_timing_events()
        b.synchronize()
        times.append(a.elapsed_time(b))
        assert_same("bf16", dst.cpu().numpy().view(np.uint16), ref)
    assert plr.plr_check(L, ws) == plr.PLR_OK
    # 18 MiB of HBM traffic: more than 1 us, far less than a second
    assert all(1e-3 < t < 1e3 for t in times), times

    R, rb = 2000, 1024
    p = synth.zipf_weights(1.1, W)
    dests_np = [synth.categorical_np(21, 5, s, R, p) for s in range(W)]
    vs_np = [synth.bits_np(21, 6, s, R * rb) for s in range(W)]
    vs = [to_dev(v) for v in vs_np]
    dests = [torch.from_numpy(d.copy()).cuda() for d in dests_np]
    out = torch.empty(W * R * rb, dtype=torch.uint8, device="cuda")
    counts = torch.empty(W * W, dtype=torch.int64, device="cuda")
    offsets = torch.empty(W * W, dtype=torch.int64, device="cuda")
    scratch = torch.zeros(plr.plr_copy_v_scratch_bytes(W, [R] * W), dtype=torch.uint8, device="cuda")
    a, b = _pair()
    plr.plr_set_timing_events(a, b)
    plr.plr_copy_v(vs, [R] * W, dests, rb, out, counts, offsets, scratch)
    plr.plr_set_timing_events()
    b.synchronize()
    assert 1e-3 < a.elapsed_time(b) < 1e3
    ref_out, _, _ = oracle_mod.copy_v(vs_np, dests_np, rb)
    assert np.array_equal(out.cpu().numpy(), ref_out)


def test_one_sided_events_rejected(plr):
    a, _ = _pair()
    a.record()
    import ctypes
    assert plr._lib.plr_set_timing_events(ctypes.c_void_p(a.cuda_event), None) == plr.PLR_EINVAL
    assert plr._lib.plr_set_timing_events(None, None) == plr.PLR_OK


def test_split_events_time_each_kernel(plr, oracle_mod):
    """The four-event form: a two-kernel call (AllToAllV) carries one pair on each of
    its kernels, which lie in order inside the whole call; a one-kernel call carries the
    outer pair only. Results are unchanged."""
    from bench import TimingEvents

    E = TimingEvents(torch)
    ev = [E.create() for _ in range(4)]
    W, R, rb = 8, 3000, 2048
    p = synth.zipf_weights(1.1, W)
    dests_np = [synth.categorical_np(22, 5, s, R, p) for s in range(W)]
    vs_np = [synth.bits_np(22, 6, s, R * rb) for s in range(W)]
    vs = [to_dev(v) for v in vs_np]
    dests = [torch.from_numpy(d.copy()).cuda() for d in dests_np]
    out = torch.empty(W * R * rb, dtype=torch.uint8, device="cuda")
    counts = torch.empty(W * W, dtype=torch.int64, device="cuda")
    offsets = torch.empty(W * W, dtype=torch.int64, device="cuda")
    scratch = torch.zeros(plr.plr_copy_v_scratch_bytes(W, [R] * W), dtype=torch.uint8, device="cuda")
    plr.plr_set_timing_events_split(*ev)
    plr.plr_copy_v(vs, [R] * W, dests, rb, out, counts, offsets, scratch)
    plr.plr_set_timing_events_split()
    torch.cuda.synchronize()
    first, second, whole = E.elapsed_ms(ev[0], ev[1]), E.elapsed_ms(ev[2], ev[3]), E.elapsed_ms(ev[0], ev[3])
    assert 0 < first and 0 < second and first + second <= whole * 1.001 + 1e-3, (first, second, whole)
    assert E.elapsed_ms(ev[1], ev[2]) >= 0  # the second kernel starts after the first ends
    ref_out, _, _ = oracle_mod.copy_v(vs_np, dests_np, rb)
    assert np.array_equal(out.cpu().numpy(), ref_out)

    ev2 = [E.create() for _ in range(4)]
    n = 1 << 20
    srcs_np = [synth.normal_np(22, 2, w, n) for w in range(W)]
    L = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed")
    dst = torch.empty(2 * n, dtype=torch.uint8, device="cuda")
    plr.plr_set_timing_events_split(*ev2)
    plr.plr_reduce(L, [to_dev(s) for s in srcs_np], dst)
    plr.plr_set_timing_events_split()
    torch.cuda.synchronize()
    assert 1e-3 < E.elapsed_ms(ev2[0], ev2[3]) < 1e3
    assert_same("bf16", dst.cpu().numpy().view(np.uint16), oracle_mod.reduce("bf16", srcs_np))
    E.destroy_all()


def test_split_events_all_or_none(plr):
    import ctypes

    a, _ = _pair()
    a.record()
    h = ctypes.c_void_p(a.cuda_event)
    for k in range(1, 4):
        args = [h] * k + [None] * (4 - k)
        assert plr._lib.plr_set_timing_events_split(*args) == plr.PLR_EINVAL
    assert plr._lib.plr_set_timing_events_split(None, None, None, None) == plr.PLR_OK
