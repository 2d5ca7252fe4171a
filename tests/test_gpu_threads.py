"""Distinct layouts used from distinct host threads, each on its own stream (the header
allows it): four threads run notified reduces, copies and variable-length copies
concurrently, each with its own timing events set and cleared, and every result matches
the oracle bit for bit."""
import threading

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def plr():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import reduce_atom_amd

    return reduce_atom_amd


def _worker(plr, oracle_mod, k, results):
    try:
        stream = torch.cuda.Stream()
        W, n, B, R, rb = 4 + k, 3 * 1024 * 16 + 16 * k, 16 * 1024 * (k + 1), 300 + k, 64
        rs_np = [synth.uniform_pm1_np(k, 50, w, n) for w in range(W)]
        cs_np = [synth.bits_np(k, 51, s, B) for s in range(W)]
        p = synth.zipf_weights(1.1, W)
        dn = [synth.categorical_np(k, 52, s, R, p) for s in range(W)]
        vs_np = [synth.bits_np(k, 53, s, R * rb) for s in range(W)]
        with torch.cuda.stream(stream):
            rs = [torch.from_numpy(a.view(np.int16).copy()).cuda().view(torch.bfloat16) for a in rs_np]
            rd = torch.empty(n, dtype=torch.bfloat16, device="cuda")
            Lr = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed", chunk_bytes=4096)
            ws = torch.zeros(Lr.workspace_bytes, dtype=torch.uint8, device="cuda")
            cs = [torch.from_numpy(a.copy()).cuda() for a in cs_np]
            Lc = plr.plr_layout_create("copy", "bf16", W, B, "packed", "packed")
            cd = torch.empty(Lc.dst_bytes, dtype=torch.uint8, device="cuda")
            vs = [torch.from_numpy(a.copy()).cuda() for a in vs_np]
            ds = [torch.from_numpy(d.copy()).cuda() for d in dn]
            vd = torch.empty(W * R * rb, dtype=torch.uint8, device="cuda")
            cnt = torch.empty(W * W, dtype=torch.int64, device="cuda")
            off = torch.empty(W * W, dtype=torch.int64, device="cuda")
            sc = torch.zeros(plr.plr_copy_v_scratch_bytes(W, [R] * W), dtype=torch.uint8, device="cuda")
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(20):
                plr.plr_notify(Lr, -1, ws)
                plr.plr_set_timing_events(*ev)
                plr.plr_reduce(Lr, rs, rd, ws)
                plr.plr_set_timing_events()
                plr.plr_copy(Lc, cs, cd)
                plr.plr_copy_v(vs, [R] * W, ds, rb, vd, cnt, off, sc)
            stream.synchronize()
            assert plr.plr_check(Lr, ws) == plr.PLR_OK
        ok = np.array_equal(rd.view(torch.int16).cpu().numpy().view(np.uint16), oracle_mod.reduce("bf16", rs_np))
        ok &= np.array_equal(cd.cpu().numpy(), oracle_mod.copy_layout("packed", "packed", cs_np))
        ref, rc, ro = oracle_mod.copy_v(vs_np, dn, rb)
        ok &= np.array_equal(vd.cpu().numpy(), ref) and np.array_equal(cnt.cpu().numpy().reshape(W, W), rc) \
            and np.array_equal(off.cpu().numpy().reshape(W, W), ro)
        results[k] = ok
    except Exception as e:  # noqa: BLE001  (reported by the main thread)
        results[k] = repr(e)


def test_four_threads_four_streams(plr, oracle_mod):
    results = {}
    threads = [threading.Thread(target=_worker, args=(plr, oracle_mod, k, results)) for k in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert all(not t.is_alive() for t in threads)
    assert results == {k: True for k in range(4)}, results
