"""Buffers past 4 GiB: byte offsets and output positions that need 64-bit arithmetic
in every kernel path (reduce share, layout copy, row scatter). Inputs are generated on
the device in chunks by the counter-based generators; every output byte is checked
against the oracle (its threaded form), chunk by chunk for the reduce and the copy,
whole for the row scatter."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

CH = 1 << 28  # elements (or bytes) generated per device chunk


@pytest.fixture(scope="module")
def plr():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import reduce_atom_amd

    return reduce_atom_amd


def _host(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.uint8).cpu().numpy()


def test_reduce_share_past_4gib(plr, oracle_mod):
    W, n = 2, (9 << 30) // 4  # 2 x 4.5 GiB of bf16
    srcs = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    for w in range(W):
        for c0 in range(0, n, CH):
            m = min(CH, n - c0)
            srcs[w][c0:c0 + m] = synth.uniform_pm1_t(3, 40, w, m, start=c0, device="cuda")
    dst = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    L = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed")
    plr.plr_reduce(L, srcs, dst)
    torch.cuda.synchronize()
    T = oracle_mod.default_threads()
    for c0 in range(0, n, CH):  # every element, the 2^31 and 2^32 byte marks included
        m = min(CH, n - c0)
        host = [_host(srcs[w][c0:c0 + m]).view(np.uint16) for w in range(W)]
        got = _host(dst[c0:c0 + m]).view(np.uint16)
        assert np.array_equal(got, oracle_mod.reduce("bf16", host, threads=T)), f"elements from {c0}"
    del srcs, dst
    torch.cuda.empty_cache()


def test_allgather_past_4gib(plr, oracle_mod):
    W, B = 2, 5 << 29  # 2 x 2.5 GiB -> 5 GiB
    srcs = [torch.empty(B, dtype=torch.uint8, device="cuda") for _ in range(W)]
    for w in range(W):
        for c0 in range(0, B, CH):
            m = min(CH, B - c0)
            srcs[w][c0:c0 + m] = synth.bits_t(3, 41, w, m, start_byte=c0, device="cuda")
    L = plr.plr_layout_create("copy", "bf16", W, B, "packed", "packed")
    dst = torch.empty(L.dst_bytes, dtype=torch.uint8, device="cuda")
    plr.plr_copy(L, srcs, dst)
    torch.cuda.synchronize()
    T = oracle_mod.default_threads()
    for s in range(W):  # source s lands at bytes [s * B, (s + 1) * B) of the output
        for c0 in range(0, B, CH):
            m = min(CH, B - c0)
            ref = oracle_mod.copy([_host(srcs[s][c0:c0 + m])], [(0, 0, 0, m)], m, threads=T)
            assert np.array_equal(_host(dst[s * B + c0:s * B + c0 + m]), ref), f"source {s} bytes from {c0}"
    del srcs, dst
    torch.cuda.empty_cache()


def test_row_scatter_past_4gib(plr, oracle_mod):
    W, R, rb = 2, 200_000, 14336  # 2 x 2.87 GB of rows -> 5.7 GB packed output
    p = synth.zipf_weights(1.1, W)
    srcs = [torch.empty(R * rb, dtype=torch.uint8, device="cuda") for _ in range(W)]
    for w in range(W):
        for c0 in range(0, R * rb, CH):
            m = min(CH, R * rb - c0)
            srcs[w][c0:c0 + m] = synth.bits_t(3, 42, w, m, start_byte=c0, device="cuda")
    dests_np = [synth.categorical_np(3, 43, w, R, p) for w in range(W)]
    dests = [torch.from_numpy(d).cuda() for d in dests_np]
    dst = torch.empty(W * R * rb, dtype=torch.uint8, device="cuda")
    counts = torch.empty(W * W, dtype=torch.int64, device="cuda")
    offsets = torch.empty(W * W, dtype=torch.int64, device="cuda")
    scratch = torch.zeros(plr.plr_copy_v_scratch_bytes(W, [R] * W), dtype=torch.uint8, device="cuda")
    plr.plr_copy_v(srcs, [R] * W, dests, rb, dst, counts, offsets, scratch)
    torch.cuda.synchronize()
    ref, rc, ro = oracle_mod.copy_v([_host(x) for x in srcs], dests_np, rb, threads=oracle_mod.default_threads())
    assert np.array_equal(counts.cpu().numpy().reshape(W, W), rc)
    assert np.array_equal(offsets.cpu().numpy().reshape(W, W), ro)
    for c0 in range(0, ref.size, CH):  # every output byte, past the 2^32 byte mark included
        m = min(CH, ref.size - c0)
        assert np.array_equal(_host(dst[c0:c0 + m]), ref[c0:c0 + m]), f"output bytes from {c0}"
    del srcs, dst
    torch.cuda.empty_cache()
