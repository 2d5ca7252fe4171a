"""Buffers past 4 GiB: byte offsets and output positions that need 64-bit arithmetic
in every kernel path (reduce share, layout copy, row scatter). Inputs are generated on
the device in chunks by the counter-based generators, so any element can be generated
again on the host from its index alone; outputs are checked against the oracle at
sampled positions, including the first and last elements and the 2^31 and 2^32 byte
boundaries."""
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


def _positions(rng, n, unit, extra=()):
    """Sorted distinct element positions in [0, n): random ones plus the ends and the
    elements at and around the 2^31 and 2^32 byte marks."""
    marks = [0, 1, n - 2, n - 1, *extra]
    for b in (1 << 31, 1 << 32):
        e = b // unit
        marks += [e - 1, e, e + 1]
    p = np.concatenate([rng.integers(0, n, 3000), np.asarray(marks, dtype=np.int64)])
    return np.unique(p[(p >= 0) & (p < n)])


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
    pos = _positions(np.random.default_rng(0), n, 2)
    got = dst[torch.from_numpy(pos).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    host = [np.array([synth.uniform_pm1_np(3, 40, w, 1, start=int(i))[0] for i in pos], np.uint16) for w in range(W)]
    assert np.array_equal(got, oracle_mod.reduce("bf16", host))
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
    vec = _positions(np.random.default_rng(1), W * B // 16, 16, extra=(B // 16 - 1, B // 16))
    got = dst.view(-1, 16)[torch.from_numpy(vec).cuda()].cpu().numpy()
    segs = [(s, 0, s * B, B) for s in range(W)]
    for k, v in enumerate(vec):
        off = int(v) * 16
        s, so = next((s, off - d0 + so) for s, so, d0, ln in segs if d0 <= off < d0 + ln)
        assert np.array_equal(got[k], synth.bits_np(3, 41, s, 16, start_byte=so)), off
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
    # counts, offsets and where every row lands, from the oracle run on 16-byte stand-in
    # rows that carry their own (source, row) tag (placement does not depend on the bytes)
    tags = [np.stack([np.full(R, s, np.int64), np.arange(R, dtype=np.int64)], 1).view(np.uint8).reshape(-1)
            for s in range(W)]
    placed, rc, ro = oracle_mod.copy_v(tags, dests_np, 16)
    assert np.array_equal(counts.cpu().numpy().reshape(W, W), rc)
    assert np.array_equal(offsets.cpu().numpy().reshape(W, W), ro)
    out_row = placed.view(np.int64).reshape(-1, 2)
    rows = _positions(np.random.default_rng(2), W * R, rb)
    got = dst.view(-1, rb)[torch.from_numpy(rows).cuda()].cpu().numpy()
    for k, r in enumerate(rows):
        s, i = (int(v) for v in out_row[int(r)])
        assert np.array_equal(got[k], synth.bits_np(3, 42, s, rb, start_byte=i * rb)), int(r)
    del srcs, dst
    torch.cuda.empty_cache()
