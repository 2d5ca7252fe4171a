"""The allocation-free variable-length AllToAll (plr_copy_v_noalloc, scratch in the
library's fixed per-GPU array) against plr_copy_v with a caller-allocated scratch, bit
for bit, on calls in a row that shrink (the array keeps the last call's contents), in
both the small form (at most 256 segment counts) and the ticket form; both are also
checked against the oracle. The call captured in a HIP graph is replayed with new
inputs, eager calls on the same array in between."""
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


def _case(W, R, rb, seed):
    rows = [R - (s % 3) * 7 for s in range(W)]  # ragged sources
    p = synth.zipf_weights(1.1, W)
    srcs_np = [synth.bits_np(seed, 60, s, rows[s] * rb) for s in range(W)]
    dests_np = [synth.categorical_np(seed, 61, s, rows[s], p) for s in range(W)]
    return rows, srcs_np, dests_np


def _run(plr, noalloc, rows, srcs, dests, rb):
    W = len(srcs)
    total = sum(rows)
    dst = torch.full((total * rb,), 0x5A, dtype=torch.uint8, device="cuda")
    counts = torch.full((W * W,), -1, dtype=torch.int64, device="cuda")
    offsets = torch.full((W * W,), -1, dtype=torch.int64, device="cuda")
    if noalloc:
        plr.plr_copy_v_noalloc(srcs, rows, dests, rb, dst, counts, offsets)
    else:
        scratch = torch.zeros(plr.plr_copy_v_scratch_bytes(W, rows), dtype=torch.uint8, device="cuda")
        plr.plr_copy_v(srcs, rows, dests, rb, dst, counts, offsets, scratch)
    torch.cuda.synchronize()
    return dst.cpu().numpy(), counts.cpu().numpy().reshape(W, W), offsets.cpu().numpy().reshape(W, W)


# calls in a row on the one shared array, each with fewer rows (less scratch) than the
# one before it: (W, rows per source, row bytes) -- ticket form, small form, ticket
# form, small form
SEQUENCE = [(16, 3000, 2048), (8, 4096, 14336), (16, 1100, 64), (8, 1000, 1024)]


def test_noalloc_matches_copy_v_on_shrinking_calls(plr, oracle_mod):
    for k, (W, R, rb) in enumerate(SEQUENCE):
        rows, srcs_np, dests_np = _case(W, R, rb, seed=k)
        need = plr.plr_copy_v_scratch_bytes(W, rows)
        assert need <= plr.plr_copy_v_noalloc_max_scratch_bytes()
        srcs = [torch.from_numpy(s.copy()).cuda() for s in srcs_np]
        dests = [torch.from_numpy(d).cuda() for d in dests_np]
        want = _run(plr, False, rows, srcs, dests, rb)
        got = _run(plr, True, rows, srcs, dests, rb)
        for a, b, what in zip(got, want, ("rows", "counts", "offsets")):
            assert np.array_equal(a, b), f"call {k} (W={W}, R={R}, rb={rb}): {what}"
        ref = oracle_mod.copy_v(srcs_np, dests_np, rb, threads=oracle_mod.default_threads())
        for a, b, what in zip(got, ref, ("rows", "counts", "offsets")):
            assert np.array_equal(a, b), f"call {k} against the oracle: {what}"


def test_noalloc_twice_in_a_row_second_smaller(plr, oracle_mod):
    """The bench's shape, then a smaller call of the same form, back to back on one
    stream with no synchronisation between them."""
    W, rb = 8, 14336
    outs = []
    cases = [_case(W, 4096, rb, seed=20), _case(W, 1500, rb, seed=21)]
    for rows, srcs_np, dests_np in cases:
        srcs = [torch.from_numpy(s.copy()).cuda() for s in srcs_np]
        dests = [torch.from_numpy(d).cuda() for d in dests_np]
        dst = torch.empty(sum(rows) * rb, dtype=torch.uint8, device="cuda")
        counts = torch.empty(W * W, dtype=torch.int64, device="cuda")
        offsets = torch.empty(W * W, dtype=torch.int64, device="cuda")
        plr.plr_copy_v_noalloc(srcs, rows, dests, rb, dst, counts, offsets)
        outs.append((dst, counts, offsets, srcs, dests))
    torch.cuda.synchronize()
    for (rows, srcs_np, dests_np), (dst, counts, offsets, srcs, dests) in zip(cases, outs):
        want = _run(plr, False, rows, srcs, dests, rb)
        got = (dst.cpu().numpy(), counts.cpu().numpy().reshape(W, W), offsets.cpu().numpy().reshape(W, W))
        for a, b in zip(got, want):
            assert np.array_equal(a, b)


def test_noalloc_rejects_requests_beyond_its_scratch(plr):
    W = 2
    rows = [plr.plr_copy_v_noalloc_max_scratch_bytes() // 4, 16]
    src = torch.empty(16, dtype=torch.uint8, device="cuda")
    dest = torch.zeros(16, dtype=torch.int32, device="cuda")
    # raw addresses: the library itself must refuse the request before it reads anything
    # (tensors this small would already be refused by the binding's size checks)
    s, d = src.data_ptr(), dest.data_ptr()
    with pytest.raises(plr.PlrError) as e:
        plr.plr_copy_v_noalloc([s, s], rows, [d, d], 16, s, s, s)
    assert e.value.code == plr.PLR_ETOOLARGE


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


@pytest.mark.parametrize("W,R,rb", [(16, 1100, 64), (8, 1000, 1024)], ids=["ticket_form", "small_form"])
def test_noalloc_replayed_from_a_graph(plr, oracle_mod, W, R, rb):
    """The callers it is for: the call captured in a HIP graph (it allocates nothing and
    records kernel launches only), replayed three times with new inputs written by eager
    work in between and an eager call of another size on the same array before each
    replay; every replay matches the oracle."""
    rows = [R - (s % 3) * 7 for s in range(W)]
    p = synth.zipf_weights(1.1, W)
    srcs = [torch.empty(rows[s] * rb, dtype=torch.uint8, device="cuda") for s in range(W)]
    dests = [torch.empty(rows[s], dtype=torch.int32, device="cuda") for s in range(W)]
    dst = torch.empty(sum(rows) * rb, dtype=torch.uint8, device="cuda")
    counts = torch.empty(W * W, dtype=torch.int64, device="cuda")
    offsets = torch.empty(W * W, dtype=torch.int64, device="cuda")
    o_rows, o_srcs_np, o_dests_np = _case(4, 700, 32, seed=90)  # the other call's shape
    o_srcs = [torch.from_numpy(s.copy()).cuda() for s in o_srcs_np]
    o_dests = [torch.from_numpy(d).cuda() for d in o_dests_np]
    _run(plr, True, o_rows, o_srcs, o_dests, 32)  # an eager call first, as before any capture
    g = _capture(lambda: plr.plr_copy_v_noalloc(srcs, rows, dests, rb, dst, counts, offsets))
    for replay in range(3):
        srcs_np = [synth.bits_np(70 + replay, 62, s, rows[s] * rb) for s in range(W)]
        dests_np = [synth.categorical_np(70 + replay, 63, s, rows[s], p) for s in range(W)]
        for t, a in zip(srcs, srcs_np):
            t.copy_(torch.from_numpy(a))
        for t, a in zip(dests, dests_np):
            t.copy_(torch.from_numpy(a))
        other = _run(plr, True, o_rows, o_srcs, o_dests, 32)
        g.replay()
        torch.cuda.synchronize()
        ref = oracle_mod.copy_v(srcs_np, dests_np, rb)
        got = (dst.cpu().numpy(), counts.cpu().numpy().reshape(W, W), offsets.cpu().numpy().reshape(W, W))
        for a, b, what in zip(got, ref, ("rows", "counts", "offsets")):
            assert np.array_equal(a, b), f"replay {replay}: {what}"
        o_ref = oracle_mod.copy_v(o_srcs_np, o_dests_np, 32)
        for a, b, what in zip(other, o_ref, ("rows", "counts", "offsets")):
            assert np.array_equal(a, b), f"eager call before replay {replay}: {what}"
