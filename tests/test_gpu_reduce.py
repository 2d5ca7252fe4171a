"""Parity of plr_reduce (HIP, through the C ABI) with the oracle: bit-exact, NaN as a class."""
import numpy as np
import pytest
import torch

import synth
from plrtest import assert_same, empty_dev, from_dev, to_dev, NP_RAW

pytestmark = pytest.mark.gpu
EB = {"bf16": 2, "f16": 2, "f32": 4}


@pytest.fixture(scope="module")
def plr():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import reduce_atom_amd

    return reduce_atom_amd


def _mixed(dtype, W, n, seed):
    """Normal values with a sprinkling of specials (zeros, subnormals, max, inf, NaN)."""
    srcs = [synth.normal_np(seed, 9, w, n, 1.0, dtype).copy() for w in range(W)]
    raw = NP_RAW[dtype]
    if dtype == "f32":
        sp = np.array([0, 0x80000000, 1, 0x807FFFFF, 0x7F7FFFFF, 0x7F800000, 0xFF800000, 0x7FC00000],
                      dtype=np.uint32).view(np.float32)
    elif dtype == "bf16":
        sp = np.array([0, 0x8000, 1, 0x807F, 0x7F7F, 0x7F80, 0xFF80, 0x7FC0], dtype=np.uint16)
    else:
        sp = np.array([0, 0x8000, 1, 0x83FF, 0x7BFF, 0x7C00, 0xFC00, 0x7E00], dtype=np.uint16)
    rng = np.random.default_rng(seed)
    for s in srcs:
        idx = rng.integers(0, n, max(1, n // 97))
        s[idx] = sp[rng.integers(0, sp.size, idx.size)]
    return srcs


def _run(plr, L, srcs_np, dst_bytes, workspace=False, notify=True):
    srcs = [to_dev(s) for s in srcs_np]
    dst = empty_dev(dst_bytes, fill=0xA5)
    ws = None
    if workspace:
        ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device="cuda")
        if notify:
            plr.plr_notify(L, -1, ws)
    plr.plr_reduce(L, srcs, dst, ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert plr.plr_check(L, ws) == plr.PLR_OK
    return dst


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("W", [1, 2, 3, 5, 8, 16])
def test_small_ragged(plr, oracle_mod, dtype, W):
    # several chunks of 4 KiB plus a ragged tail (one 16-byte vector past a chunk edge)
    nbytes = 3 * 4096 + 3 * 256 + 16
    n = nbytes // EB[dtype]
    srcs = _mixed(dtype, W, n, seed=W)
    ref = oracle_mod.reduce(dtype, srcs)
    for kw in (dict(), dict(chunk_bytes=4096), dict(chunk_bytes=4096, workgroups=2, block=64, unroll=4)):
        L = plr.plr_layout_create("reduce", dtype, W, nbytes, "packed", "packed", **kw)
        out = _run(plr, L, srcs, nbytes)
        assert_same(dtype, from_dev(out)[:nbytes].view(NP_RAW[dtype]), ref, f"{dtype} W={W} {kw}")


@pytest.mark.parametrize("block", [64, 128, 256, 512])
@pytest.mark.parametrize("unroll", [1, 2, 4])
def test_launch_shapes(plr, oracle_mod, block, unroll):
    W, nbytes = 8, (1 << 18) + 4096 + 48
    n = nbytes // 2
    srcs = [synth.uniform_pm1_np(3, 1, w, n) for w in range(W)]
    ref = oracle_mod.reduce("bf16", srcs)
    for chunk, wg in ((8192, 0), (65536, 3), (1 << 20, 0)):
        L = plr.plr_layout_create("reduce", "bf16", W, nbytes, "packed", "packed", chunk_bytes=chunk,
                                  workgroups=wg, block=block, unroll=unroll)
        out = _run(plr, L, srcs, nbytes)
        assert_same("bf16", from_dev(out).view(np.uint16)[:n], ref, f"b{block} u{unroll} c{chunk}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_rounding_ties_and_overflow(plr, oracle_mod, dtype):
    """x + y with y a half-ulp (and near it) of x for every 16-bit pattern x: exercises
    every tie, carry into the exponent, overflow to infinity and subnormal rounding."""
    allp = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = oracle_mod.widen(dtype, allp).astype(np.float64)
    frac = 7 if dtype == "bf16" else 10
    e = np.floor(np.log2(np.where(np.isfinite(x) & (x != 0), np.abs(x), 1.0)))
    half = np.exp2(e - frac - 1) * np.sign(np.where(np.isfinite(x), x, 0))
    xs, ys = [], []
    for k in (1.0, 1.5, 0.75, -1.0, 3.0):
        y = oracle_mod.narrow(dtype, (half * k).astype(np.float32))
        xs.append(allp)
        ys.append(y)
    xs, ys = np.concatenate(xs), np.concatenate(ys)
    pad = (-xs.size) % 8
    xs = np.concatenate([xs, np.zeros(pad, np.uint16)])
    ys = np.concatenate([ys, np.zeros(pad, np.uint16)])
    ref = oracle_mod.reduce(dtype, [xs, ys])
    L = plr.plr_layout_create("reduce", dtype, 2, xs.nbytes, "packed", "packed")
    out = _run(plr, L, [xs, ys], xs.nbytes)
    assert_same(dtype, from_dev(out).view(np.uint16)[:xs.size], ref, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_random_patterns_w3(plr, oracle_mod, dtype):
    """Uniformly random bit patterns: every exponent, NaN payloads, infinities."""
    n = 1 << 20
    raw = NP_RAW[dtype]
    srcs = [synth.bits_np(5, 7, w, n * EB[dtype]).view(raw) for w in range(3)]
    ref = oracle_mod.reduce(dtype, srcs)
    L = plr.plr_layout_create("reduce", dtype, 3, n * EB[dtype], "packed", "packed")
    out = _run(plr, L, srcs, n * EB[dtype])
    assert_same(dtype, from_dev(out).view(raw), ref, dtype)


@pytest.mark.parametrize("W", [2, 4, 8])
def test_scattered_share_every_rank(plr, oracle_mod, W):
    per = 16 * W * 300
    n = per // 2
    srcs = _mixed("bf16", W, n, seed=40 + W)
    for rank in range(W):
        ref = oracle_mod.reduce_layout("bf16", "scattered", rank, srcs)
        L = plr.plr_layout_create("reduce", "bf16", W, per, "scattered", "packed", rank=rank,
                                  chunk_bytes=1024)
        out = _run(plr, L, srcs, L.dst_bytes)
        assert_same("bf16", from_dev(out).view(np.uint16)[:ref.size], ref, f"rank {rank}")


def test_explicit_source_offsets(plr, oracle_mod):
    W, n = 4, 4096
    srcs = [synth.normal_np(1, 2, w, 3 * n) for w in range(W)]
    offs = [0, n, 2 * n, 16]
    ref = oracle_mod.reduce("bf16", srcs, src_off=offs, n=n)
    L = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed",
                              in_offsets=[2 * o for o in offs])
    out = _run(plr, L, srcs, 2 * n)
    assert_same("bf16", from_dev(out).view(np.uint16)[:n], ref)


def test_config1_local_reduce(plr, oracle_mod):
    """8 contributions of 1,048,576 bf16, uniform[-1, 1]: the whole output."""
    W, n = 8, 1 << 20
    srcs = [synth.uniform_pm1_np(0, 1, w, n) for w in range(W)]
    ref = oracle_mod.reduce("bf16", srcs)
    L = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed")
    assert_same("bf16", from_dev(_run(plr, L, srcs, 2 * n)).view(np.uint16), ref)
    L2 = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed")
    assert_same("bf16", from_dev(_run(plr, L2, srcs, 2 * n, workspace=True)).view(np.uint16), ref)


@pytest.mark.parametrize("T", [1, 8, 32, 37, 64, 128])
def test_config2_decode_share(plr, oracle_mod, T):
    """8 contributions of [T, 7168] bf16, N(0, 1): the whole output, notify off and on.
    From T = 37 (over 512 KiB per source) the two launch with different tiles and
    workgroups (8 KiB of 512 threads notified, 4 KiB of 256 not); odd T leave a ragged
    last tile in both."""
    W, n = 8, T * 7168
    srcs = [synth.normal_np(0, 2, w, n, 1.0) for w in range(W)]
    ref = oracle_mod.reduce("bf16", srcs)
    pol = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed").policy()
    assert (pol["tile_bytes"] != pol["plain_tile_bytes"]) == (T >= 37)
    for ws in (False, True):
        L = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed")
        assert_same("bf16", from_dev(_run(plr, L, srcs, 2 * n, workspace=ws)).view(np.uint16), ref,
                    f"T={T} ws={ws}")


@pytest.mark.parametrize("notified", [False, True])
def test_config3_prefill_share_full(plr, oracle_mod, notified):
    """8 contributions of [8192, 7168] bf16, N(0, 0.5), at full size with the default
    policy, un-notified and in the bench's launch configuration (notified, check mode):
    all 58,720,256 output elements against the oracle (its threaded form, the same
    per-element code on every host core). The output starts as NaN, so an element the
    grid skipped cannot pass."""
    W, R, C = 8, 8192, 7168
    srcs = [synth.normal_t(0, 3, w, R * C, 0.5, device="cuda") for w in range(W)]
    dst = torch.full((R * C,), float("nan"), dtype=torch.bfloat16, device="cuda")
    L = plr.plr_layout_create("reduce", "bf16", W, R * C * 2, "packed", "packed")
    ws = None
    if notified:
        assert L.policy()["notify_mode"] == plr.PLR_NOTIFY_CHECK
        ws = torch.zeros(L.workspace_bytes, dtype=torch.uint8, device="cuda")
        plr.plr_notify(L, -1, ws)
    plr.plr_reduce(L, srcs, dst, ws)
    torch.cuda.synchronize()
    if notified:
        assert plr.plr_check(L, ws) == plr.PLR_OK
        words = ws[:24].view(torch.int64).cpu().numpy()
        assert words[1] == 1 and words[2] == 0  # every flag was set at check time: no waits
    got = dst.view(torch.int16).cpu().numpy().view(np.uint16)
    host = [s.view(torch.int16).cpu().numpy().view(np.uint16) for s in srcs]
    ref = oracle_mod.reduce("bf16", host, threads=oracle_mod.default_threads())
    assert_same("bf16", got, ref)


@pytest.mark.parametrize("cap", [-1, 3, 5, 16])
def test_resident_workgroup_caps(plr, oracle_mod, cap):
    """The launch's LDS reservation only bounds how many workgroups share a compute unit:
    a reduce of 8 x 6 MiB (ragged: not a whole number of tiles), notified and not, a copy
    and a fused AllReduce under each cap give the oracle's bits."""
    W, n = 8, 3 * (1 << 20) + 2 * 72
    srcs_np = [synth.normal_np(7, 30, w, n, 1.0) for w in range(W)]
    ref = oracle_mod.reduce("bf16", srcs_np, threads=oracle_mod.default_threads())
    for ws in (False, True):
        L = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed", wgs_per_cu=cap)
        assert L.policy()["wgs_per_cu"] == (0 if cap == -1 else cap)
        assert_same("bf16", from_dev(_run(plr, L, srcs_np, 2 * n, workspace=ws)).view(np.uint16), ref,
                    f"reduce cap {cap} ws {ws}")
    B = 4 << 20
    csrcs = [synth.bits_np(7, 31, s, B) for s in range(W)]
    C = plr.plr_layout_create("copy", "bf16", W, B, "scattered", "transposed", wgs_per_cu=cap)
    cdst = torch.empty(C.dst_bytes, dtype=torch.uint8, device="cuda")
    plr.plr_copy(C, [to_dev(x) for x in csrcs], cdst)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(cdst), oracle_mod.copy_layout("scattered", "transposed", csrcs)), f"copy {cap}"
    m = W * 16384
    asrcs_np = [synth.normal_np(7, 32, w, m, 1.0) for w in range(W)]
    A = plr.plr_layout_create("allreduce", "bf16", W, 2 * m, "scattered", "scattered", wgs_per_cu=cap)
    adst = [torch.empty(m, dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    plr.plr_allreduce(A, [to_dev(x) for x in asrcs_np], adst)
    torch.cuda.synchronize()
    aref = oracle_mod.reduce("bf16", asrcs_np)
    for w in range(W):
        assert_same("bf16", adst[w].view(torch.int16).cpu().numpy().view(np.uint16), aref, f"allreduce {cap} out {w}")


def test_repeatable_bits(plr):
    W, n = 8, (1 << 20) + 8
    srcs = [synth.normal_t(0, 4, w, n, 1.0, device="cuda") for w in range(W)]
    L = plr.plr_layout_create("reduce", "bf16", W, 2 * n, "packed", "packed")
    first = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    plr.plr_reduce(L, srcs, first)
    for _ in range(10):
        again = torch.full((n,), float("nan"), dtype=torch.bfloat16, device="cuda")
        plr.plr_reduce(L, srcs, again)
        assert torch.equal(first.view(torch.int16), again.view(torch.int16))


def test_empty_share_is_a_no_op(plr):
    L = plr.plr_layout_create("reduce", "bf16", 4, 0, "packed", "packed")
    x = torch.zeros(16, dtype=torch.uint8, device="cuda")
    plr.plr_reduce(L, [x, x, x, x], torch.zeros(16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
