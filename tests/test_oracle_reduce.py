"""The oracle's ordered reduction, pinned to hand-derived vectors, closed forms,
exact-arithmetic regimes, permutation invariants and an independent straight-line
evaluation with numpy binary32 additions and library conversions."""
import itertools

import numpy as np
import pytest
import torch

from conftest import golden_lines

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _nan_mask(dtype, p):
    if dtype == "bf16":
        return ((p & 0x7F80) == 0x7F80) & ((p & 0x7F) != 0)
    if dtype == "f16":
        return ((p & 0x7C00) == 0x7C00) & ((p & 0x3FF) != 0)
    return np.isnan(p.view(np.float32))


def _same(dtype, got, ref):
    """Bitwise equality, NaN compared as a class."""
    g = got.view(np.uint32 if dtype == "f32" else np.uint16)
    r = ref.view(np.uint32 if dtype == "f32" else np.uint16)
    gn, rn = _nan_mask(dtype, got), _nan_mask(dtype, ref)
    return np.array_equal(gn, rn) and np.array_equal(g[~gn], r[~rn])


def _arr(dtype, words):
    if dtype == "f32":
        return np.array([int(w, 16) for w in words], dtype=np.uint32).view(np.float32)
    return np.array([int(w, 16) for w in words], dtype=np.uint16)


def test_golden_vectors(oracle_mod):
    n_checked = 0
    for line in golden_lines("reduce_vectors.txt"):
        lhs, rhs = line.split("->")
        dtype, *ins = lhs.split()
        srcs = [_arr(dtype, [w]) for w in ins]
        out = oracle_mod.reduce(dtype, srcs)
        if rhs.strip() == "nan":
            assert _nan_mask(dtype, out).all(), line
        else:
            assert _same(dtype, out, _arr(dtype, [rhs.strip()])), (line, out)
        n_checked += 1
    assert n_checked >= 25


# ---- independent evaluation: numpy binary32 adds + library conversions ----
def _widen_lib(dtype, bits):
    if dtype == "bf16":
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    return bits.view(np.float32)


def _narrow_lib(dtype, x32):
    if dtype == "bf16":
        return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return x32.astype(np.float16).view(np.uint16)
    return x32


def _straight_line(dtype, srcs):
    acc = _widen_lib(dtype, srcs[0]).astype(np.float32)
    with np.errstate(all="ignore"):
        for s in srcs[1:]:
            acc = (acc + _widen_lib(dtype, s)).astype(np.float32)
    return _narrow_lib(dtype, acc)


def _palette(dtype):
    if dtype == "bf16":
        vals = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80,
                0x7FC0, 0x3F80, 0xBF80, 0x3F81, 0x3B80, 0x2F80, 0x4B80, 0xCB80, 0x7B00, 0x7A80,
                0x3FC0, 0xBFC0, 0x4000, 0x3F7F, 0x0100, 0x80FF, 0x4780, 0xC780, 0x3C00, 0xBC00]
    elif dtype == "f16":
        vals = [0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF, 0x7C00, 0xFC00,
                0x7E00, 0x3C00, 0xBC00, 0x3C01, 0x1000, 0x1400, 0x4C00, 0x4800, 0x6400, 0xE400,
                0x3E00, 0xBE00, 0x4000, 0x3BFF, 0x0200, 0x83FF]
        return np.array(vals + list(np.random.default_rng(3).integers(0, 1 << 16, 38)), dtype=np.uint16)
    else:
        vals = [0, 0x80000000, 1, 0x80000001, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0xFF7FFFFF,
                0x7F800000, 0xFF800000, 0x7FC00000, 0x3F800000, 0xBF800000, 0x3F800001,
                0x33800000, 0x4B800000, 0xCB800000, 0x3FC00000, 0xBFC00000, 0x40000000]
        r = np.random.default_rng(4).integers(0, 1 << 32, 44, dtype=np.uint64).astype(np.uint32)
        return np.array(vals + list(r), dtype=np.uint32).view(np.float32)
    return np.array(vals + list(np.random.default_rng(2).integers(0, 1 << 16, 64 - len(vals))),
                    dtype=np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("W", [1, 2, 3])
@pytest.mark.parametrize("n", [8, 16, 24])
def test_brute_force_palette(oracle_mod, dtype, W, n):
    pal = _palette(dtype)
    rng = np.random.default_rng(W * 100 + n)
    for trial in range(40):
        srcs = [pal[rng.integers(0, pal.size, n)] for _ in range(W)]
        assert _same(dtype, oracle_mod.reduce(dtype, srcs), _straight_line(dtype, srcs))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_w1_identity_all_patterns(oracle_mod, dtype):
    assert _same(dtype, oracle_mod.reduce(dtype, [ALL16]), ALL16)


def test_x_plus_minus_x_is_positive_zero(oracle_mod):
    fin = ALL16[(ALL16 & 0x7F80) != 0x7F80]
    out = oracle_mod.reduce("bf16", [fin, fin ^ np.uint16(0x8000)])
    assert (out == 0).all()


@pytest.mark.parametrize("k", [1, 2, 3])
def test_power_of_two_copies_scale_exactly(oracle_mod, k):
    W = 1 << k
    rng = np.random.default_rng(k)
    x = rng.integers(0, 1 << 16, 4096).astype(np.uint16)
    x = x[((x & 0x7F80) != 0x7F80) & ((x & 0x7F80) < 0x7E00)]  # finite, no overflow
    out = oracle_mod.reduce("bf16", [x] * W)
    exact = _widen_lib("bf16", x).astype(np.float64) * W  # exact in binary32
    assert np.array_equal(out, _narrow_lib("bf16", exact.astype(np.float32)))


def _exact_regime_inputs(rng, W, n, lo_exp=-4, span=16):
    # bf16 values with exponents inside a window of `span` binades: every partial sum of
    # <= 8 of them fits in 24 bits, so binary32 accumulation is exact
    e = rng.integers(lo_exp, lo_exp + span - 4, size=(W, n))
    m = rng.integers(128, 256, size=(W, n))
    sgn = rng.choice([-1.0, 1.0], size=(W, n))
    vals = (sgn * m * np.exp2(e - 7)).astype(np.float32)
    return [_narrow_lib("bf16", v) for v in vals]


def test_exact_regime_is_single_rounding_of_the_real_sum(oracle_mod):
    rng = np.random.default_rng(11)
    srcs = _exact_regime_inputs(rng, 8, 4096)
    out = oracle_mod.reduce("bf16", srcs)
    exact = sum(_widen_lib("bf16", s).astype(np.float64) for s in srcs)
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)
    assert np.array_equal(out, _narrow_lib("bf16", exact.astype(np.float32)))


def test_exact_regime_permutation_invariant(oracle_mod):
    rng = np.random.default_rng(12)
    srcs = _exact_regime_inputs(rng, 8, 16)
    ref = oracle_mod.reduce("bf16", srcs)
    for perm in itertools.permutations(range(8)):
        assert np.array_equal(oracle_mod.reduce("bf16", [srcs[p] for p in perm]), ref)


def test_order_is_rank_order_not_sorted(oracle_mod):
    a, b, c = (np.array([v], dtype=np.uint16) for v in (0x4B80, 0x3F80, 0xCB80))
    assert oracle_mod.reduce("bf16", [a, b, c])[0] == 0x0000
    assert oracle_mod.reduce("bf16", [a, c, b])[0] == 0x3F80
    assert oracle_mod.reduce("bf16", [b, a, c])[0] == 0x0000  # 1 + 2^24 -> 2^24


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("W", [2, 4, 8])
def test_scattered_share_is_slice_rank(oracle_mod, dtype, W):
    rng = np.random.default_rng(W)
    per = 16 * W
    pal = _palette(dtype)
    srcs = [pal[rng.integers(0, pal.size, per)] for _ in range(W)]
    for rank in range(W):
        got = oracle_mod.reduce_layout(dtype, "scattered", rank, srcs)
        n = per // W
        ref = _straight_line(dtype, [s[rank * n:(rank + 1) * n] for s in srcs])
        assert _same(dtype, got, ref)
    got = oracle_mod.reduce_layout(dtype, "packed", 0, srcs)
    assert _same(dtype, got, _straight_line(dtype, srcs))


def test_random_configs_match_straight_line(oracle_mod):
    import synth

    for dtype in ("bf16", "f16", "f32"):
        srcs = [synth.normal_np(0, 2, w, 20000, 1.0, dtype) for w in range(8)]
        assert _same(dtype, oracle_mod.reduce(dtype, srcs), _straight_line(dtype, srcs))
    srcs = [synth.uniform_pm1_np(0, 1, w, 20000) for w in range(8)]
    assert _same("bf16", oracle_mod.reduce("bf16", srcs), _straight_line("bf16", srcs))
