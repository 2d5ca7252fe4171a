"""Oracle element formats, pinned to library conversions (numpy binary16, torch bfloat16)
and to the format definitions (bf16 is the upper half of a binary32 pattern)."""
import numpy as np
import torch

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _bf16_lib(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _is_nan_bf16(p):
    return ((p & 0x7F80) == 0x7F80) & ((p & 0x7F) != 0)


def _is_nan_f16(p):
    return ((p & 0x7C00) == 0x7C00) & ((p & 0x3FF) != 0)


def _tricky_f32():
    """Structured sample: every bf16 pattern's neighbourhood (ties and near-ties of
    bf16 rounding), every fp16 value's midpoints and their neighbours, random patterns,
    random values inside the fp16 range, and specials."""
    rng = np.random.default_rng(1)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    a = (hi[:, None] | lows[None, :]).reshape(-1)
    f16 = ALL16[~_is_nan_f16(ALL16) & ((ALL16 & 0x7C00) != 0x7C00)]
    v = f16.view(np.float16).astype(np.float64)
    v = np.sort(np.unique(v))
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)  # exact in binary32
    mb = mids.view(np.uint32)
    b = np.concatenate([mb, mb + 1, mb - 1])
    c = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    d = (np.exp2(rng.uniform(-26, 17, size=1 << 18)) * rng.choice([-1, 1], size=1 << 18)
         ).astype(np.float32).view(np.uint32)
    e = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001,
                  0x7F7FFFFF, 0x00000001, 0x807FFFFF, 0x477FF000, 0x477FEFFF], dtype=np.uint32)
    return np.concatenate([a, b, c, d, e]).view(np.float32)


def test_widen_bf16_is_upper_half_of_binary32(oracle_mod):
    got = oracle_mod.widen("bf16", ALL16)
    ref = (ALL16.astype(np.uint32) << 16).view(np.float32)
    nan = _is_nan_bf16(ALL16)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.isnan(got[nan]).all()
    lib = torch.from_numpy(ALL16.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(got[~nan].view(np.uint32), lib[~nan].view(np.uint32))


def test_widen_f16_matches_numpy(oracle_mod):
    got = oracle_mod.widen("f16", ALL16)
    ref = ALL16.view(np.float16).astype(np.float32)
    nan = _is_nan_f16(ALL16)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.isnan(got[nan]).all()


def test_narrow_f16_matches_numpy(oracle_mod):
    x = _tricky_f32()
    got = oracle_mod.narrow("f16", x)
    with np.errstate(over="ignore"):  # values past the fp16 range become infinities, as intended
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert _is_nan_f16(got[nan]).all()


def test_narrow_bf16_matches_torch(oracle_mod):
    x = _tricky_f32()
    got = oracle_mod.narrow("bf16", x)
    ref = _bf16_lib(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert _is_nan_bf16(got[nan]).all()


def test_round_trip_identity(oracle_mod):
    for dt, isnan in (("bf16", _is_nan_bf16), ("f16", _is_nan_f16)):
        keep = ALL16[~isnan(ALL16)]
        assert np.array_equal(oracle_mod.narrow(dt, oracle_mod.widen(dt, keep)), keep)


def test_narrow_f32_is_identity(oracle_mod):
    x = _tricky_f32()
    assert np.array_equal(oracle_mod.narrow("f32", x).view(np.uint32), x.view(np.uint32))


def test_binary32_add_keeps_subnormals(oracle_mod):
    tiny = np.array([1], dtype=np.uint32).view(np.float32)[0]
    r = np.float32(oracle_mod.add_f32(float(tiny), float(tiny)))
    assert r.view(np.uint32) == 2
