"""The oracle's threaded variants (used to compare full-size GPU outputs in seconds and
to time the oracle on every host core) against its single-threaded functions, which
the other oracle tests pin to the pages and to the mathematics. Splitting the work
over threads must change no bit: random bit patterns (NaN payloads, infinities,
subnormals included), ragged lengths, more threads than elements, scattered shares,
every copy layout and random variable-length rows."""
import numpy as np
import pytest

import synth

THREADS = (2, 3, 8, 17)
RAW = {"bf16": np.uint16, "f16": np.uint16, "f32": np.uint32}


def _bits(dtype, seed, buf, n):
    """n elements of random bit patterns (every class of value appears)."""
    eb = 4 if dtype == "f32" else 2
    nb = (n * eb + 15) // 16 * 16
    return synth.bits_np(seed, 90, buf, max(16, nb))[: n * eb].view(RAW[dtype])


def _special(dtype, seed, buf, n):
    """n elements drawn from a palette of special values and near-ties."""
    if dtype == "f32":
        pal = np.array([0, 0x80000000, 1, 0x80000001, 0x007FFFFF, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000,
                        0xFF800000, 0x7FC00000, 0x3F800000, 0x33800000, 0x3F800001, 0xBF800000],
                       dtype=np.uint32)
    else:
        pal = np.array([0, 0x8000, 1, 0x8001, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0, 0x3F80, 0x3B80,
                        0x3F81, 0xBF80, 0x0080, 0x03FF, 0x7BFF], dtype=np.uint16)
    idx = synth.raw_np(seed, 91, buf, n) % np.uint64(pal.size)
    return pal[idx.astype(np.int64)]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("W", [1, 2, 3, 8, 16])
def test_reduce_threads_bitwise(oracle_mod, dtype, W):
    for n in (0, 1, 7, 1000, 12345):
        for gen in (_bits, _special):
            srcs = [gen(dtype, W * 31 + n, w, n) for w in range(W)]
            one = oracle_mod.reduce(dtype, srcs, threads=1)
            for t in THREADS + (n + 5,):
                many = oracle_mod.reduce(dtype, srcs, threads=t)
                assert np.array_equal(one.view(RAW[dtype]), many.view(RAW[dtype])), (dtype, W, n, t)


def test_reduce_threads_scattered_share(oracle_mod):
    W, n = 8, 8 * 999
    srcs = [_bits("bf16", 5, w, n) for w in range(W)]
    for rank in (0, 3, 7):
        one = oracle_mod.reduce_layout("bf16", "scattered", rank, srcs)
        for t in THREADS:
            assert np.array_equal(one, oracle_mod.reduce_layout("bf16", "scattered", rank, srcs, threads=t))


@pytest.mark.parametrize("kinds", [("packed", "packed"), ("scattered", "transposed"), ("scattered", "scattered")])
@pytest.mark.parametrize("W", [1, 3, 8, 16])
def test_copy_threads_bitwise(oracle_mod, kinds, W):
    for per in (16 * W, 16 * W * 37):
        srcs = [synth.bits_np(W, 92, s, per) for s in range(W)]
        one = oracle_mod.copy_layout(*kinds, srcs)
        for t in THREADS + (per + 3,):
            assert np.array_equal(one, oracle_mod.copy_layout(*kinds, srcs, threads=t)), (kinds, W, per, t)


def test_copy_threads_ragged_segments(oracle_mod):
    parts = [16 * 7, 0, 16 * 1001, 16, 16 * 64]
    srcs = [synth.bits_np(3, 93, w, max(16, parts[w])) for w in range(len(parts))]
    one = oracle_mod.allgather_v(srcs, parts)
    for t in THREADS:
        assert np.array_equal(one, oracle_mod.allgather_v(srcs, parts, threads=t))


@pytest.mark.parametrize("W", [1, 2, 8, 16])
def test_copy_v_threads_bitwise(oracle_mod, W):
    rng = np.random.default_rng(W)
    for rows in ([0] * W, [1] * W, list(rng.integers(0, 300, W)), [1000] * W):
        rb = 48
        srcs = [synth.bits_np(W, 94, s, max(16, int(rows[s]) * rb)) for s in range(W)]
        p = synth.zipf_weights(1.1, W)
        dests = [synth.categorical_np(W, 95, s, int(rows[s]), p) for s in range(W)]
        one = oracle_mod.copy_v(srcs, dests, rb)
        for t in THREADS + (max(rows) + 4,):
            many = oracle_mod.copy_v(srcs, dests, rb, threads=t)
            for a, b in zip(one, many):
                assert np.array_equal(a, b), (W, rows, t)


def test_copy_v_threads_rejects_bad_destination(oracle_mod):
    srcs = [synth.bits_np(0, 96, s, 64) for s in range(2)]
    with pytest.raises(ValueError):
        oracle_mod.copy_v(srcs, [np.array([0, 2], dtype=np.int32), np.array([1, 0], dtype=np.int32)], 32,
                          threads=4)


def test_hardware_threads(oracle_mod):
    import os

    assert oracle_mod.hardware_threads() >= 1
    assert 1 <= oracle_mod.default_threads() <= 16
    assert oracle_mod.hardware_threads() <= (os.cpu_count() or 1024)
