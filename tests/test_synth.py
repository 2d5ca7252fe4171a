"""The seeded generators: pinned to published SplitMix64 outputs, backends agree."""
import numpy as np
import pytest
import torch

import synth
from conftest import golden_lines


def test_splitmix64_published_vectors():
    for line in golden_lines("splitmix64.txt"):
        seed, *expect = [int(x) for x in line.split()]
        state, got = seed, []
        for _ in expect:
            state = (state + synth.GAMMA) & synth.MASK64
            got.append(synth._mix_int(state))
        assert got == expect


def test_counter_form_is_the_sequential_generator():
    # value k of a stream is the (k+1)-th output of a generator seeded with the key
    key = synth.stream_key(7, 3, 2)
    state, seq = key, []
    for _ in range(20):
        state = (state + synth.GAMMA) & synth.MASK64
        seq.append(synth._mix_int(state))
    assert seq == [synth.stream_value_int(7, 3, 2, k) for k in range(20)]
    assert list(synth.raw_np(7, 3, 2, 20)) == seq


@pytest.mark.parametrize("start", [0, 5, 1000])
def test_backends_agree_bits(start):
    a = synth.raw_np(1, 2, 3, 4096, start)
    b = synth.raw_t(1, 2, 3, 4096, start).numpy().view(np.uint64)
    assert np.array_equal(a, b)
    assert np.array_equal(synth.bits_np(1, 4, 0, 1024, 8 * start),
                          synth.bits_t(1, 4, 0, 1024, 8 * start).numpy())


def test_slices_are_consistent():
    full = synth.uniform_pm1_np(0, 1, 0, 1000)
    part = synth.uniform_pm1_np(0, 1, 0, 300, start=500)
    assert np.array_equal(full[500:800], part)


def test_uniform_and_categorical_backends_agree():
    x = synth.uniform_pm1_np(0, 1, 2, 50000)
    y = synth.uniform_pm1_t(0, 1, 2, 50000).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(x, y)
    p = synth.zipf_weights(1.1, 8)
    assert np.array_equal(synth.categorical_np(0, 5, 1, 50000, p),
                          synth.categorical_t(0, 5, 1, 50000, p).numpy())


def test_normal_backends_agree_nearly():
    x = synth.normal_np(0, 3, 1, 50000, 0.5)
    y = synth.normal_t(0, 3, 1, 50000, 0.5).view(torch.int16).numpy().view(np.uint16)
    assert (x == y).mean() > 0.999


def test_distributions():
    x = torch.from_numpy(synth.uniform_pm1_np(0, 1, 0, 200000).view(np.int16)).view(torch.bfloat16).float()
    assert x.min() >= -1 and x.max() <= 1 and abs(float(x.mean())) < 0.01
    z = torch.from_numpy(synth.normal_np(0, 3, 0, 200000, 0.5).view(np.int16)).view(torch.bfloat16).float()
    assert abs(float(z.mean())) < 0.01 and abs(float(z.std()) - 0.5) < 0.01


def test_zipf_weights_closed_form():
    # weight(d) = (d+1)^-1.1 / sum: the values a hot-expert MoE dispatch uses
    p = synth.zipf_weights(1.1, 8)
    ref = [0.39816, 0.18575, 0.11891, 0.08666, 0.06779, 0.05547, 0.04682, 0.04043]
    assert np.allclose(p, ref, atol=1e-5)
    assert abs(p.sum() - 1) < 1e-12 and abs(p[0] / p[1] - 2 ** 1.1) < 1e-12
    d = synth.categorical_np(0, 5, 0, 8 * 4096, p)
    frac = np.bincount(d, minlength=8) / d.size
    assert np.allclose(frac, p, atol=0.01)
