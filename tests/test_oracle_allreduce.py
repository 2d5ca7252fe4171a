"""The oracle's AllReduce, pinned to its composition from the oracle's ReduceScatter
shares and AllGather-style gather (Purlin paper, section 3.1: AllReduce is
ReduceScatter followed by AllGather, a scattered-to-scattered transformation), and to
the elementwise definition on a straight-line numpy evaluation."""
import numpy as np
import pytest

import synth


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("W", [1, 2, 3, 8])
def test_composition_reduce_scatter_then_gather(oracle_mod, dtype, W):
    per = 16 * W * 37 // (4 if dtype == "f32" else 2)  # elements per source, divisible by W
    srcs = [synth.normal_np(W, 2, w, per, 1.0, dtype) for w in range(W)]
    outs = oracle_mod.allreduce(dtype, srcs)
    # ReduceScatter: rank r reduces slice r of every source
    shares = [oracle_mod.reduce_layout(dtype, "scattered", r, srcs) for r in range(W)]
    # AllGather of the shares: slice s of every rank's output is share s
    gathered = oracle_mod.copy_layout("scattered", "scattered",
                                      [np.concatenate([shares[s] if k == s else np.zeros_like(shares[s])
                                                       for k in range(W)]) for s in range(W)])
    for r in range(W):
        assert outs[r].tobytes() == gathered.tobytes()
        assert outs[r].tobytes() == np.concatenate(shares).tobytes()


def test_outputs_are_independent_arrays(oracle_mod):
    srcs = [synth.uniform_pm1_np(0, 1, w, 64) for w in range(3)]
    outs = oracle_mod.allreduce("bf16", srcs)
    outs[0][0] ^= 1
    assert outs[1][0] != outs[0][0]
