"""The C ABI used from a plain C program with no Python in it (tests/c_abi/abi_driver,
built by __graft_entry__.build()): this test writes seeded inputs to files, runs the
program as a child process and compares what it wrote with the oracle, bit for bit.
The first test needs no GPU: the program loads libplr.so and the HIP runtime and
prints its usage."""
import os
import subprocess

import numpy as np
import pytest

import synth
from conftest import ROOT

DRIVER = os.path.join(ROOT, "tests", "c_abi", "abi_driver")


def _run(*args, timeout=120):
    return subprocess.run([DRIVER, *map(str, args)], capture_output=True, text=True, timeout=timeout)


def _need_driver():
    if not os.path.exists(DRIVER):
        import __graft_entry__

        __graft_entry__.build()


def test_driver_links_and_loads():
    _need_driver()
    r = _run()
    assert r.returncode == 2 and "plr " in r.stderr and "gfx950" in r.stderr, r.stderr


def _write(prefix, arrays, suffix=""):
    for w, a in enumerate(arrays):
        np.ascontiguousarray(a).tofile(f"{prefix}{suffix}.{w}")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,W,n,notify", [("bf16", 8, 70000, 0), ("f16", 3, 4096 + 8, 1), ("f32", 16, 1000, 1)])
def test_reduce_from_c(tmp_path, oracle_mod, dtype, W, n, notify):
    _need_driver()
    srcs = [synth.normal_np(5, 30, w, n, 1.0, dtype=dtype) for w in range(W)]
    prefix, out = str(tmp_path / "src"), str(tmp_path / "out")
    _write(prefix, srcs)
    code = {"bf16": 0, "f16": 1, "f32": 2}[dtype]
    r = _run("reduce", code, W, srcs[0].nbytes, notify, prefix, out)
    assert r.returncode == 0, r.stderr
    got = np.fromfile(out, dtype=srcs[0].dtype)
    ref = oracle_mod.reduce(dtype, srcs)
    assert np.array_equal(got.view(np.uint8), np.asarray(ref).view(np.uint8))


@pytest.mark.gpu
@pytest.mark.parametrize("kind,W,B,notify", [("ag", 8, 1 << 20, 0), ("a2a", 8, 8 * 4096 + 8 * 16, 1), ("ag", 5, 48, 1)])
def test_copy_from_c(tmp_path, oracle_mod, kind, W, B, notify):
    _need_driver()
    srcs = [synth.bits_np(5, 31, s, B) for s in range(W)]
    prefix, out = str(tmp_path / "src"), str(tmp_path / "out")
    _write(prefix, srcs)
    r = _run("copy", kind, W, B, notify, prefix, out)
    assert r.returncode == 0, r.stderr
    pair = ("packed", "packed") if kind == "ag" else ("scattered", "transposed")
    assert np.array_equal(np.fromfile(out, dtype=np.uint8), oracle_mod.copy_layout(*pair, srcs))


@pytest.mark.gpu
@pytest.mark.parametrize("W,rows,rb", [(8, [300, 0, 17, 1024, 5, 1025, 2, 64], 64), (2, [0, 0], 16),
                                       (8, [2000, 1500, 3000, 10, 0, 2048, 1, 4096], 32)])
def test_copy_v_from_c(tmp_path, oracle_mod, W, rows, rb):
    _need_driver()
    p = synth.zipf_weights(1.1, W)
    dests = [synth.categorical_np(W, 32, s, rows[s], p).astype(np.int32) for s in range(W)]
    srcs = [synth.bits_np(W, 33, s, rows[s] * rb) for s in range(W)]
    prefix, out = str(tmp_path / "src"), str(tmp_path / "out")
    _write(prefix, srcs)
    _write(prefix, dests, ".dest")
    r = _run("copy_v", W, rb, prefix, out)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(out, dtype=np.uint8)
    total = sum(rows) * rb
    ref, rc, ro = oracle_mod.copy_v(srcs, dests, rb)
    assert np.array_equal(raw[:total], ref)
    assert np.array_equal(raw[total:total + 8 * W * W].view(np.int64).reshape(W, W), rc)
    assert np.array_equal(raw[total + 8 * W * W:].view(np.int64).reshape(W, W), ro)
