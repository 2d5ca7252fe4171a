"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only): the
layout compiler (reduce_atom_amd/csrc/layout.cpp, which runs on the host and touches
no device) and the oracle (oracle/oracle.c), each linked into a seeded fuzz driver
under tests/sanitize/ and built here with the host compilers. A driver exits non-zero
on any sanitizer report or on a broken property (see the drivers' headers)."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _build(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr


def _run(exe, *args):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0 and "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, \
        (r.returncode, r.stderr[-3000:])
    return r.stdout


@pytest.mark.skipif(not os.path.exists(CLANGXX), reason="ROCm's host clang++ is not installed")
def test_layout_compiler_fuzz(tmp_path):
    exe = str(tmp_path / "layout_fuzz")
    _build([CLANGXX, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
            "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "reduce_atom_amd", "csrc", "layout.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "layout_fuzz.cpp"), "-o", exe])
    for seed in (1, 2, 3):
        out = _run(exe, 40000, seed)
        assert "accepted" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_fuzz(tmp_path):
    exe = str(tmp_path / "oracle_fuzz")
    _build(["gcc", "-std=c11", *SAN, "-ffp-contract=off", "-fno-fast-math",
            os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_fuzz.c"),
            "-o", exe, "-lm"])
    for seed in (1, 2):
        assert "iterations" in _run(exe, 1500, seed)
