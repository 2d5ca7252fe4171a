"""Build the HIP library in-tree: reduce_atom_amd/libplr.so for gfx950.

Every source is compiled by hipcc (device code for gfx950 only) and linked into one
shared library exporting the C ABI of include/plr.h. Run as
``python reduce_atom_amd/_build.py`` or through ``__graft_entry__.build()`` (not as
``-m reduce_atom_amd._build``: importing the package loads the library).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libplr.so")
BUILD = os.path.join(ROOT, "_build", "plr")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
    "-fno-fast-math", "-ffp-contract=off",
]
# gfx950 device code; packed fp32 instructions are kept out of the device code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]

SOURCES = ["api.cpp", "layout.cpp", "reduce.hip", "copy.hip", "copy_v.hip", "notify.hip", "allreduce.hip",
           "packets.hip", "noalloc.hip"]


def _compile(src: str, build_dir: str = BUILD, defines=(), csrc: str = CSRC) -> str:
    path = os.path.join(csrc, src)
    obj = os.path.join(build_dir, src + ".o")
    cmd = [HIPCC, *COMMON, "-I", csrc, *[f"-D{d}" for d in defines]]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE]
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False, out: str = OUT, defines=(),
          csrc: str = CSRC) -> str:
    """Compile and link libplr.so (always rebuilds). `defines` (extra -D macros) and
    `csrc` (another source directory) are for tuning builds written to another `out`."""
    build_dir = BUILD if out == OUT else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines, csrc), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build_user_kernels(src: str, out: str) -> str:
    """Compile one HIP file of user kernels written on the device-callable Atom
    (include/plr_atom.h) into its own shared library for gfx950 (always rebuilds)."""
    build_dir = out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", *DEVICE, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    shutil.rmtree(build_dir, ignore_errors=True)
    return out


def build_host_program(src: str, out: str) -> str:
    """Compile a host-only C program that calls the C ABI of include/plr.h and links
    libplr.so (found next to the program through its run path) and the HIP runtime.
    Always rebuilds."""
    cc = os.environ.get("PLR_CC", "/opt/rocm/llvm/bin/clang")
    rel = os.path.relpath(PKG, os.path.dirname(os.path.abspath(out)))
    tmp = out + ".tmp"
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), src, "-L", PKG, "-lplr", "-L/opt/rocm/lib", "-lamdhip64",
           f"-Wl,-rpath,$ORIGIN/{rel}", "-Wl,-rpath,/opt/rocm/lib", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
