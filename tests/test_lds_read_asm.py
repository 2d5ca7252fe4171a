"""The LDS-staged kernels' reads, checked in their gfx950 assembly (CPU only: hipcc
cross-compiles). Each slab's ds_read_b128 reads come from inline assembly, and their
results may be used only after the s_waitcnt that waits for them. Were the reads and
the wait separate statements, the compiler could place arithmetic on a read's
registers between them, before the data has arrived (as a restructured reduce once
was compiled). So between a ds_read_b128 and the next s_waitcnt lgkmcnt(0) nothing
may stand but further ds_read_b128."""
import os
import re
import subprocess

import pytest

import __graft_entry__

B = __graft_entry__._load_builder()


def _device_asm(src: str, out: str) -> str:
    cmd = [B.HIPCC, *B.COMMON, "-I", B.CSRC, "-x", "hip", *B.DEVICE, "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    with open(out) as f:
        return f.read()


def _functions(asm: str, pattern: str):
    """Instruction lines of every function whose symbol matches `pattern`."""
    out, name, body = {}, None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            if name and re.search(pattern, name):
                out[name] = body
            name, body = m.group(1), []
            continue
        s = line.split(";")[0].strip()
        if name and s and not s.startswith(".") and not s.endswith(":"):
            body.append(s)
    if name and re.search(pattern, name):
        out[name] = body
    return out


def _read_groups(body):
    """(reads, instructions between the first read and its wait) for every run of
    LDS reads; the list is empty when only reads precede the wait."""
    groups, i = [], 0
    while i < len(body):
        if body[i].startswith("ds_read_b128"):
            reads, between, j = 1, [], i + 1
            while j < len(body) and not re.match(r"s_waitcnt\b.*lgkmcnt\(0\)", body[j]):
                if body[j].startswith("ds_read_b128"):
                    reads += 1
                else:
                    between.append(body[j])
                j += 1
            assert j < len(body), "an LDS read with no wait after it"
            groups.append((reads, between))
            i = j
        i += 1
    return groups


@pytest.mark.parametrize("src, pattern", [("reduce.hip", r"k_reduce_lds"), ("copy.hip", r"k_copy_lds")])
def test_lds_reads_wait_before_use(tmp_path, src, pattern):
    fns = _functions(_device_asm(src, str(tmp_path / (src + ".s"))), pattern)
    assert fns, f"no {pattern} kernel in the assembly of {src}"
    for name, body in fns.items():
        groups = _read_groups(body)
        assert groups, f"{name}: no LDS reads"
        for reads, between in groups:
            assert not between, f"{name}: {between[:3]} between {reads} LDS reads and their wait"
