"""The pins against plausible mistakes: each case plants one mistake in a copy of
oracle/oracle.c (the real file is never touched), builds that copy, and runs the
oracle's CPU pins against it in a child process (PLR_ORACLE_LIB); at least one pin
must fail. A control case builds an unmodified copy the same way and must pass, so a
failure is the planted mistake's and not the harness's."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), ".."))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (text in oracle.c, replacement): each a mistake an implementation could plausibly make,
# chosen so that the mutated oracle still writes only inside its buffers (a mistake must be
# caught by a pin, not by a crash of the child process)
MUTATIONS = {
    "ties_away_from_even": ("else r = (p & 1) ? p + 1 : p;", "else r = (p & 1) ? p : p + 1;"),
    "accumulator_starts_at_zero": ("float a = widen(dtype, srcs[0], src_off[0] + i);\n    for (int w = 1;",
                                   "float a = 0.0f;\n    for (int w = 0;"),
    "sources_in_reverse_order": ("for (int w = 1; w < W; ++w) a = a + widen(dtype, srcs[w], src_off[w] + i);",
                                 "for (int w = W - 1; w >= 1; --w) a = a + widen(dtype, srcs[w], src_off[w] + i);"),
    "last_source_dropped": ("for (int w = 1; w < W; ++w) a = a +", "for (int w = 1; w < W - 1; ++w) a = a +"),
    "fp16_exponent_bias": ("ldexp((double)(1024 + f), e - 15 - 10)", "ldexp((double)(1024 + f), e - 14 - 10)"),
    "bf16_subnormal_scale": ("ldexp((double)f, -126 - 7)", "ldexp((double)f, -127 - 7)"),
    "overflow_saturates": ("F->past_max : F->value", "1e300 : F->value"),
    "blocks_packed_source_major": ("for (int d = 0; d < W; ++d) {\n    int64_t off = base;\n    for (int s = 0; s < W; ++s) {",
                                   "for (int s = 0; s < W; ++s) {\n    int64_t off = base;\n    for (int d = 0; d < W; ++d) {"),
    "rows_reversed_within_a_block": ("for (int64_t i = i0; i < i1; ++i) {\n    int32_t d = dest[s][i];",
                                     "for (int64_t i = i1 - 1; i >= i0; --i) {\n    int32_t d = dest[s][i];"),
    "denormals_flushed": ("_mm_setcsr(old & ~(0x8000u | 0x0040u | 0x6000u));", "_mm_setcsr((old | 0x8040u) & ~0x6000u);"),
    "last_thread_stops_short": ("return (int64_t)((__int128)n * k / parts); }",
                                "return k == parts ? n - (n > 0) : (int64_t)((__int128)n * k / parts); }"),
    "thread_rank_prefix_short": ("  for (int64_t i = 0; i < i0; ++i) seen[dest[s][i]] += 1;",
                                 "  for (int64_t i = 1; i < i0; ++i) seen[dest[s][i]] += 1;"),
}


def _pins_against(tmp_path, text):
    src = tmp_path / "oracle.c"
    src.write_text(text)
    so = oracle.build(out=str(tmp_path / "liboracle.so"), src=str(src))
    env = dict(os.environ, PLR_ORACLE_LIB=so)
    return subprocess.run([sys.executable, "-m", "pytest", "tests", "-q", "-x", "-m", "not gpu",
                           "-k", "oracle and not mutation", "-p", "no:cacheprovider"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_unmodified_copy_passes_the_pins(tmp_path):
    with open(SRC) as f:
        r = _pins_against(tmp_path, f.read())
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(tmp_path, name):
    with open(SRC) as f:
        text = f.read()
    find, repl = MUTATIONS[name]
    assert text.count(find) == 1, f"{name}: the text to mutate is not in oracle.c exactly once"
    r = _pins_against(tmp_path, text.replace(find, repl))
    assert r.returncode == 1, f"{name}: exit {r.returncode}\n{r.stdout[-2000:]}"  # 1 = tests failed
    assert " failed" in r.stdout.strip().splitlines()[-1], r.stdout[-500:]
