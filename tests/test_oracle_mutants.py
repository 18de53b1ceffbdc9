"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them.  The shipped oracle source is not modified."""
import os
import subprocess
import sys
import tempfile

import pytest

from oracle import build as obuild

# (name, text in csf_oracle.c, replacement, replace every occurrence?)
MUTANTS = [
    ("window one wider in base choice", "u <= v + W - 1 && u <= 255", "u <= v + W && u <= 255", False),
    ("window one narrower in base choice", "u <= v + W - 1 && u <= 255", "u <= v + W - 2 && u <= 255", False),
    ("ties go to the largest base", "if (count > best_count) {", "if (count >= best_count) {", False),
    ("window check admits W", "return d >= 0 && d < W;", "return d >= 0 && d <= W;", False),
    ("window check below base", "return d >= 0 && d < W;", "return d >= -1 && d < W;", False),
    ("window wraps past 255", "int d = value - base;", "int d = (value - base) & 255;", False),
    ("field and byte index swapped in both coder halves",
     "int64_t byte_in_group = p % 16;\n                int64_t field_index = (p % G) / 16;",
     "int64_t byte_in_group = (p % G) / 16;\n                int64_t field_index = p % 16;", False),
    ("byte order reversed in both coder halves", "16 * group + byte_in_group", "16 * group + (15 - byte_in_group)", True),
    ("exception keeps the offset instead of the byte", "| (uint32_t)value;", "| (uint32_t)(value - base);", False),
    ("exception position off by one", "((uint32_t)p << 8)", "((uint32_t)(p + 1) << 8)", False),
    ("prefix written one expert early", "prefix[e + 1] = (int32_t)n;", "prefix[e] = (int32_t)n;", False),
    ("decoder skips the exception pass", "if (pos < P) ws[", "if (pos < 0) ws[", False),
    ("decoder keeps entries past the plane", "if (pos < P) ws[", "if (pos < P + 64) ws[", False),
    ("routed skip admits equal starts", "!(expert_start[e + 1] > expert_start[e])", "!(expert_start[e + 1] >= expert_start[e])", False),
    ("routing ignored", "if (expert_start != NULL && !(", "if (0 && !(", False),
    ("decoder row from column", "int64_t r = p / C;", "int64_t r = p % C;", False),
    ("field mask one bit short", "& (W - 1);", "& ((W >> 1) - 1);", False),
    ("index counts entries at the tile start", "< ORACLE_INDEX_TILE * j) below++;",
     "<= ORACLE_INDEX_TILE * j) below++;", False),
    ("index tile of 1024 positions", "#define ORACLE_INDEX_TILE 2048", "#define ORACLE_INDEX_TILE 1024", False),
    ("row window end inclusive", "for (int64_t r = row_begin; r < row_end; r++) {",
     "for (int64_t r = row_begin; r <= row_end && r < R; r++) {", False),
    ("row window begins a row early", "for (int64_t r = row_begin; r < row_end; r++) {",
     "for (int64_t r = row_begin > 0 ? row_begin - 1 : 0; r < row_end; r++) {", False),
    ("windowed exception pass ignores the window", "if (pos < P && row >= row_begin && row < row_end)",
     "if (pos < P)", False),
    ("index tiles rounded down", "return (P + ORACLE_INDEX_TILE - 1) / ORACLE_INDEX_TILE;",
     "return P / ORACLE_INDEX_TILE + 1;", False),
]


_CHILD = """
import sys
sys.path[:0] = {paths!r}
import oracle
from oracle_pins import ALL_PINS
orc = oracle.Oracle({lib!r})
failed = []
for pin in ALL_PINS:
    try:
        pin(orc)
    except AssertionError:
        failed.append(pin.__name__)
    except Exception as exc:
        failed.append(pin.__name__ + " (" + type(exc).__name__ + ")")
print("FAILED:" + ",".join(failed))
"""


def _run_pins(lib_path):
    """Run every pin against the library at lib_path in a child process; a
    mutant that crashes the child counts as caught."""
    here = os.path.dirname(os.path.abspath(__file__))
    code = _CHILD.format(paths=[here, os.path.dirname(here)], lib=lib_path)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    if res.returncode != 0:
        return [f"child exited with {res.returncode}"]
    line = [l for l in res.stdout.splitlines() if l.startswith("FAILED:")][-1]
    return [n for n in line[len("FAILED:"):].split(",") if n]


@pytest.mark.parametrize("name,old,new,every", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, every):
    src = open(obuild.SOURCE).read()
    assert old in src, f"mutation site for '{name}' not found in the oracle source"
    mutated = src.replace(old, new) if every else src.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        open(path, "w").write(mutated)
        lib = obuild.build(path, os.path.join(d, "libmutant.so"), extra_flags=["-Wno-error"])
        failed = _run_pins(lib)
    assert failed, f"no pin caught the planted mistake: {name}"
