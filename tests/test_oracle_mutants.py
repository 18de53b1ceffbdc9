"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them.  The shipped oracle source is not modified."""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
from oracle import build as obuild
from oracle_pins import ALL_PINS

# (name, text in csf_oracle.c, replacement, replace every occurrence?)
MUTANTS = [
    ("window one wider in base choice", "u <= v + W - 1 && u <= 255", "u <= v + W && u <= 255", False),
    ("window one narrower in base choice", "u <= v + W - 1 && u <= 255", "u <= v + W - 2 && u <= 255", False),
    ("ties go to the largest base", "if (count > best_count) {", "if (count >= best_count) {", False),
    ("window check admits W", "return d >= 0 && d < W;", "return d >= 0 && d <= W;", False),
    ("window check below base", "return d >= 0 && d < W;", "return d >= -1 && d < W;", False),
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
]


def _run_pins(lib_path):
    orc = oracle.Oracle(lib_path)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
        except Exception as exc:  # a crash or bad output also counts as caught
            failed.append(f"{pin.__name__} ({type(exc).__name__})")
    return failed


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
