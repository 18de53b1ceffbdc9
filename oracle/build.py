"""Build the CPU oracle shared library with gcc (test infrastructure only)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "csf_oracle.c")
LIBRARY = os.path.join(HERE, "libcsf_oracle.so")


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile ``source`` into ``output``; returns the library path."""
    tmp = output + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared",
           *extra_flags, source, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(), file=sys.stderr)
