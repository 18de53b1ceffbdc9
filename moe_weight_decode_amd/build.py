"""Build libcsf.so (the CSF decoder's C ABI and its gfx950 kernels) in-tree.

    python -m moe_weight_decode_amd.build [-D NAME=VALUE ...]
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "csf_api.cpp"), os.path.join(CSRC, "csf_kernels.hip"),
           os.path.join(CSRC, "csf_encode.hip"), os.path.join(CSRC, "csf_moe.hip")]
HEADERS = [os.path.join(ROOT, "include", "csf.h"), os.path.join(CSRC, "csf_launch.h"),
           os.path.join(CSRC, "csf_device.h")]
LIBRARY = os.path.join(PKG, "libcsf.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Werror",
    "-Wno-unused-command-line-argument",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(output: str = LIBRARY, defines=(), extra_flags=()) -> str:
    """Compile the library; returns its path.  ``defines`` are NAME=VALUE strings."""
    tmp = output + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, *[f"-D{d}" for d in defines],
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *SOURCES, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass names the device-only target feature it ignores; only
    # that warning is tolerated
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, output)
    return output


def stale(path: str = LIBRARY) -> bool:
    if not os.path.exists(path):
        return True
    t = os.path.getmtime(path)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    defs = [a[2:] if a.startswith("-D") else a for a in sys.argv[1:]]
    print(build(defines=defs), file=sys.stderr)
