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
# measurement kernels (ceilings, launch floors, host cost), linked to libcsf.so
PROBE_SOURCES = [os.path.join(CSRC, "csf_probe.hip")]
PROBE_HEADERS = [os.path.join(ROOT, "include", "csf_probe.h")]
PROBE_LIBRARY = os.path.join(PKG, "libcsf_probe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Werror",
    "-Wno-unused-command-line-argument",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # load a kernel's leading scalar arguments (up to 8 arguments) into scalar
    # registers at wave launch (the routed decode's routing inputs)
    "-mllvm", "-amdgpu-kernarg-preload-count=8",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(output: str = LIBRARY, defines=(), extra_flags=(), probe: bool = True) -> str:
    """Compile the library (and, with ``probe``, libcsf_probe.so next to it);
    returns the library's path.  ``defines`` are NAME=VALUE strings."""
    _compile(SOURCES, output, defines, extra_flags)
    if probe and output == LIBRARY:
        _compile(PROBE_SOURCES, PROBE_LIBRARY, defines, extra_flags,
                 link=["-L", PKG, "-lcsf", "-Wl,-rpath,$ORIGIN"])
    return output


def _compile(sources, output, defines=(), extra_flags=(), link=()):
    tmp = output + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, *[f"-D{d}" for d in defines],
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *sources, "-o", tmp, *link]
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


def stale(path: str = LIBRARY) -> bool:
    if not os.path.exists(path) or not os.path.exists(PROBE_LIBRARY):
        return True
    t = min(os.path.getmtime(path), os.path.getmtime(PROBE_LIBRARY))
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS + PROBE_SOURCES + PROBE_HEADERS)


if __name__ == "__main__":
    defs = [a[2:] if a.startswith("-D") else a for a in sys.argv[1:]]
    print(build(defines=defs), file=sys.stderr)
