"""The benchmark's byte accounting and host helpers (no GPU).

Algorithmic bytes of a decode follow from the layout alone: bases E*R,
offsets E*S with S = 16 * ceil(R*C / G) (G = 32 positions per 16-byte group
for NVFP4, 128 for MXFP4), 4 bytes per exception entry, the int32 prefix
[E+1] and the int32 tile index [E * ceil(R*C / 2048) + 1]; a routed decode
counts only its routed experts' planes, streams and index segments."""
import math
import os
import shutil

import numpy as np
import pytest

import bench
import workloads

mwd = pytest.importorskip("moe_weight_decode_amd")


def closed_form(spec, n, active=None):
    E, R, C = spec.E, spec.R, spec.C
    G = 32 if spec.fmt == workloads.NVFP4 else 128
    S = 16 * math.ceil(R * C / G)
    NT = math.ceil(R * C / 2048)
    k = E if active is None else int(np.count_nonzero(active))
    index = 4 * (E * NT + 1) if active is None else 4 * k * (NT + 1)
    return k * (R + S), 4 * n + 4 * (E + 1), k * R * C, index


@pytest.mark.parametrize("name", ["tiny_nvfp4", "gate_nvfp4", "mxfp4"])
def test_full_decode_bytes(name):
    spec = workloads.STACKS[name]
    stack = mwd.prepare(spec.generate(), spec.fmt)
    b = bench.stack_bytes(stack)
    assert tuple(b) == closed_form(spec, stack.num_exceptions)
    assert b.metric == b.fixed + b.exc + b.dense
    if name == "gate_nvfp4":
        # the default benchmark line's bytes per step: 512 x 800 x 128 dense
        # bytes (52,428,800, as on the pages) plus the compressed streams
        # (bases, offsets, entries, prefix); the tile index is listed apart
        assert b.metric == 85_348_500
        assert b.dense == 52_428_800 and b.index == 102_404


def test_routed_decode_bytes_count_routed_experts_only():
    spec = workloads.TINY
    stack = mwd.prepare(spec.generate(), spec.fmt)
    active = np.array([True, False, False, True])
    pfx = stack.prefix.numpy()
    n = int(pfx[1] - pfx[0] + pfx[4] - pfx[3])
    assert tuple(bench.stack_bytes(stack, active)) == closed_form(spec, n, active)
    b = bench.stack_bytes(stack.without_index(), active)
    assert b.exc == 4 * n + 4 * (spec.E + 1) and b.index == 0   # no index without one


def test_cpu_baseline_slices_cover_every_expert():
    for E, n in ((512, 16), (384, 7), (4, 16), (1, 1)):
        sl = bench._slices(E, n)
        assert sl[0][0] == 0 and sl[-1][1] == E and len(sl) <= n
        assert all(a < b for a, b in sl) and all(sl[i][1] == sl[i + 1][0] for i in range(len(sl) - 1))


def test_routed_sets_are_disjoint_groups_of_one_permutation():
    E, k, m = 512, 8, 64
    sets = bench.routed_sets(workloads, E, k, m, 177, 64)
    seen = set()
    for es in sets:
        assert es.dtype == np.int32 and es.shape == (E + 1,) and es[0] == 0
        counts = np.diff(es)
        act = np.flatnonzero(counts)
        assert len(act) == k and counts[act].min() >= 1 and counts[act].max() <= m
        assert not seen & set(act.tolist())
        seen |= set(act.tolist())
    assert len(seen) == E                        # 64 x 8 = every expert once


def test_source_hash_ignores_comments_only(tmp_path):
    src = os.path.join(bench.ROOT, "moe_weight_decode_amd", "csrc")
    d = tmp_path / "csrc"
    shutil.copytree(src, d)
    h0 = bench.source_hash("csf_moe_w4a16_kernel", str(d))
    assert h0 == bench.source_hash("csf_moe_w4a16_kernel")
    p = d / "csf_moe.hip"
    text = p.read_text()
    p.write_text("// a comment\n/* another\n comment */\n" + text.replace("\n", "\n  ", 3))
    assert bench.source_hash("csf_moe_w4a16_kernel", str(d)) == h0
    p.write_text(text.replace("kMoeWaves = 8", "kMoeWaves = 4", 1))
    assert bench.source_hash("csf_moe_w4a16_kernel", str(d)) != h0
    assert bench.source_hash("csf_fused_kernel", str(d)) == bench.source_hash("csf_fused_kernel")


@pytest.mark.parametrize("argv", [["--two-pass", "--workload", "routed_paired"],
                                  ["--two-pass", "--workload", "routed_moe"],
                                  ["--two-pass", "--encode", "gate_nvfp4"]])
def test_two_pass_only_for_full_stack_workloads(argv):
    """--two-pass times a full-stack decode without its index; the routed and
    encode modes refuse it before touching a GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *argv], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode != 0
    assert "--two-pass applies to the full-stack workloads" in res.stderr


def test_two_pass_bytes_drop_the_index():
    """The two-pass line's metric bytes are the stack's streams and dense bytes,
    with no tile index read."""
    import moe_weight_decode_amd as mwd
    spec = workloads.TINY
    stack = mwd.prepare(spec.generate(), spec.fmt)
    b, b2 = bench.stack_bytes(stack), bench.stack_bytes(stack.without_index())
    assert b2.index == 0 and b.index > 0
    assert (b2.fixed, b2.exc, b2.dense) == (b.fixed, b.exc, b.dense)
