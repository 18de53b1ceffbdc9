"""The gfx950 kernels keep the register budget their launch plan assumes (no GPU).

The host launches the fused kernel with 7 workgroups per CU for 8K tiles and 6
for 16K tiles (one wave of each workgroup per SIMD), so those variants must fit
512 / 7 and 512 / 6 VGPRs per lane; the W4A16 consumer runs one 8-wave
workgroup per CU (2 waves per SIMD, 256 VGPRs each); no kernel may spill to
scratch memory."""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_weight_decode_amd", "csrc")

# fused kernel instantiation (runs, entries per lane, load schedule; the routed kernel is schedule 2)
# -> waves per SIMD the plan needs
PLAN_WAVES = {("2", "4", "1"): 7, ("2", "8", "1"): 7, ("4", "4", "0"): 6, ("1", "4", "2"): 2}


def _kernel_resources(source):
    from moe_weight_decode_amd import build as b
    with tempfile.TemporaryDirectory() as d:
        flags = [f for f in b.HIPCC_FLAGS if f not in ("-shared", "-Wall", "-Werror")]
        cmd = [b.hipcc(), *flags,
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--save-temps", "-c", source,
               "-o", os.path.join(d, "k.o")]
        subprocess.run(cmd, cwd=d, check=True, capture_output=True)
        asm = [f for f in os.listdir(d) if f.endswith("gfx950.s")][0]
        text = open(os.path.join(d, asm)).read()
    out = {}
    for block in text.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        vgpr = int(re.search(r"\.vgpr_count:\s+(\d+)", block).group(1))
        scratch = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", block).group(1))
        out[name] = (vgpr, scratch)
    return out


@pytest.mark.parametrize("source", ["csf_kernels.hip", "csf_encode.hip", "csf_moe.hip"])
def test_no_scratch_and_plan_occupancy(source):
    res = _kernel_resources(os.path.join(CSRC, source))
    assert res, "no kernels found"
    for name, (vgpr, scratch) in res.items():
        assert scratch == 0, f"{name} uses {scratch} bytes of scratch"
        m = re.search(r"csf_fused_kernelILj(\d+)ELj(\d+)ELj(\d)E", name)
        r = re.search(r"csf_routed_kernelILj(\d+)ELj(\d+)E", name)
        if m or r:
            waves = PLAN_WAVES[m.groups() if m else r.groups() + ("2",)]
            granted = 512 // (((vgpr + 7) // 8) * 8)
            assert granted >= waves, f"{name}: {vgpr} VGPRs allow {granted} waves per SIMD, plan needs {waves}"
        if "csf_moe_w4a16_kernel" in name:  # one 8-wave workgroup per CU: 2 waves per SIMD
            granted = 512 // (((vgpr + 7) // 8) * 8)
            assert granted >= 2, f"{name}: {vgpr} VGPRs allow {granted} waves per SIMD, the launch needs 2"
