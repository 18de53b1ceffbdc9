"""CPU pins of the oracle (no GPU): see tests/oracle_pins.py for what each pins."""
import json
import os

import numpy as np
import pytest

import workloads
from oracle_pins import ALL_PINS

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)


def test_page_figures_closed_form(orc):
    """Stack and checkpoint sizes printed on the pages follow from the shapes:
    dense bytes = experts x rows x K / 16 for NVFP4."""
    g = json.load(open(os.path.join(HERE, "golden", "page_figures.json")))
    fig, shapes = g["figures"], g["shapes"]
    per_scale = fig["nvfp4_weights_per_scale"]["value"]
    planes = []
    for name in ("gate", "down"):
        s = shapes[name]
        C = s["K"] // per_scale
        dense = s["experts"] * s["rows"] * C
        assert round(dense / 1e6, 2) == fig["dense_stack_MB"]["value"]
        planes.append(s["rows"] * C)
    # every projection plane holds the same 102,400 scale bytes
    assert planes[0] == planes[1]
    cp = fig["checkpoint_planes"]
    assert cp["layers"] * cp["experts"] * cp["projections"] == cp["value"]
    assert round(cp["value"] * planes[0] / 2**30, 2) == fig["checkpoint_dense_scales_GiB"]["value"]


def test_layout_no_larger_than_pages(orc):
    """The fixed part of this layout (bases, offsets, prefix) for the pages'
    stacks fits inside the compressed sizes the pages measured, so the layout
    is at least as compact as theirs before exceptions are counted."""
    g = json.load(open(os.path.join(HERE, "golden", "page_figures.json")))
    fig, shapes = g["figures"], g["shapes"]
    for name, key in (("gate", "compressed_gate_MB"), ("down", "compressed_down_MB")):
        s = shapes[name]
        E, R, C = s["experts"], s["rows"], s["K"] // 16
        fixed = E * R + E * orc.segment_bytes(workloads.NVFP4, R, C) + 4 * (E + 1)
        assert fixed <= fig[key]["value"] * 1e6


def test_sizes_closed_form(orc):
    """Offsets take 16 bytes per 32 positions (NVFP4) or per 128 (MXFP4)."""
    assert orc.segment_bytes(workloads.NVFP4, 800, 128) == 51200
    assert orc.segment_bytes(workloads.NVFP4, 2048, 50) == 51200
    assert orc.segment_bytes(workloads.MXFP4, 1024, 160) == 20480
    assert orc.segment_bytes(workloads.NVFP4, 64, 8) == 256
    assert orc.segment_bytes(workloads.NVFP4, 1, 1) == 16
    assert orc.segment_bytes(workloads.MXFP4, 1, 129) == 32


def test_rejects_bad_shapes(orc):
    with pytest.raises(ValueError):
        orc.choose_bases(workloads.NVFP4, np.zeros((1, 1 << 12, 1 << 12), dtype=np.uint8))
    with pytest.raises(ValueError):
        orc.choose_bases(7, np.zeros((1, 2, 2), dtype=np.uint8))


def test_decode_experts_slices_equal_whole_decode(orc):
    """The CPU baseline's threaded decode: disjoint expert ranges decoded from
    several threads give the whole-stack decode, full and routed."""
    from concurrent.futures import ThreadPoolExecutor
    x = workloads.nvfp4_stack(16, 40, 50, 3, 0.1)
    st = orc.encode(workloads.NVFP4, x)
    ws = np.zeros_like(x)
    with ThreadPoolExecutor(4) as pool:
        list(pool.map(lambda r: orc.decode_experts(st, r[0], r[1], ws), [(0, 3), (3, 9), (9, 16)]))
    assert np.array_equal(ws, x)
    es = workloads.routing(16, 5, 4, seed=1)
    ws = np.full_like(x, 0xA5)
    orc.decode_experts(st, 0, 7, ws, es)
    orc.decode_experts(st, 7, 16, ws, es)
    assert np.array_equal(ws, orc.decode(st, es, np.full_like(x, 0xA5)))
