"""Pins of the W4A16 consumer oracle (oracle/w4a16.py), CPU only.

Each pin ties the oracle to something outside itself: the E2M1 value table of
the OCP MX specification (tests/golden/e2m1_ocp_mx.json), torch's float8_e4m3fn
and float8_e8m0fnu conversions for every scale byte, a scalar brute-force
evaluation written independently of the vectorised reference (both weight
formats), and closed-form special cases."""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import w4a16

HERE = os.path.dirname(os.path.abspath(__file__))


def test_e2m1_table_matches_ocp_spec():
    g = json.load(open(os.path.join(HERE, "golden", "e2m1_ocp_mx.json")))
    pos = g["code_to_value"]
    want = pos + [-v for v in pos]
    assert w4a16.E2M1_TABLE.tolist() == want


def test_e4m3_table_matches_torch_for_every_byte():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = w4a16.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))  # -0 at 0x80


def test_ue8m0_table_matches_torch_for_every_byte():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = w4a16.UE8M0_TABLE
    assert np.isnan(got[255]) and np.isnan(ref[255]) and not np.isnan(got[:255]).any()
    assert np.array_equal(got[:255], ref[:255])


def test_bf16_bits_exact():
    bits = workloads.bf16_bits(7, 33, np.random.default_rng(3))
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(w4a16.bf16_to_f64(bits), ref)


def _brute(inp: workloads.W4A16Inputs, fmt: str = "nvfp4"):
    """Scalar evaluation with its own bit extraction (Python ints and floats)."""
    T, K = inp.x_bits.shape
    E, N = inp.w_packed.shape[:2]
    y = [[0.0] * N for _ in range(T)]

    def f4(c):
        s = -1.0 if c >= 8 else 1.0
        c &= 7
        return s * (c / 2.0 if c < 2 else (2 + (c & 1)) * 2.0 ** ((c >> 1) - 2))

    def f8(b):
        s = -1.0 if b >= 128 else 1.0
        b &= 127
        e, m = b >> 3, b & 7
        return s * (m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10))

    def e8(b):
        return float("nan") if b == 255 else math.ldexp(1.0, b - 127)

    block, scale = (16, f8) if fmt == "nvfp4" else (32, e8)

    def bf(u):
        s = -1.0 if u >= 32768 else 1.0
        e, m = (u >> 7) & 255, u & 127
        return s * (m * 2.0 ** -133 if e == 0 else (128 + m) * 2.0 ** (e - 134))

    for e in range(E):
        for t in range(int(inp.expert_start[e]), int(inp.expert_start[e + 1])):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    byte = int(inp.w_packed[e, n, k // 2])
                    code = (byte >> 4) if k % 2 else (byte & 15)
                    acc += bf(int(inp.x_bits[t, k])) * f4(code) * scale(int(inp.scales[e, n, k // block]))
                y[t][n] = float(np.float32(inp.alpha[e])) * acc
    return np.array(y)


def _tiny(fmt: str = "nvfp4"):
    es = np.array([0, 2, 2, 5], dtype=np.int32)   # expert 1 has no tokens
    if fmt == "nvfp4":
        return workloads.w4a16_inputs(3, 3, 64, es, seed=11)
    return workloads.w4a16_inputs(3, 3, 96, es, seed=12, exc_rate=0.3, fmt=workloads.MXFP4)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_reference_matches_brute_force(fmt):
    inp = _tiny(fmt)
    y, mag = w4a16.moe_w4a16(inp.x_bits, inp.w_packed, inp.scales, inp.alpha, inp.expert_start, fmt=fmt)
    want = _brute(inp, fmt)
    assert np.allclose(y, want, rtol=1e-12, atol=1e-300)
    assert np.all(mag >= np.abs(y) * (1 - 1e-12))


def test_unit_weights_sum_activations():
    inp = _tiny()
    inp.w_packed[:] = 0x22            # every code 1.0
    inp.scales[:] = 0x38              # every scale 1.0
    inp.alpha[:] = 1.0
    y, _ = w4a16.moe_w4a16(inp.x_bits, inp.w_packed, inp.scales, inp.alpha, inp.expert_start)
    x = w4a16.bf16_to_f64(inp.x_bits)
    assert np.array_equal(y, np.repeat(x.sum(axis=1, keepdims=True), 3, axis=1))


def test_mxfp4_unit_scales_equal_plain_e2m1():
    # UE8M0 byte 127 is 1.0: y is the plain E2M1 product
    inp = _tiny("mxfp4")
    inp.scales[:] = 127
    y, _ = w4a16.moe_w4a16(inp.x_bits, inp.w_packed, inp.scales, inp.alpha, inp.expert_start, fmt="mxfp4")
    x = w4a16.bf16_to_f64(inp.x_bits)
    codes = w4a16.E2M1_TABLE[w4a16.unpack_codes(inp.w_packed)]
    for e in range(3):
        t0, t1 = inp.expert_start[e], inp.expert_start[e + 1]
        assert np.array_equal(y[t0:t1], float(inp.alpha[e]) * (x[t0:t1] @ codes[e].T))


def test_sign_bit_negates():
    inp = _tiny()
    y, _ = w4a16.moe_w4a16(inp.x_bits, inp.w_packed, inp.scales, inp.alpha, inp.expert_start)
    y2, _ = w4a16.moe_w4a16(inp.x_bits, inp.w_packed ^ 0x88, inp.scales, inp.alpha, inp.expert_start)
    assert np.array_equal(y2, -y)


@pytest.mark.parametrize("mistake", ["nibbles swapped", "scale per 32 weights", "subnormal code as 1.0",
                                     "routing one token late"])
def test_brute_force_catches_plausible_mistakes(mistake):
    """The brute-force pin is sensitive to each of these reference mistakes."""
    inp = _tiny()
    w, s, es = inp.w_packed, inp.scales, inp.expert_start.copy()
    if mistake == "nibbles swapped":
        w = ((w & 0x0F) << 4) | (w >> 4)
    elif mistake == "scale per 32 weights":
        s = np.repeat(s[..., ::2], 2, axis=-1)
    elif mistake == "routing one token late":
        es[1:-1] += 1
    if mistake == "subnormal code as 1.0":
        saved = w4a16.E2M1_TABLE.copy()
        w4a16.E2M1_TABLE[[1, 9]] = [1.0, -1.0]
        try:
            y, _ = w4a16.moe_w4a16(inp.x_bits, w, s, inp.alpha, es)
        finally:
            w4a16.E2M1_TABLE[:] = saved
    else:
        y, _ = w4a16.moe_w4a16(inp.x_bits, w, s, inp.alpha, es)
    assert not np.allclose(y, _brute(inp), rtol=1e-9)


@pytest.mark.parametrize("mistake", ["scale per 16 weights", "exponent bias 126", "nibbles swapped"])
def test_brute_force_catches_plausible_mxfp4_mistakes(mistake):
    """The MXFP4 brute-force pin is sensitive to each of these reference mistakes."""
    inp = _tiny("mxfp4")
    w, s = inp.w_packed, inp.scales
    if mistake == "nibbles swapped":
        w = ((w & 0x0F) << 4) | (w >> 4)
    if mistake == "scale per 16 weights":
        # the row's MX scale bytes read as one per 16 weights (the row's bytes twice over)
        s16 = np.concatenate([s, s], axis=-1)
        saved = w4a16.FORMATS["mxfp4"]
        w4a16.FORMATS["mxfp4"] = (16, w4a16.UE8M0_TABLE)
        try:
            y, _ = w4a16.moe_w4a16(inp.x_bits, w, s16, inp.alpha, inp.expert_start, fmt="mxfp4")
        finally:
            w4a16.FORMATS["mxfp4"] = saved
    elif mistake == "exponent bias 126":
        saved = w4a16.UE8M0_TABLE.copy()
        w4a16.UE8M0_TABLE[:255] *= 2.0
        try:
            y, _ = w4a16.moe_w4a16(inp.x_bits, w, s, inp.alpha, inp.expert_start, fmt="mxfp4")
        finally:
            w4a16.UE8M0_TABLE[:] = saved
    else:
        y, _ = w4a16.moe_w4a16(inp.x_bits, w, s, inp.alpha, inp.expert_start, fmt="mxfp4")
    assert not np.allclose(y, _brute(inp, "mxfp4"), rtol=1e-9)
