"""W4A16 MoE projection with NVFP4 weights: CPU ORACLE.

TEST INFRASTRUCTURE ONLY.  The plain, slow, obviously correct statement of
what the consumer kernel computes.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may use it; the product library shares
nothing with it.

What is computed (float64 throughout):

  "finegrained-kernels: decode losslessly compressed NVFP4 scales (CSF)"
  (kernels-community PR 1236), paragraph on the format: NVFP4 keeps 4-bit
  weights and one 8-bit (E4M3) scale for every 16 weights.

  "NVFP4-CSF: expand_scales() for ahead-of-call scale expansion (canonical
  twin of #477)" (b12x PR 478), last commit message: a W4A16 MoE kernel
  (4-bit weights, 16-bit activations) that keeps the E4M3 block scales (one
  per 16 weights) compressed and turns the ones it is about to use back into
  plain bytes in on-chip shared memory.

  For every expert e with routed tokens t in [expert_start[e], expert_start[e+1])
  (the grouped routing: tokens sorted by expert):

      y[t, n] = alpha[e] * sum_k  x[t, k] * e2m1(W[e, n, k]) * e4m3(S[e, n, k // 16])

  x is bfloat16 (given as its 16-bit patterns), W holds E2M1 codes, S the E4M3
  scale bytes (the dense plane a CSF decode gives back), alpha[e] a float32
  per-expert tensor scale.

  MXFP4 weights (fmt="mxfp4"): the same E2M1 codes with one UE8M0 scale byte
  per 32 weights, y[t, n] = alpha[e] * sum_k x[t, k] * e2m1(W[e, n, k]) *
  2^(S[e, n, k // 32] - 127) (OCP Microscaling Formats v1.0: MXFP4 blocks of
  32 E2M1 elements sharing an E8M0 scale; E8M0 = 2^(byte - 127), 0xFF NaN).
  The pages compress MXFP4 scale planes the same way, with one-bit offsets
  ("NVFP4-CSF: expand_scales() ...", b12x PR 478, commit messages); they give
  no MXFP4 consumer, so this is the plainest one.

Readings fixed here (the pages give no consumer layout):
  * W is packed two codes per byte, row-major [E][N][K/2]: code k of row n is
    the low nibble of byte k // 2 for even k and the high nibble for odd k.
  * The output is float32 [T, N] (the reference returns float64).
  * E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa; exponent 0
    is subnormal: m * 0.5 (OCP Microscaling Formats v1.0, FP4 E2M1).
  * E4M3 ("E4M3FN"): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
    mantissa; exponent 0 is subnormal m/8 * 2^-6; S.1111.111 is NaN; no
    infinities (OCP 8-bit floating point specification, E4M3).

Pins: tests/test_w4a16_oracle.py.
"""
from __future__ import annotations

import numpy as np


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code."""
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        mag = man * 0.5
    else:
        mag = (1.0 + man / 2.0) * 2.0 ** (exp - 1)
    return sign * mag


def e4m3_value(byte: int) -> float:
    """Value of an E4M3 (FN) byte; NaN for S.1111.111."""
    sign = -1.0 if byte & 0x80 else 1.0
    exp = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        mag = (man / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return sign * mag


def ue8m0_value(byte: int) -> float:
    """Value of a UE8M0 (E8M0) scale byte: 2^(byte - 127); 0xFF is NaN."""
    if byte == 0xFF:
        return float("nan")
    return 2.0 ** (byte - 127)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)
UE8M0_TABLE = np.array([ue8m0_value(b) for b in range(256)], dtype=np.float64)
# weights per scale and scale byte table of each weight format
FORMATS = {"nvfp4": (16, E4M3_TABLE), "mxfp4": (32, UE8M0_TABLE)}


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16)."""
    u32 = np.asarray(bits, dtype=np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def unpack_codes(w_packed: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] -> E2M1 codes [..., K] (even k: low nibble)."""
    w = np.asarray(w_packed, dtype=np.uint8)
    out = np.empty(w.shape[:-1] + (2 * w.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = w & 0x0F
    out[..., 1::2] = w >> 4
    return out


def dequant_weights(w_packed: np.ndarray, scales: np.ndarray, fmt: str = "nvfp4") -> np.ndarray:
    """Dense float64 weights [..., N, K] = e2m1(code) * value of the scale of
    its block (16 weights, E4M3 for NVFP4; 32 weights, UE8M0 for MXFP4)."""
    block, table = FORMATS[fmt]
    codes = unpack_codes(w_packed)
    K = codes.shape[-1]
    s = table[np.asarray(scales, dtype=np.uint8)]               # [..., N, K/block]
    return E2M1_TABLE[codes] * np.repeat(s, block, axis=-1)[..., :K]


def moe_w4a16(x_bits: np.ndarray, w_packed: np.ndarray, scales: np.ndarray, alpha: np.ndarray,
              expert_start: np.ndarray, experts=None, fmt: str = "nvfp4"):
    """Reference output y (float64 [T, N]) and the bound sum |x * w| * |alpha|
    per output (float64 [T, N]) for the routed projection.  ``experts``
    limits the computation to those expert indices (rows of other tokens stay 0)."""
    x = bf16_to_f64(x_bits)
    T, K = x.shape
    E, N = w_packed.shape[0], w_packed.shape[1]
    block = FORMATS[fmt][0]
    assert w_packed.shape[2] * 2 == K and scales.shape == (E, N, K // block)
    es = np.asarray(expert_start, dtype=np.int64)
    y = np.zeros((T, N), dtype=np.float64)
    mag = np.zeros((T, N), dtype=np.float64)
    for e in (range(E) if experts is None else experts):
        t0, t1 = es[e], es[e + 1]
        if t1 <= t0:
            continue
        w = dequant_weights(w_packed[e], scales[e], fmt)         # [N, K]
        a = float(np.float32(alpha[e]))
        y[t0:t1] = a * (x[t0:t1] @ w.T)
        mag[t0:t1] = abs(a) * (np.abs(x[t0:t1]) @ np.abs(w).T)
    return y, mag
