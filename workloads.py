"""Seeded synthetic inputs for the CSF block-scale decoder.

This module only draws input bytes (dense scale planes and routing metadata).
It holds none of the codec's arithmetic: no base choice, no offset packing, no
exception stream.  Both the CPU oracle tests and the GPU path take their inputs
from here, so the two never share anything beyond the input bytes.

The value distributions imitate the stacks the pages measure (512-expert
Qwen gate/down projections and a 384-expert MXFP4 projection): each row's
scales cluster just above a per-row base byte, with a minority of outliers.
The pages' real checkpoint streams are not available; these stand in for them.

Every array is drawn whole, in a fixed call order, from ``numpy.random.
default_rng(seed)`` (PCG64), so a (config, seed) pair always gives the same
bytes on every machine.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

NVFP4 = 0  # E4M3 scale per 16 weights
MXFP4 = 1  # UE8M0 scale per 32 weights

WEIGHTS_PER_SCALE = {NVFP4: 16, MXFP4: 32}


def nvfp4_stack(E: int, R: int, C: int, seed: int, exc_rate: float,
                hot_row_frac: float = 0.0) -> np.ndarray:
    """Dense E4M3 scale bytes ``uint8[E, R, C]``.

    In-window values are ``base + U{0..15}`` with a per-row base drawn from
    U[0x28, 0x48].  Outliers are uniform over the finite E4M3 encodings (every
    byte except 0x7F and 0xFF) that lie outside ``[base, base + 15]``: 238
    candidates.  With ``hot_row_frac > 0`` that fraction of rows is made of
    outliers only, and the other rows draw outliers at the rate that keeps the
    overall rate at ``exc_rate``.
    """
    rng = np.random.default_rng(seed)
    base = rng.integers(0x28, 0x48, (E, R), endpoint=True, dtype=np.uint8)
    off = rng.integers(0, 16, (E, R, C), dtype=np.uint8)
    if hot_row_frac > 0.0:
        n_hot = int(round(hot_row_frac * E * R))
        hot = rng.choice(E * R, n_hot, replace=False)
        p = (exc_rate - hot_row_frac) / (1.0 - hot_row_frac)
    else:
        hot = None
        p = exc_rate
    exc = rng.random((E, R, C), dtype=np.float32) < np.float32(p)
    if hot is not None:
        exc.reshape(E * R, C)[hot, :] = True
    u = rng.integers(0, 238, (E, R, C), dtype=np.uint8).astype(np.uint16)
    b3 = base[:, :, None].astype(np.uint16)
    v = np.where(u < b3, u, u + 16)
    v = v + (v >= 0x7F)
    x = np.where(exc, v, b3 + off).astype(np.uint8)
    return x


def mxfp4_stack(E: int, R: int, C: int, seed: int, exc_rate: float) -> np.ndarray:
    """Dense UE8M0 scale bytes ``uint8[E, R, C]``.

    Per-row base U[118, 130]; in-window values ``base + {0, 1}``; outliers
    uniform over [100, 140] minus the row's two window bytes.
    """
    rng = np.random.default_rng(seed)
    base = rng.integers(118, 130, (E, R), endpoint=True, dtype=np.uint8)
    off = rng.integers(0, 2, (E, R, C), dtype=np.uint8)
    exc = rng.random((E, R, C), dtype=np.float32) < np.float32(exc_rate)
    u = rng.integers(0, 39, (E, R, C), dtype=np.uint8).astype(np.uint16)
    b3 = base[:, :, None].astype(np.uint16)
    v = 100 + u
    v = v + 2 * (v >= b3)
    x = np.where(exc, v, b3 + off).astype(np.uint8)
    return x


def uniform_bytes(E: int, R: int, C: int, seed: int) -> np.ndarray:
    """Worst-case input: every byte uniform over 0..255."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, (E, R, C), dtype=np.uint8)


def routing(E: int, n_active: int, max_tokens: int, seed: int) -> np.ndarray:
    """Grouped-routing ``expert_start`` (int32[E + 1]).

    ``n_active`` distinct experts drawn uniformly get U{1..max_tokens} tokens
    each; all others get none.  ``expert_start`` is the exclusive prefix of the
    per-expert token counts, i.e. offsets into the expert-sorted token list.
    """
    rng = np.random.default_rng(seed)
    act = rng.choice(E, n_active, replace=False)
    tok = rng.integers(1, max_tokens, n_active, endpoint=True)
    counts = np.zeros(E, dtype=np.int64)
    counts[act] = tok
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def expert_start_from_mask(active: np.ndarray, tokens: int = 1) -> np.ndarray:
    """``expert_start`` giving ``tokens`` tokens to each expert flagged in ``active``."""
    counts = np.asarray(active, dtype=np.int64) * tokens
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


@dataclass(frozen=True)
class StackSpec:
    name: str
    fmt: int
    E: int
    R: int
    C: int
    seed: int
    exc_rate: float
    hot_row_frac: float = 0.0
    desc: str = ""

    @property
    def K(self) -> int:
        return self.C * WEIGHTS_PER_SCALE[self.fmt]

    @property
    def dense_bytes(self) -> int:
        return self.E * self.R * self.C

    def generate(self) -> np.ndarray:
        if self.fmt == NVFP4:
            return nvfp4_stack(self.E, self.R, self.C, self.seed, self.exc_rate,
                               self.hot_row_frac)
        return mxfp4_stack(self.E, self.R, self.C, self.seed, self.exc_rate)


@dataclass(frozen=True)
class RoutedSpec:
    name: str
    stacks: tuple = field(default_factory=tuple)
    n_active: int = 8
    max_tokens: int = 64
    seed: int = 3
    desc: str = ""

    def expert_start(self) -> np.ndarray:
        return routing(self.stacks[0].E, self.n_active, self.max_tokens, self.seed)


# The five workloads.  Seeds: the tiny stack uses seed 0; the others use their
# 0-based position in this list.
TINY = StackSpec("tiny_nvfp4", NVFP4, 4, 64, 8, seed=0, exc_rate=0.05,
                 desc="4 experts x 64 rows x 8 scale columns (K=128), 5% outliers")
GATE = StackSpec("gate_nvfp4", NVFP4, 512, 800, 128, seed=1, exc_rate=0.03,
                 desc="512 experts x 800 rows x 128 scale columns (K=2048), 3% outliers")
DOWN = StackSpec("down_nvfp4", NVFP4, 512, 2048, 50, seed=2, exc_rate=0.10,
                 hot_row_frac=0.01,
                 desc="512 experts x 2048 rows x 50 scale columns (K=800), 10% outliers, "
                      "1% of rows all-outlier")
ROUTED = RoutedSpec("routed_paired", stacks=(GATE, DOWN), n_active=8, max_tokens=64,
                    seed=3, desc="gate + down stacks, 8 of 512 experts routed, "
                                 "1..64 tokens each")
MX = StackSpec("mxfp4", MXFP4, 384, 1024, 160, seed=4, exc_rate=0.15,
               desc="384 experts x 1024 rows x 160 scale columns (K=5120), 15% outliers")

STACKS = {s.name: s for s in (TINY, GATE, DOWN, MX)}


# -- W4A16 MoE projection inputs (the consumer of the decoded scales) ----------

@dataclass
class W4A16Inputs:
    x_bits: np.ndarray        # uint16 [T, K]: bfloat16 bit patterns of the routed tokens
    w_packed: np.ndarray      # uint8 [E, N, K/2]: two E2M1 codes per byte (even k low nibble)
    scales: np.ndarray        # uint8 [E, N, K/16] E4M3 (NVFP4) or [E, N, K/32] UE8M0 (MXFP4) scale bytes
    alpha: np.ndarray         # float32 [E]: per-expert tensor scale
    expert_start: np.ndarray  # int32 [E + 1]: grouped routing (tokens sorted by expert)
    fmt: int = NVFP4          # NVFP4 or MXFP4


def bf16_bits(T: int, K: int, rng) -> np.ndarray:
    """Random bfloat16 bit patterns: random sign and mantissa, exponent field
    in [118, 130] (magnitudes ~2^-9 .. 2^4), no zeros, NaNs or infinities."""
    sign = rng.integers(0, 2, (T, K), dtype=np.uint16) << 15
    exp = rng.integers(118, 131, (T, K), dtype=np.uint16) << 7
    man = rng.integers(0, 128, (T, K), dtype=np.uint16)
    return (sign | exp | man).astype(np.uint16)


def w4a16_inputs(E: int, N: int, K: int, expert_start: np.ndarray, seed: int,
                 exc_rate: float = 0.03, fmt: int = NVFP4) -> W4A16Inputs:
    """Seeded inputs of a routed NVFP4 or MXFP4 projection: scales shaped like
    the gate-like stack (nvfp4_stack with C = K / 16) or the MXFP4 stack
    (mxfp4_stack with C = K / 32), uniform random E2M1 codes, bfloat16
    activations for the routed tokens, alpha uniform in [0.5, 2)."""
    assert K % 32 == 0
    es = np.ascontiguousarray(expert_start, dtype=np.int32)
    T = int(es[-1])
    if fmt == NVFP4:
        scales = nvfp4_stack(E, N, K // 16, seed, exc_rate)
    else:
        scales = mxfp4_stack(E, N, K // 32, seed, exc_rate)
    rng = np.random.default_rng(seed + 1000)
    w = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    x = bf16_bits(T, K, rng)
    alpha = rng.uniform(0.5, 2.0, E).astype(np.float32)
    return W4A16Inputs(x, w, scales, alpha, es, fmt)
