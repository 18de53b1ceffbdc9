"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError on
a mismatch.  ``test_oracle.py`` runs them on the shipped oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with planted
mistakes and requires every mistake to be caught by at least one pin.

What pins what:
  * pin_two_column_closed_form: all 65,536 two-value rows, both formats, against
    the closed form of the base rule (base = smaller value; the larger one is an
    exception iff the two are at least W apart).
  * pin_base_optimal: on random rows, the chosen base leaves the fewest
    out-of-window values over all 256 candidate bytes, and is the smallest
    present value doing so.
  * pin_nvfp4_layout_bytes / pin_mxfp4_layout_bits / pin_exception_entries:
    hand-worked offset bytes and exception words for small planes.
  * pin_round_trip_*: decode(encode(x)) == x, x being the generator's input.
  * pin_window_invariant: every stored offset is x - base < W; every exception
    byte lies outside its row's window; entries ascend within each expert.
  * pin_special_cases: one-column rows, constant rows, widely spaced rows.
  * pin_window_does_not_wrap: a base above 240 keeps values below it out of
    the window.
  * pin_routed_subsets: every subset of routed experts leaves inactive planes
    byte-identical to the poison and active planes equal to x.
  * pin_alternative_bases: any per-row base decodes back to x.
  * pin_out_of_plane_entries: entries past the plane are ignored.
"""
from __future__ import annotations

import itertools

import numpy as np

import workloads

POISON = 0xA5


def _W(orc, fmt):
    return 1 << orc.offset_bits(fmt)


def pin_two_column_closed_form(orc):
    a, b = np.meshgrid(np.arange(256), np.arange(256), indexing="ij")
    x = np.stack([a.ravel(), b.ravel()], axis=1).astype(np.uint8).reshape(1, 65536, 2)
    lo = np.minimum(a, b).ravel()
    hi = np.maximum(a, b).ravel()
    for fmt in (workloads.NVFP4, workloads.MXFP4):
        W = _W(orc, fmt)
        st = orc.encode(fmt, x)
        assert np.array_equal(st["bases"], lo.astype(np.uint8)), "base of a two-value row is its smaller value"
        far = (hi - lo) >= W
        rows = (st["exceptions"] >> 8) // 2
        assert np.array_equal(np.sort(rows), np.nonzero(far)[0]), "one exception exactly for rows spanning >= W"
        col = (st["exceptions"] >> 8) % 2
        val = st["exceptions"] & 0xFF
        xr = x.reshape(-1, 2)
        assert np.array_equal(val, xr[rows, col]), "exception holds the original byte"
        assert np.array_equal(val, hi[rows]), "the exception is the larger value"
        assert st["prefix"][0] == 0 and st["prefix"][1] == far.sum()
        assert np.array_equal(orc.decode(st), x)


def _brute_force_base(rows: np.ndarray, W: int):
    """Smallest present value v maximising #{c : v <= x_c <= v+W-1}; plus the
    fewest out-of-window values over all 256 candidate bases."""
    v = np.arange(256)[None, :, None]
    xr = rows[:, None, :].astype(np.int64)
    inside = ((xr >= v) & (xr <= v + W - 1)).sum(axis=2)  # (N, 256)
    present = np.zeros((rows.shape[0], 256), dtype=bool)
    np.put_along_axis(present, rows.astype(np.int64), True, axis=1)
    masked = np.where(present, inside, -1)
    base = masked.argmax(axis=1)  # first maximum = smallest v
    fewest_out = rows.shape[1] - inside.max(axis=1)
    return base.astype(np.uint8), fewest_out


def pin_base_optimal(orc):
    rng = np.random.default_rng(1234)
    cases = [
        (workloads.NVFP4, workloads.TINY.generate()),
        (workloads.NVFP4, workloads.nvfp4_stack(2, 300, 50, 7, 0.10, hot_row_frac=0.05)),
        (workloads.NVFP4, rng.integers(0, 256, (1, 400, 33), dtype=np.uint8)),
        (workloads.NVFP4, rng.integers(0x20, 0x50, (1, 400, 64), dtype=np.uint8)),
        (workloads.NVFP4, rng.integers(240, 256, (1, 100, 9), dtype=np.uint8)),
        (workloads.MXFP4, workloads.mxfp4_stack(2, 200, 160, 5, 0.15)),
        (workloads.MXFP4, rng.integers(0, 256, (1, 400, 17), dtype=np.uint8)),
        (workloads.MXFP4, rng.integers(120, 126, (1, 400, 40), dtype=np.uint8)),
    ]
    for fmt, x in cases:
        E, R, C = x.shape
        W = _W(orc, fmt)
        bases = orc.choose_bases(fmt, x)
        want, fewest = _brute_force_base(x.reshape(E * R, C), W)
        assert np.array_equal(bases.reshape(-1), want), f"base rule, fmt {fmt}, shape {x.shape}"
        st = orc.encode(fmt, x)
        row_of = np.repeat(np.arange(E), np.diff(st["prefix"])) * R + (st["exceptions"] >> 8) // C
        per_row = np.bincount(row_of.astype(np.int64), minlength=E * R)
        assert np.array_equal(per_row, fewest), "exceptions per row are the fewest any base allows"


def pin_nvfp4_layout_bytes(orc):
    # One row of 64 values: positions 0..63 -> two 16-byte groups of 32 positions.
    # Base 0x30 (every value is inside [0x30, 0x3F]).
    c = np.arange(64)
    # (a) field = c % 16: group byte j holds position j (low nibble) and j+16
    #     (high nibble), both with field j, so every byte is 0x11 * j.
    x = (0x30 + (c % 16)).astype(np.uint8).reshape(1, 1, 64)
    st = orc.encode(workloads.NVFP4, x)
    want = bytes([0x00, 0x11, 0x22, 0x33, 0x44, 0x55, 0x66, 0x77,
                  0x88, 0x99, 0xAA, 0xBB, 0xCC, 0xDD, 0xEE, 0xFF]) * 2
    assert st["bases"].tolist() == [0x30]
    assert st["offsets"].tobytes() == want
    # (b) field = c // 16 (0,1,2,3 per run of 16): group 0 low nibbles 0, high 1;
    #     group 1 low nibbles 2, high 3.
    x = (0x30 + (c // 16)).astype(np.uint8).reshape(1, 1, 64)
    st = orc.encode(workloads.NVFP4, x)
    assert st["offsets"].tobytes() == bytes([0x10] * 16 + [0x32] * 16)
    # (c) a 40-column row: one full group plus 8 positions of a second group;
    #     fields past the plane stay zero.  Values 0x40 + (c % 16) with base 0x40.
    x = (0x40 + (np.arange(40) % 16)).astype(np.uint8).reshape(1, 1, 40)
    st = orc.encode(workloads.NVFP4, x)
    assert st["stride"] == 32
    got = st["offsets"]
    assert got[:16].tobytes() == want[:16]
    # positions 32..39 -> group 1 bytes 0..7 low nibble = 0..7; all else 0
    assert got[16:].tobytes() == bytes(list(range(8)) + [0] * 8)


def pin_mxfp4_layout_bits(orc):
    base = 120
    hand = {0: (0, 0x01), 17: (1, 0x02), 40: (8, 0x04), 127: (15, 0x80), 112: (0, 0x80)}
    for q in range(128):
        x = np.full((1, 1, 128), base, dtype=np.uint8)
        x[0, 0, q] = base + 1
        st = orc.encode(workloads.MXFP4, x)
        assert st["bases"].tolist() == [base] and st["exceptions"].size == 0
        off = st["offsets"]
        assert off.size == 16 and np.count_nonzero(off) == 1
        if q in hand:
            j, bit = hand[q]
            assert off[j] == bit, f"position {q}"
        # contiguous decoding: bit f of the 16 bytes is positions 16f .. 16f+15
        for f in range(8):
            run = (off >> f) & 1
            assert np.array_equal(run, (x[0, 0, 16 * f:16 * f + 16] - base)), f"position {q} field {f}"


def pin_exception_entries(orc):
    # Row [0x30, 0x31, 0x90, 0x3F]: base 0x30; 0x90 at position 2 is the only
    # exception -> word (2 << 8) | 0x90; its field is 0.
    x = np.array([[[0x30, 0x31, 0x90, 0x3F]]], dtype=np.uint8)
    st = orc.encode(workloads.NVFP4, x)
    assert st["bases"].tolist() == [0x30]
    assert st["exceptions"].tolist() == [0x290]
    assert st["prefix"].tolist() == [0, 1]
    assert st["offsets"].tobytes() == bytes([0x00, 0x01, 0x00, 0x0F] + [0] * 12)
    # Two experts, 2 rows x 3 columns: entries are plane-local and expert-major.
    x = np.array([[[10, 200, 11], [50, 50, 49]],
                  [[7, 7, 7], [0, 255, 128]]], dtype=np.uint8)
    st = orc.encode(workloads.NVFP4, x)
    # expert 0 row 0: base 10, 200 at p=1; row 1: base 49 (window 49..64).
    # expert 1 row 0: base 7; row 1: base 0, exceptions 255 at p=4, 128 at p=5.
    assert st["bases"].tolist() == [10, 49, 7, 0]
    assert st["exceptions"].tolist() == [(1 << 8) | 200, (4 << 8) | 255, (5 << 8) | 128]
    assert st["prefix"].tolist() == [0, 1, 3]


def pin_round_trip_generated(orc):
    for spec in (workloads.TINY,):
        x = spec.generate()
        st = orc.encode(spec.fmt, x)
        assert np.array_equal(orc.decode(st), x)
    x = workloads.nvfp4_stack(3, 100, 50, 11, 0.10, hot_row_frac=0.01)
    assert np.array_equal(orc.decode(orc.encode(workloads.NVFP4, x)), x)
    x = workloads.mxfp4_stack(3, 64, 160, 12, 0.15)
    assert np.array_equal(orc.decode(orc.encode(workloads.MXFP4, x)), x)


def pin_round_trip_uniform(orc):
    for fmt in (workloads.NVFP4, workloads.MXFP4):
        for shape in [(3, 17, 13), (2, 5, 1), (1, 1, 1), (2, 9, 300), (4, 33, 7)]:
            x = workloads.uniform_bytes(*shape, seed=sum(shape) + fmt)
            assert np.array_equal(orc.decode(orc.encode(fmt, x)), x), (fmt, shape)


def pin_window_invariant(orc):
    for fmt, x in ((workloads.NVFP4, workloads.TINY.generate()),
                   (workloads.MXFP4, workloads.mxfp4_stack(2, 50, 160, 3, 0.15)),
                   (workloads.NVFP4, workloads.uniform_bytes(2, 40, 24, 9))):
        E, R, C = x.shape
        W = _W(orc, fmt)
        st = orc.encode(fmt, x)
        pfx = st["prefix"]
        base = st["bases"].reshape(E, R)[:, :, None].astype(np.int64)
        d = x.astype(np.int64) - base
        outside = (d < 0) | (d >= W)
        assert pfx[0] == 0 and np.all(np.diff(pfx) >= 0) and pfx[-1] == st["exceptions"].size
        assert pfx[-1] == outside.sum(), "exceptions are exactly the out-of-window values"
        for e in range(E):
            ent = st["exceptions"][pfx[e]:pfx[e + 1]]
            pos = (ent >> 8).astype(np.int64)
            assert np.all(np.diff(pos) > 0) and np.all(pos < R * C)
            assert np.array_equal(np.sort(pos), np.nonzero(outside[e].ravel())[0])
            assert np.array_equal(ent & 0xFF, x[e].ravel()[pos])
        # every in-window offset is stored; exception positions hold field 0
        w = orc.offset_bits(fmt)
        G = 128 // w
        S = st["stride"]
        p = np.arange(R * C)
        byte_idx = 16 * (p // G) + p % 16
        shift = w * ((p % G) // 16)
        for e in range(E):
            seg = st["offsets"][e * S:(e + 1) * S].astype(np.int64)
            field = (seg[byte_idx] >> shift) & (W - 1)
            want = np.where(outside[e].ravel(), 0, d[e].ravel())
            assert np.array_equal(field, want)


def pin_special_cases(orc):
    # one column: base = the value, no exceptions, zero fields
    x = workloads.uniform_bytes(3, 50, 1, 5)
    for fmt in (workloads.NVFP4, workloads.MXFP4):
        st = orc.encode(fmt, x)
        assert np.array_equal(st["bases"], x.reshape(-1))
        assert st["exceptions"].size == 0 and not st["offsets"].any()
    # constant rows: base = the value, all fields zero
    x = np.repeat(np.arange(0, 256, 17, dtype=np.uint8)[None, :, None], 37, axis=2)
    for fmt in (workloads.NVFP4, workloads.MXFP4):
        st = orc.encode(fmt, x)
        assert np.array_equal(st["bases"], x[0, :, 0])
        assert st["exceptions"].size == 0 and not st["offsets"].any()
    # values spaced >= W apart: base = smallest, every other value an exception
    x = np.array([[[200, 16, 48, 32, 0, 255]]], dtype=np.uint8)
    st = orc.encode(workloads.NVFP4, x)
    assert st["bases"].tolist() == [0] and st["exceptions"].size == 5
    x = np.array([[[9, 3, 5, 7, 1]]], dtype=np.uint8)
    st = orc.encode(workloads.MXFP4, x)
    assert st["bases"].tolist() == [1] and st["exceptions"].size == 4
    # MXFP4 rows of {b, b+1} only: no exceptions, field = value - b
    x = np.array([[[121, 120, 120, 121, 121]]], dtype=np.uint8)
    st = orc.encode(workloads.MXFP4, x)
    assert st["bases"].tolist() == [120] and st["exceptions"].size == 0
    assert st["offsets"][:5].tolist() == [1, 0, 0, 1, 1]


def pin_window_does_not_wrap(orc):
    # Base 250: the window is 250..255 only; 0..9 lie below the base and are
    # exceptions, not offsets 6..15 of a window wrapping past 255.
    x = np.array([[[250, 250, 250, 0, 1, 9, 255, 252]]], dtype=np.uint8)
    st = orc.encode(workloads.NVFP4, x)
    assert st["bases"].tolist() == [250]
    assert st["exceptions"].tolist() == [(3 << 8) | 0, (4 << 8) | 1, (5 << 8) | 9]
    assert st["offsets"][:8].tolist() == [0, 0, 0, 0, 0, 0, 5, 2]
    x = np.array([[[255, 255, 255, 0, 0]]], dtype=np.uint8)
    st = orc.encode(workloads.MXFP4, x)
    assert st["bases"].tolist() == [255]
    assert st["exceptions"].tolist() == [(3 << 8) | 0, (4 << 8) | 0]


def pin_routed_subsets(orc):
    x = workloads.TINY.generate()
    E = x.shape[0]
    st = orc.encode(workloads.TINY.fmt, x)
    for mask in itertools.product([0, 1], repeat=E):
        es = workloads.expert_start_from_mask(np.array(mask), tokens=3)
        ws = np.full(x.shape, POISON, dtype=np.uint8)
        orc.decode(st, es, ws)
        for e in range(E):
            if mask[e]:
                assert np.array_equal(ws[e], x[e])
            else:
                assert np.all(ws[e] == POISON)
    # non-increasing expert_start entries count as "no tokens"
    es = np.array([0, 5, 5, 3, 9], dtype=np.int32)
    ws = np.full(x.shape, POISON, dtype=np.uint8)
    orc.decode(st, es, ws)
    assert np.array_equal(ws[0], x[0]) and np.all(ws[1] == POISON)
    assert np.all(ws[2] == POISON) and np.array_equal(ws[3], x[3])


def pin_alternative_bases(orc):
    rng = np.random.default_rng(77)
    for fmt in (workloads.NVFP4, workloads.MXFP4):
        x = workloads.uniform_bytes(3, 20, 21, 31 + fmt)
        bases = rng.integers(0, 256, (3, 20), dtype=np.uint8)
        st = orc.encode_with_bases(fmt, x, bases)
        assert np.array_equal(orc.decode(st), x)


def pin_out_of_plane_entries(orc):
    # Two 16-byte planes; expert 0 carries entries at p = 16 and p = 20, which
    # would land in expert 1's plane if they were not dropped.
    x = np.full((2, 2, 8), 0x40, dtype=np.uint8)
    st = dict(orc.encode(workloads.NVFP4, x))
    st["exceptions"] = np.array([(3 << 8) | 0x99, (16 << 8) | 0x77, (20 << 8) | 0x11,
                                 (4000 << 8) | 0x22], dtype=np.uint32)
    st["prefix"] = np.array([0, 4, 4], dtype=np.int32)
    out = orc.decode(st)
    want = x.copy()
    want[0, 0, 3] = 0x99
    assert np.array_equal(out, want)
    # with expert 1 routed off its poisoned plane must stay intact
    ws = np.full(x.shape, POISON, dtype=np.uint8)
    orc.decode(st, np.array([0, 1, 1], dtype=np.int32), ws)
    assert np.array_equal(ws[0], want[0]) and np.all(ws[1] == POISON)


def pin_row_window(orc):
    # Rows begin .. end-1 of every routed plane equal the input x; every other
    # byte keeps the poison (the round trip, restricted to the window).
    cases = [(workloads.NVFP4, workloads.nvfp4_stack(3, 40, 50, 5, 0.10, hot_row_frac=0.05)),
             (workloads.MXFP4, workloads.mxfp4_stack(2, 24, 160, 6, 0.15)),
             (workloads.NVFP4, workloads.uniform_bytes(2, 9, 7, 12))]
    rng = np.random.default_rng(5)
    for fmt, x in cases:
        E, R, C = x.shape
        st = orc.encode(fmt, x)
        windows = [(0, R), (0, R // 2), (R // 2, R), (0, 0), (R, R), (0, 1), (R - 1, R)]
        windows += [tuple(sorted(rng.integers(0, R + 1, 2))) for _ in range(4)]
        for b, e in windows:
            for es in (None, workloads.expert_start_from_mask(np.arange(E) % 2 == 0, tokens=1)):
                ws = np.full(x.shape, POISON, dtype=np.uint8)
                orc.decode_rows(st, b, e, es, ws)
                for k in range(E):
                    if es is not None and not es[k + 1] > es[k]:
                        assert np.all(ws[k] == POISON)
                        continue
                    assert np.array_equal(ws[k, b:e], x[k, b:e]), (b, e)
                    assert np.all(ws[k, :b] == POISON) and np.all(ws[k, e:] == POISON), (b, e)
        # a window outside the plane is refused
        for b, e in ((-1, 2), (3, 2), (0, R + 1)):
            try:
                orc.decode_rows(st, b, e)
            except ValueError:
                continue
            raise AssertionError(f"window {(b, e)} accepted")


def pin_index_hand_worked(orc):
    # Two experts, one row of 5000 columns: tiles [0, 2048), [2048, 4096), [4096, 5000).
    # Expert 0 outliers at 5, 2047, 2048, 4999; expert 1 outliers at 100, 4096.
    x = np.full((2, 1, 5000), 0x30, dtype=np.uint8)
    for p in (5, 2047, 2048, 4999):
        x[0, 0, p] = 0x90
    for p in (100, 4096):
        x[1, 0, p] = 0x90
    st = orc.encode(workloads.NVFP4, x)
    assert st["prefix"].tolist() == [0, 4, 6]
    assert orc.index_tiles(1, 5000) == 3
    assert st["tile_index"].tolist() == [0, 2, 3, 4, 5, 5, 6]
    # exactly one tile per plane, and a plane of exactly two tiles
    assert orc.index_tiles(1, 2048) == 1 and orc.index_tiles(2, 2048) == 2


def pin_index_covers_entries(orc):
    for fmt, x in ((workloads.NVFP4, workloads.nvfp4_stack(3, 300, 50, 9, 0.10, hot_row_frac=0.02)),
                   (workloads.MXFP4, workloads.mxfp4_stack(2, 100, 160, 8, 0.15)),
                   (workloads.NVFP4, workloads.uniform_bytes(2, 3, 7, 1))):
        E, R, C = x.shape
        st = orc.encode(fmt, x)
        ti, pfx = st["tile_index"], st["prefix"]
        NT = orc.index_tiles(R, C)
        assert ti.size == E * NT + 1 and ti[-1] == pfx[-1]
        assert np.all(np.diff(ti) >= 0)
        pos = (st["exceptions"] >> 8).astype(np.int64)
        for e in range(E):
            assert ti[e * NT] == pfx[e]
            for j in range(NT):
                lo, hi = ti[e * NT + j], ti[e * NT + j + 1]
                assert np.all((pos[lo:hi] >= 2048 * j) & (pos[lo:hi] < 2048 * (j + 1)))


ALL_PINS = [
    pin_window_does_not_wrap,
    pin_index_hand_worked,
    pin_index_covers_entries,
    pin_two_column_closed_form,
    pin_base_optimal,
    pin_nvfp4_layout_bytes,
    pin_mxfp4_layout_bits,
    pin_exception_entries,
    pin_round_trip_generated,
    pin_round_trip_uniform,
    pin_window_invariant,
    pin_special_cases,
    pin_routed_subsets,
    pin_alternative_bases,
    pin_out_of_plane_entries,
    pin_row_window,
]
