"""CPU oracle for the CSF block-scale codec (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product library never loads it and shares no code with it.

Thin ctypes wrapper over ``libcsf_oracle.so`` (built from ``csf_oracle.c`` by
``oracle/build.py``); every computation happens in that C file.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

NVFP4 = 0
MXFP4 = 1

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_i32p = ctypes.POINTER(ctypes.c_int32)


def _ptr(a: np.ndarray | None, t):
    if a is None:
        return ctypes.cast(None, t)
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(t)


class Oracle:
    """Handle on one compiled oracle library (the default one, or a test variant)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_offset_bits.argtypes = [ctypes.c_int]
        lib.oracle_offset_bits.restype = ctypes.c_int
        lib.oracle_segment_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.oracle_segment_bytes.restype = ctypes.c_int64
        lib.oracle_choose_bases.argtypes = [ctypes.c_int] * 4 + [_u8p, _u8p]
        lib.oracle_choose_bases.restype = ctypes.c_int
        lib.oracle_count_exceptions.argtypes = [ctypes.c_int] * 4 + [_u8p, _u8p]
        lib.oracle_count_exceptions.restype = ctypes.c_int64
        lib.oracle_encode_streams.argtypes = [ctypes.c_int] * 4 + [_u8p, _u8p, _u8p, _u32p, _i32p]
        lib.oracle_encode_streams.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [ctypes.c_int] * 4 + [_u8p, _u8p, _u32p, _i32p, _i32p, _u8p]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_decode_rows.argtypes = ([ctypes.c_int] * 4 + [_u8p, _u8p, _u32p, _i32p, _i32p]
                                           + [ctypes.c_int] * 2 + [_u8p])
        lib.oracle_decode_rows.restype = ctypes.c_int
        lib.oracle_index_tiles.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.oracle_index_tiles.restype = ctypes.c_int64
        lib.oracle_build_index.argtypes = [ctypes.c_int] * 3 + [_u32p, _i32p, _i32p]
        lib.oracle_build_index.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    # -- format constants -------------------------------------------------
    def offset_bits(self, fmt: int) -> int:
        return self.lib.oracle_offset_bits(fmt)

    def segment_bytes(self, fmt: int, R: int, C: int) -> int:
        return int(self.lib.oracle_segment_bytes(fmt, R, C))

    # -- encoder ------------------------------------------------------------
    def choose_bases(self, fmt: int, x: np.ndarray) -> np.ndarray:
        E, R, C = x.shape
        x = np.ascontiguousarray(x, dtype=np.uint8)
        bases = np.empty((E, R), dtype=np.uint8)
        rc = self.lib.oracle_choose_bases(fmt, E, R, C, _ptr(x, _u8p), _ptr(bases, _u8p))
        if rc != 0:
            raise ValueError(f"oracle_choose_bases rejected shape {x.shape} fmt {fmt}")
        return bases

    def encode_with_bases(self, fmt: int, x: np.ndarray, bases: np.ndarray) -> dict:
        """Offsets, exceptions and prefix for caller-chosen row bases."""
        E, R, C = x.shape
        x = np.ascontiguousarray(x, dtype=np.uint8)
        bases = np.ascontiguousarray(bases, dtype=np.uint8).reshape(E, R)
        n = int(self.lib.oracle_count_exceptions(fmt, E, R, C, _ptr(x, _u8p), _ptr(bases, _u8p)))
        if n < 0:
            raise ValueError(f"oracle rejected shape {x.shape} fmt {fmt}")
        S = self.segment_bytes(fmt, R, C)
        offsets = np.empty(E * S, dtype=np.uint8)
        exc = np.empty(max(n, 1), dtype=np.uint32)
        prefix = np.empty(E + 1, dtype=np.int32)
        rc = self.lib.oracle_encode_streams(fmt, E, R, C, _ptr(x, _u8p), _ptr(bases, _u8p),
                                            _ptr(offsets, _u8p), _ptr(exc, _u32p),
                                            _ptr(prefix, _i32p))
        if rc != 0:
            raise ValueError("oracle_encode_streams failed")
        st = dict(fmt=fmt, E=E, R=R, C=C, stride=S, bases=bases.reshape(-1).copy(),
                  offsets=offsets, exceptions=exc[:n].copy(), prefix=prefix)
        st["tile_index"] = self.build_index(st)
        return st

    def encode(self, fmt: int, x: np.ndarray) -> dict:
        return self.encode_with_bases(fmt, x, self.choose_bases(fmt, x))

    def index_tiles(self, R: int, C: int) -> int:
        return int(self.lib.oracle_index_tiles(R, C))

    def build_index(self, stack: dict) -> np.ndarray:
        """Per-tile exception index of a stack (int32[E * tiles + 1])."""
        E, R, C = stack["E"], stack["R"], stack["C"]
        exc = np.ascontiguousarray(stack["exceptions"], dtype=np.uint32)
        if exc.size == 0:
            exc = np.zeros(1, dtype=np.uint32)
        out = np.empty(E * self.index_tiles(R, C) + 1, dtype=np.int32)
        rc = self.lib.oracle_build_index(E, R, C, _ptr(exc, _u32p),
                                         _ptr(np.ascontiguousarray(stack["prefix"], dtype=np.int32), _i32p),
                                         _ptr(out, _i32p))
        if rc != 0:
            raise ValueError("oracle_build_index rejected its arguments")
        return out

    # -- decoder ------------------------------------------------------------
    def decode(self, stack: dict, expert_start: np.ndarray | None = None,
               ws: np.ndarray | None = None) -> np.ndarray:
        """Expand ``stack`` into ``ws`` (uint8[E, R, C]); returns ``ws``.

        With ``expert_start`` only routed experts are written, so pass a
        pre-filled ``ws`` to see the untouched planes.
        """
        fmt, E, R, C = stack["fmt"], stack["E"], stack["R"], stack["C"]
        if ws is None:
            ws = np.zeros((E, R, C), dtype=np.uint8)
        assert ws.shape == (E, R, C) and ws.dtype == np.uint8 and ws.flags["C_CONTIGUOUS"]
        exc = np.ascontiguousarray(stack["exceptions"], dtype=np.uint32)
        if exc.size == 0:
            exc = np.zeros(1, dtype=np.uint32)
        es = None if expert_start is None else np.ascontiguousarray(expert_start, dtype=np.int32)
        if es is not None:
            assert es.shape == (E + 1,)
        rc = self.lib.oracle_decode(fmt, E, R, C,
                                    _ptr(np.ascontiguousarray(stack["bases"], dtype=np.uint8), _u8p),
                                    _ptr(np.ascontiguousarray(stack["offsets"], dtype=np.uint8), _u8p),
                                    _ptr(exc, _u32p),
                                    _ptr(np.ascontiguousarray(stack["prefix"], dtype=np.int32), _i32p),
                                    _ptr(es, _i32p), _ptr(ws, _u8p))
        if rc != 0:
            raise ValueError("oracle_decode rejected its arguments")
        return ws


    def decode_experts(self, stack: dict, e0: int, e1: int, ws: np.ndarray,
                       expert_start: np.ndarray | None = None) -> None:
        """``decode`` of experts e0 .. e1-1 only, into their planes of ``ws``
        (uint8[E, R, C], C-contiguous): the same C function called on the
        sub-stack those experts form (their bases, offset segments, prefix
        entries and planes; entry indices stay those of the whole stream).
        Several threads may decode disjoint expert ranges at once; the call
        releases the GIL."""
        fmt, E, R, C = stack["fmt"], stack["E"], stack["R"], stack["C"]
        assert 0 <= e0 <= e1 <= E and ws.shape == (E, R, C) and ws.dtype == np.uint8 and ws.flags["C_CONTIGUOUS"]
        if e0 == e1:
            return
        S = self.segment_bytes(fmt, R, C)
        bases = np.ascontiguousarray(stack["bases"], dtype=np.uint8)
        offsets = np.ascontiguousarray(stack["offsets"], dtype=np.uint8)
        prefix = np.ascontiguousarray(stack["prefix"], dtype=np.int32)
        exc = np.ascontiguousarray(stack["exceptions"], dtype=np.uint32)
        if exc.size == 0:
            exc = np.zeros(1, dtype=np.uint32)
        es = None
        if expert_start is not None:
            es = np.ascontiguousarray(expert_start, dtype=np.int32)
            assert es.shape == (E + 1,)
        at = lambda a, off, t: ctypes.cast(a.ctypes.data + off, t)
        rc = self.lib.oracle_decode(fmt, e1 - e0, R, C, at(bases, e0 * R, _u8p), at(offsets, e0 * S, _u8p),
                                    _ptr(exc, _u32p), at(prefix, 4 * e0, _i32p),
                                    at(es, 4 * e0, _i32p) if es is not None else ctypes.cast(None, _i32p),
                                    at(ws, e0 * R * C, _u8p))
        if rc != 0:
            raise ValueError("oracle_decode rejected its arguments")

    def decode_rows(self, stack: dict, row_begin: int, row_end: int,
                    expert_start: np.ndarray | None = None, ws: np.ndarray | None = None) -> np.ndarray:
        """Expand rows ``row_begin .. row_end-1`` of every (routed) plane into
        ``ws`` (uint8[E, R, C]); every other byte of ``ws`` keeps its value."""
        fmt, E, R, C = stack["fmt"], stack["E"], stack["R"], stack["C"]
        if ws is None:
            ws = np.zeros((E, R, C), dtype=np.uint8)
        assert ws.shape == (E, R, C) and ws.dtype == np.uint8 and ws.flags["C_CONTIGUOUS"]
        exc = np.ascontiguousarray(stack["exceptions"], dtype=np.uint32)
        if exc.size == 0:
            exc = np.zeros(1, dtype=np.uint32)
        es = None if expert_start is None else np.ascontiguousarray(expert_start, dtype=np.int32)
        if es is not None:
            assert es.shape == (E + 1,)
        rc = self.lib.oracle_decode_rows(fmt, E, R, C,
                                         _ptr(np.ascontiguousarray(stack["bases"], dtype=np.uint8), _u8p),
                                         _ptr(np.ascontiguousarray(stack["offsets"], dtype=np.uint8), _u8p),
                                         _ptr(exc, _u32p),
                                         _ptr(np.ascontiguousarray(stack["prefix"], dtype=np.int32), _i32p),
                                         _ptr(es, _i32p), int(row_begin), int(row_end), _ptr(ws, _u8p))
        if rc != 0:
            raise ValueError("oracle_decode_rows rejected its arguments")
        return ws


_default: Oracle | None = None


def load(rebuild: bool = False) -> Oracle:
    """The oracle built from ``csf_oracle.c`` (compiled on first use)."""
    global _default
    if _default is None or rebuild:
        path = _build.LIBRARY
        if rebuild or not os.path.exists(path) or (
                os.path.getmtime(path) < os.path.getmtime(_build.SOURCE)):
            _build.build()
        _default = Oracle(path)
    return _default
