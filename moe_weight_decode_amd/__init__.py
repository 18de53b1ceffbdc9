"""CSF block-scale decode for MI355X: Python binding of ``libcsf.so``.

Argument marshalling only: every decode step runs in the library's gfx950
kernels, and the binding has no other implementation to fall back to.  PyTorch
provides device memory and streams.  If the library has not been built, every
call raises ``RuntimeError`` (build it with ``python -m
moe_weight_decode_amd.build``).

The functions mirror the C ABI in ``include/csf.h``:

* ``prepare(dense, fmt)`` -> ``CompressedStack`` on ``dense``'s device
  (the preparation helper of "finegrained-kernels: decode losslessly
  compressed NVFP4 scales (CSF)", kernels-community PR 1236, API paragraph,
  which keeps the input's device): a GPU tensor is encoded on the GPU
  (``csf_encode_device``), host data by the host encoder (``csf_prepare``);
* ``decode(stack, workspace, expert_start=None, stream=None)``;
* ``decode_paired(gate_up, ws_gate_up, down, ws_down, expert_start=None, stream=None)``
  (``expert_start`` int32 or int64; int64 goes through ``csf_decode_i64``);
* ``decode_passes(...)`` to enqueue the fixed-stream or exception pass alone;
* ``decode_rows(...)`` to decode a window of rows of every plane (for example
  only the gate half of a gate/up stack);
* ``moe_w4a16(scales, weights, x, alpha, expert_start, ...)``: the routed
  W4A16 projection (NVFP4 or MXFP4 weights) that expands its scales in LDS
  from the CSF streams, or reads them from a dense workspace;
* ``Launch(...)``: a decode with its arguments marshalled once, for loops
  and graph capture;
* ``decode_traced(...)``: a routed decode that also records per-workgroup
  timestamps of its steps;
* ``build_index(stack)`` (the per-tile exception index, built on the GPU);
* ``validate(stack)`` (host-side layout check).

A stack with a tile index decodes in one kernel that writes every dense byte
once; without one the decode runs the fixed stream and the exception pass as
two kernels.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch  # load torch's HIP runtime first so libcsf binds to the same one

NVFP4 = 0
MXFP4 = 1
PASS_FIXED = 1
PASS_EXCEPTIONS = 2
PASS_ALL = 3
ENCODE_STREAMS = 1
ENCODE_ENTRIES = 2
MAX_EXPERTS = 2048
INDEX_TILE = 2048

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsf.so")

STATUS = {0: "CSF_OK", 1: "CSF_E_NULL", 2: "CSF_E_SHAPE", 3: "CSF_E_FORMAT", 4: "CSF_E_SIZE",
          5: "CSF_E_ALIGN", 6: "CSF_E_CORRUPT", 7: "CSF_E_MISMATCH", 8: "CSF_E_HIP"}

EXPORTS = ("csf_abi_version", "csf_status_str", "csf_prepare", "csf_encode_device", "csf_build_index",
           "csf_decode", "csf_decode_paired", "csf_decode_i64", "csf_decode_passes", "csf_decode_rows",
           "csf_moe_w4a16", "csf_decode_traced", "csf_validate")
STAMPS_PER_GROUP = 8


class CsfError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        msg = _lib().csf_status_str(status).decode() if _LIB is not None else ""
        super().__init__(f"{where}: {self.name} ({msg})")


class csf_sizes(ctypes.Structure):
    _fields_ = [("dense_bytes", ctypes.c_int64), ("bases_bytes", ctypes.c_int64),
                ("offsets_stride", ctypes.c_int64), ("offsets_bytes", ctypes.c_int64),
                ("num_exceptions", ctypes.c_int64), ("exceptions_bytes", ctypes.c_int64),
                ("prefix_bytes", ctypes.c_int64), ("index_tiles", ctypes.c_int64),
                ("index_bytes", ctypes.c_int64), ("compressed_bytes", ctypes.c_int64)]


class csf_rows(ctypes.Structure):
    _fields_ = [("begin", ctypes.c_int32), ("end", ctypes.c_int32)]


class csf_stack(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("offsets_stride", ctypes.c_int64), ("num_exceptions", ctypes.c_int64),
                ("bases", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("exceptions", ctypes.c_void_p), ("exc_prefix", ctypes.c_void_p),
                ("tile_index", ctypes.c_void_p)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is not built; run `python -m moe_weight_decode_amd.build`")
        lib = ctypes.CDLL(LIBRARY)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        lib.csf_abi_version.restype = ctypes.c_int
        lib.csf_abi_version.argtypes = []
        lib.csf_status_str.restype = ctypes.c_char_p
        lib.csf_status_str.argtypes = [ctypes.c_int]
        lib.csf_prepare.restype = ctypes.c_int
        lib.csf_prepare.argtypes = [i32, i32, i32, i32, vp, ctypes.POINTER(csf_sizes), vp, vp, vp, vp, vp]
        lib.csf_encode_device.restype = ctypes.c_int
        lib.csf_encode_device.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp]
        lib.csf_build_index.restype = ctypes.c_int
        lib.csf_build_index.argtypes = [ctypes.POINTER(csf_stack), vp, vp]
        lib.csf_decode.restype = ctypes.c_int
        lib.csf_decode.argtypes = [ctypes.POINTER(csf_stack), vp, vp, vp]
        lib.csf_decode_paired.restype = ctypes.c_int
        lib.csf_decode_paired.argtypes = [ctypes.POINTER(csf_stack), vp, ctypes.POINTER(csf_stack), vp,
                                          vp, vp]
        lib.csf_decode_i64.restype = ctypes.c_int
        lib.csf_decode_i64.argtypes = [ctypes.POINTER(csf_stack), vp, ctypes.POINTER(csf_stack), vp, vp, vp]
        lib.csf_decode_passes.restype = ctypes.c_int
        lib.csf_decode_passes.argtypes = [ctypes.POINTER(csf_stack), vp, ctypes.POINTER(csf_stack), vp,
                                          vp, ctypes.c_uint32, vp]
        lib.csf_decode_rows.restype = ctypes.c_int
        lib.csf_decode_rows.argtypes = [ctypes.POINTER(csf_stack), vp, ctypes.POINTER(csf_rows),
                                        ctypes.POINTER(csf_stack), vp, ctypes.POINTER(csf_rows), vp,
                                        ctypes.c_uint32, vp]
        lib.csf_moe_w4a16.restype = ctypes.c_int
        lib.csf_moe_w4a16.argtypes = [ctypes.POINTER(csf_stack), vp, vp, vp, i32, vp, vp, vp, vp]
        lib.csf_decode_traced.restype = ctypes.c_int
        lib.csf_decode_traced.argtypes = [ctypes.POINTER(csf_stack), vp, ctypes.POINTER(csf_stack), vp, vp, vp,
                                          ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint32), vp]
        lib.csf_validate.restype = ctypes.c_int
        lib.csf_validate.argtypes = [ctypes.POINTER(csf_stack)]
        _LIB = lib
    return _LIB


def library():
    """The loaded ``ctypes.CDLL`` of libcsf.so (raises if it is not built)."""
    return _lib()


@dataclass
class CompressedStack:
    """One compressed stack; tensors share one device (CPU or GPU)."""
    fmt: int
    E: int
    R: int
    C: int
    stride: int
    num_exceptions: int
    bases: torch.Tensor       # uint8 [E*R]
    offsets: torch.Tensor     # uint8 [E*stride]
    exceptions: torch.Tensor  # int32 [max(n, 1)], holding the u32 entry words
    prefix: torch.Tensor      # int32 [E+1]
    tile_index: torch.Tensor | None = None  # int32 [E*index_tiles + 1], optional

    @property
    def index_tiles(self) -> int:
        return (self.R * self.C + INDEX_TILE - 1) // INDEX_TILE

    @property
    def P(self) -> int:
        return self.R * self.C

    def tiles_per_plane(self, tile: int) -> int:
        """Tiles of ``tile`` positions covering one plane."""
        return (self.P + tile - 1) // tile

    @property
    def dense_bytes(self) -> int:
        return self.E * self.R * self.C

    @property
    def compressed_bytes(self) -> int:
        n = self.E * self.R + self.E * self.stride + 4 * self.num_exceptions + 4 * (self.E + 1)
        if self.tile_index is not None:
            n += 4 * (self.E * self.index_tiles + 1)
        return n

    @property
    def device(self) -> torch.device:
        return self.offsets.device

    def _map(self, fn) -> "CompressedStack":
        return CompressedStack(self.fmt, self.E, self.R, self.C, self.stride, self.num_exceptions,
                               fn(self.bases), fn(self.offsets), fn(self.exceptions), fn(self.prefix),
                               None if self.tile_index is None else fn(self.tile_index))

    def to(self, device) -> "CompressedStack":
        return self._map(lambda t: t.to(device, non_blocking=False).contiguous())

    def clone(self) -> "CompressedStack":
        return self._map(lambda t: t.clone())

    def without_index(self) -> "CompressedStack":
        """The same stack with no tile index (decoded by the two-pass kernels)."""
        st = self._map(lambda t: t)
        st.tile_index = None
        return st

    def descriptor(self) -> csf_stack:
        d = csf_stack()
        d.format, d.num_experts, d.rows, d.cols = self.fmt, self.E, self.R, self.C
        d.offsets_stride, d.num_exceptions = self.stride, self.num_exceptions
        d.bases = self.bases.data_ptr()
        d.offsets = self.offsets.data_ptr()
        d.exceptions = self.exceptions.data_ptr() if self.num_exceptions > 0 else None
        d.exc_prefix = self.prefix.data_ptr()
        d.tile_index = self.tile_index.data_ptr() if self.tile_index is not None else None
        return d

    def numpy(self) -> dict:
        """Host copies of the buffers (uint32 entries)."""
        d = dict(fmt=self.fmt, E=self.E, R=self.R, C=self.C, stride=self.stride,
                 bases=self.bases.cpu().numpy().copy(), offsets=self.offsets.cpu().numpy().copy(),
                 exceptions=self.exceptions.cpu().numpy()[:self.num_exceptions].view(np.uint32).copy(),
                 prefix=self.prefix.cpu().numpy().copy())
        if self.tile_index is not None:
            d["tile_index"] = self.tile_index.cpu().numpy().copy()
        return d


def from_numpy(d: dict, device="cpu") -> CompressedStack:
    """Wrap host arrays (``fmt, E, R, C, stride, bases, offsets, exceptions, prefix`` and
    optionally ``tile_index``)."""
    exc = np.ascontiguousarray(d["exceptions"], dtype=np.uint32)
    n = int(exc.size)
    exc_t = torch.from_numpy(exc.view(np.int32).copy() if n else np.zeros(1, dtype=np.int32))
    st = CompressedStack(int(d["fmt"]), int(d["E"]), int(d["R"]), int(d["C"]), int(d["stride"]), n,
                         torch.from_numpy(np.ascontiguousarray(d["bases"], dtype=np.uint8).copy()),
                         torch.from_numpy(np.ascontiguousarray(d["offsets"], dtype=np.uint8).copy()),
                         exc_t,
                         torch.from_numpy(np.ascontiguousarray(d["prefix"], dtype=np.int32).copy()))
    if d.get("tile_index") is not None:
        st.tile_index = torch.from_numpy(np.ascontiguousarray(d["tile_index"], dtype=np.int32).copy())
    return st.to(device) if str(device) != "cpu" else st


def _check(status: int, where: str):
    if status != 0:
        raise CsfError(status, where)


def offsets_stride(fmt: int, R: int, C: int) -> int:
    """Offset bytes per expert: 16 per group of 128 / w positions."""
    G = 32 if fmt == NVFP4 else 128
    return 16 * ((R * C + G - 1) // G)


class _DeviceEncode:
    """One stack's GPU encode between its two phases."""

    def __init__(self, x: torch.Tensor, fmt: int, index: bool, stream):
        lib = _lib()
        if x.dtype != torch.uint8 or x.dim() != 3 or not x.is_contiguous():
            raise ValueError("dense must be a contiguous uint8 [E, R, C] tensor")
        E, R, C = (int(v) for v in x.shape)
        dev = x.device
        S = offsets_stride(fmt, R, C)
        NT = (R * C + INDEX_TILE - 1) // INDEX_TILE
        self.x, self.fmt, self.index, self.stream = x, fmt, index, stream
        self.E, self.R, self.C, self.S = E, R, C, S
        self.bases = torch.empty(E * R, dtype=torch.uint8, device=dev)
        self.offsets = torch.empty(E * S, dtype=torch.uint8, device=dev)
        self.prefix = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.tidx = torch.empty(E * NT + 1, dtype=torch.int32, device=dev)
        cur = torch.cuda.current_stream(dev)
        self.side = stream is not None and _stream_handle(stream, dev) != cur.cuda_stream
        if self.side:
            # the outputs were allocated on the current stream, whose queued work
            # may still use their memory (freed there just before): `stream`
            # writes them only after that work
            stream.wait_stream(cur)
        self.h = _stream_handle(stream, dev)
        _check(lib.csf_encode_device(fmt, E, R, C, x.data_ptr(), self.bases.data_ptr(), self.offsets.data_ptr(),
                                     None, self.prefix.data_ptr(), self.tidx.data_ptr(), ENCODE_STREAMS, self.h),
               "csf_encode_device(streams)")

    def finish(self, n: int) -> CompressedStack:
        """The entries phase, once the entry count n (exc_prefix[E]) is known."""
        lib = _lib()
        exc = torch.empty(max(n, 1), dtype=torch.int32, device=self.x.device)
        if n > 0:
            _check(lib.csf_encode_device(self.fmt, self.E, self.R, self.C, self.x.data_ptr(), self.bases.data_ptr(),
                                         None, exc.data_ptr(), None, self.tidx.data_ptr(), ENCODE_ENTRIES, self.h),
                   "csf_encode_device(entries)")
        if self.side:
            # allocated on the current stream, written on `stream`: keep the memory
            # from being reused before `stream` is done with it
            for t in (self.bases, self.offsets, self.prefix, self.tidx, exc, self.x):
                t.record_stream(self.stream)
        return CompressedStack(self.fmt, self.E, self.R, self.C, self.S, n, self.bases, self.offsets, exc,
                               self.prefix, self.tidx if self.index else None)


def _prepare_devices(xs, fmts, index: bool, stream=None) -> list:
    """The streams phase of every stack, one read-back of all their entry
    counts, then every entries phase."""
    encs = [_DeviceEncode(x, f, index, stream) for x, f in zip(xs, fmts)]
    if stream is not None:
        stream.synchronize()
    if len(encs) == 1:
        counts = [encs[0].prefix[encs[0].E].item()]
    else:
        counts = torch.stack([e.prefix[e.E] for e in encs]).tolist()
    return [e.finish(int(n)) for e, n in zip(encs, counts)]


def _prepare_device(x: torch.Tensor, fmt: int, index: bool, stream=None) -> CompressedStack:
    return _prepare_devices([x], [fmt], index, stream)[0]


def prepare_many(denses, fmts, index: bool = True, stream=None) -> list:
    """``prepare`` of several stacks (for example a layer's gate/up and down
    projections).  Stacks on one GPU are encoded with a single read-back of
    their entry counts: every stack's first phase is enqueued, the counts are
    read together, then every stack's entries phase (same streams, result and
    stream rules as ``prepare``).  ``fmts`` is one format per stack."""
    denses, fmts = list(denses), list(fmts)
    if len(denses) != len(fmts):
        raise ValueError("one format per stack")
    on_gpu = [isinstance(d, torch.Tensor) and d.device.type == "cuda" for d in denses]
    if denses and all(on_gpu) and len({d.device for d in denses}) == 1:
        return _prepare_devices(denses, fmts, index, stream)
    return [prepare(d, f, index, stream) for d, f in zip(denses, fmts)]


def prepare(dense, fmt: int, index: bool = True, stream=None) -> CompressedStack:
    """Encode ``dense`` (uint8 [E, R, C], tensor or array), with the tile index
    unless ``index`` is False; the result lives on ``dense``'s device.  A GPU
    tensor is encoded on the GPU (the count of exception entries is read back
    once, to size their buffer); host data by the host encoder.  The GPU
    encode runs on ``stream`` (default: the current stream): ``dense`` must be
    ready there, and work on another stream that uses the result must wait
    for ``stream`` (for example ``current_stream().wait_stream(stream)``).
    A ``stream`` other than the current one first waits for the current
    stream's queued work, since the result's memory is allocated there."""
    if isinstance(dense, torch.Tensor) and dense.device.type == "cuda":
        return _prepare_device(dense, fmt, index, stream)
    lib = _lib()
    device = dense.device if isinstance(dense, torch.Tensor) else torch.device("cpu")
    x = dense.detach().cpu().numpy() if isinstance(dense, torch.Tensor) else np.asarray(dense)
    if x.dtype != np.uint8 or x.ndim != 3:
        raise ValueError("dense must be uint8 [E, R, C]")
    x = np.ascontiguousarray(x)
    E, R, C = (int(v) for v in x.shape)
    sz = csf_sizes()
    _check(lib.csf_prepare(fmt, E, R, C, x.ctypes.data, ctypes.byref(sz), None, None, None, None, None),
           "csf_prepare(sizes)")
    n = int(sz.num_exceptions)
    bases = np.empty(E * R, dtype=np.uint8)
    offsets = np.empty(int(sz.offsets_bytes), dtype=np.uint8)
    exc = np.empty(max(n, 1), dtype=np.uint32)
    prefix = np.empty(E + 1, dtype=np.int32)
    tidx = np.empty(int(sz.index_bytes) // 4, dtype=np.int32) if index else None
    _check(lib.csf_prepare(fmt, E, R, C, x.ctypes.data, ctypes.byref(sz), bases.ctypes.data,
                           offsets.ctypes.data, exc.ctypes.data, prefix.ctypes.data,
                           tidx.ctypes.data if index else None), "csf_prepare")
    return from_numpy(dict(fmt=fmt, E=E, R=R, C=C, stride=int(sz.offsets_stride), bases=bases,
                           offsets=offsets, exceptions=exc[:n], prefix=prefix, tile_index=tidx), device)


def _stream_handle(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _check_stack_tensors(stack: CompressedStack, name: str):
    """Every buffer of the stack holds at least what the layout addresses: the
    library sees only pointers, so a short tensor would be read past its end."""
    need = [("bases", stack.bases, torch.uint8, stack.E * stack.R),
            ("offsets", stack.offsets, torch.uint8, stack.E * stack.stride),
            ("exceptions", stack.exceptions, torch.int32, max(stack.num_exceptions, 1)),
            ("prefix", stack.prefix, torch.int32, stack.E + 1)]
    if stack.tile_index is not None:
        need.append(("tile_index", stack.tile_index, torch.int32, stack.E * stack.index_tiles + 1))
    for what, t, dt, n in need:
        if not isinstance(t, torch.Tensor) or t.dtype != dt or t.numel() < n:
            raise ValueError(f"{name}: {what} must be a {dt} tensor of at least {n} elements")
        if t.device != stack.device or not t.is_contiguous():
            raise ValueError(f"{name}: stack tensors must be contiguous on one device")


def _check_device(stack: CompressedStack, ws: torch.Tensor, name: str):
    if stack.device.type != "cuda":
        raise ValueError(f"{name}: compressed stack must be on a GPU")
    _check_stack_tensors(stack, name)
    if not isinstance(ws, torch.Tensor) or ws.device != stack.device or ws.dtype != torch.uint8:
        raise ValueError(f"{name}: workspace must be a uint8 tensor on {stack.device}")
    if not ws.is_contiguous() or ws.numel() < stack.dense_bytes:
        raise ValueError(f"{name}: workspace must be contiguous with >= {stack.dense_bytes} bytes")


def _es_ptr(expert_start, stack: CompressedStack):
    if expert_start is None:
        return None
    if (not isinstance(expert_start, torch.Tensor) or expert_start.dtype not in (torch.int32, torch.int64)
            or expert_start.device != stack.device or expert_start.numel() != stack.E + 1
            or not expert_start.is_contiguous()):
        raise ValueError(f"expert_start must be a contiguous int32 or int64 [{stack.E + 1}] tensor "
                         f"on {stack.device}")
    return expert_start.data_ptr()


def _is_wide(expert_start) -> bool:
    return expert_start is not None and expert_start.dtype == torch.int64


def decode(stack: CompressedStack, workspace: torch.Tensor, expert_start=None, stream=None):
    """Enqueue the full decode of ``stack`` into ``workspace`` on ``stream``;
    ``expert_start`` (int32 or int64 [E+1], on the device) limits it to the
    experts with routed tokens."""
    _check_device(stack, workspace, "decode")
    d = stack.descriptor()
    es, h = _es_ptr(expert_start, stack), _stream_handle(stream, stack.device)
    if _is_wide(expert_start):
        _check(_lib().csf_decode_i64(ctypes.byref(d), workspace.data_ptr(), None, None, es, h),
               "csf_decode_i64")
    else:
        _check(_lib().csf_decode(ctypes.byref(d), workspace.data_ptr(), es, h), "csf_decode")


def decode_paired(gate_up: CompressedStack, ws_gate_up: torch.Tensor, down: CompressedStack,
                  ws_down: torch.Tensor, expert_start=None, stream=None):
    """Enqueue the decode of two stacks of the same experts (one launch per pass)."""
    _check_device(gate_up, ws_gate_up, "decode_paired")
    _check_device(down, ws_down, "decode_paired")
    a, b = gate_up.descriptor(), down.descriptor()
    es, h = _es_ptr(expert_start, gate_up), _stream_handle(stream, gate_up.device)
    if _is_wide(expert_start):
        _check(_lib().csf_decode_i64(ctypes.byref(a), ws_gate_up.data_ptr(), ctypes.byref(b),
                                     ws_down.data_ptr(), es, h), "csf_decode_i64")
    else:
        _check(_lib().csf_decode_paired(ctypes.byref(a), ws_gate_up.data_ptr(), ctypes.byref(b),
                                        ws_down.data_ptr(), es, h), "csf_decode_paired")


def decode_passes(first: CompressedStack, ws_first: torch.Tensor, second=None, ws_second=None,
                  expert_start=None, passes: int = PASS_ALL, stream=None):
    """Enqueue the selected passes only (see ``csf_decode_passes``)."""
    _check_device(first, ws_first, "decode_passes")
    a = first.descriptor()
    b_ref, ws_b = None, None
    if second is not None:
        _check_device(second, ws_second, "decode_passes")
        b = second.descriptor()
        b_ref, ws_b = ctypes.byref(b), ws_second.data_ptr()
    _check(_lib().csf_decode_passes(ctypes.byref(a), ws_first.data_ptr(), b_ref, ws_b,
                                    _es_ptr(expert_start, first), passes,
                                    _stream_handle(stream, first.device)), "csf_decode_passes")


def decode_rows(first: CompressedStack, ws_first: torch.Tensor, rows_first=None, second=None,
                ws_second=None, rows_second=None, expert_start=None, passes: int = PASS_ALL, stream=None):
    """Enqueue the decode of a window of rows of every plane (see
    ``csf_decode_rows``): ``rows_*`` is ``(begin, end)`` or None for every row;
    ``expert_start`` is int32 [E+1] or None."""
    _check_device(first, ws_first, "decode_rows")
    if expert_start is not None and _is_wide(expert_start):
        raise ValueError("decode_rows takes an int32 expert_start")
    a = first.descriptor()
    ra = None if rows_first is None else csf_rows(*rows_first)
    b_ref, ws_b, rb = None, None, None
    if second is not None:
        _check_device(second, ws_second, "decode_rows")
        b = second.descriptor()
        b_ref, ws_b = ctypes.byref(b), ws_second.data_ptr()
        rb = None if rows_second is None else csf_rows(*rows_second)
    _check(_lib().csf_decode_rows(ctypes.byref(a), ws_first.data_ptr(), None if ra is None else ctypes.byref(ra),
                                  b_ref, ws_b, None if rb is None else ctypes.byref(rb),
                                  _es_ptr(expert_start, first), passes,
                                  _stream_handle(stream, first.device)), "csf_decode_rows")


def moe_w4a16(scales: CompressedStack, weights: torch.Tensor, x: torch.Tensor, alpha: torch.Tensor,
              expert_start: torch.Tensor, out: torch.Tensor | None = None, dense_scales=None, stream=None):
    """Enqueue the routed W4A16 projection (see ``csf_moe_w4a16``); returns y
    (float32 [T, N]).  ``x`` is bfloat16 (or int16/uint16 bit patterns)
    [T, K]; ``weights`` uint8 [E, N, K/2]; ``alpha`` float32 [E]; K is 16
    (NVFP4) or 32 (MXFP4) times the stack's scale columns.  With
    ``dense_scales`` (uint8, the stack's dense size) the scales come from it
    instead of the compressed stack."""
    dev = scales.device
    if dev.type != "cuda":
        raise ValueError("moe_w4a16: compressed stack must be on a GPU")
    _check_stack_tensors(scales, "moe_w4a16")
    T = x.shape[0]
    for name, t, dt in (("weights", weights, (torch.uint8,)), ("x", x, (torch.bfloat16, torch.int16, torch.uint16)),
                        ("alpha", alpha, (torch.float32,)), ("expert_start", expert_start, (torch.int32,))):
        if t.device != dev or t.dtype not in dt or not t.is_contiguous():
            raise ValueError(f"moe_w4a16: {name} must be a contiguous {dt} tensor on {dev}")
    K = scales.C * (16 if scales.fmt == NVFP4 else 32)  # weights per scale byte
    if weights.numel() != scales.E * scales.R * K // 2 or x.numel() != T * K:
        raise ValueError("moe_w4a16: weights / x sizes do not match the scale stack")
    if alpha.numel() != scales.E or expert_start.numel() != scales.E + 1:
        raise ValueError("moe_w4a16: alpha must be [E] and expert_start [E+1]")
    if out is None:
        out = torch.empty(T, scales.R, dtype=torch.float32, device=dev)
    elif out.device != dev or out.dtype != torch.float32 or not out.is_contiguous() or out.numel() != T * scales.R:
        raise ValueError("moe_w4a16: out must be a contiguous float32 [T, N] tensor")
    if dense_scales is not None and (dense_scales.device != dev or dense_scales.dtype != torch.uint8
                                     or not dense_scales.is_contiguous()
                                     or dense_scales.numel() < scales.dense_bytes):
        raise ValueError("moe_w4a16: dense_scales must be contiguous uint8 with the stack's dense size")
    d = scales.descriptor()
    _check(_lib().csf_moe_w4a16(ctypes.byref(d), None if dense_scales is None else dense_scales.data_ptr(),
                                weights.data_ptr(), x.data_ptr() if T > 0 else None, T, alpha.data_ptr(),
                                expert_start.data_ptr(), out.data_ptr() if T > 0 else None,
                                _stream_handle(stream, dev)),
           "csf_moe_w4a16")
    return out


class Launch:
    """A decode call with its arguments marshalled once, for enqueueing the same
    decode many times (benchmark loops, graph capture): each call is a single
    C-ABI call.  Keeps references to every tensor it points at."""

    def __init__(self, first: CompressedStack, ws_first: torch.Tensor, second=None, ws_second=None,
                 expert_start=None, stream=None):
        _check_device(first, ws_first, "Launch")
        if second is not None:
            _check_device(second, ws_second, "Launch")
        self._keep = (first, ws_first, second, ws_second, expert_start)
        self._a = first.descriptor()
        self._b = second.descriptor() if second is not None else None
        self._args_ws = (ws_first.data_ptr(), ws_second.data_ptr() if second is not None else None)
        self._es = _es_ptr(expert_start, first)
        self._wide = _is_wide(expert_start)
        self._stream = _stream_handle(stream, first.device)
        self._fn = _lib().csf_decode_passes
        self._fn64 = _lib().csf_decode_i64

    @property
    def stream(self) -> int:
        return self._stream

    def __call__(self, passes: int = PASS_ALL):
        b = ctypes.byref(self._b) if self._b is not None else None
        if self._wide:
            if passes != PASS_ALL:
                raise ValueError("an int64 expert_start decodes all passes together")
            st = self._fn64(ctypes.byref(self._a), self._args_ws[0], b, self._args_ws[1], self._es,
                            self._stream)
        else:
            st = self._fn(ctypes.byref(self._a), self._args_ws[0], b, self._args_ws[1], self._es, passes,
                          self._stream)
        if st != 0:
            raise CsfError(st, "csf_decode_passes")


def decode_traced(first: CompressedStack, ws_first: torch.Tensor, second=None, ws_second=None,
                  expert_start=None, stream=None) -> torch.Tensor:
    """Enqueue a routed decode (int32 ``expert_start``, stacks with a tile
    index) that also records per-workgroup timestamps (see
    ``csf_decode_traced``); returns the uint64 stamps as an int64 tensor
    [groups, 8] on the device."""
    _check_device(first, ws_first, "decode_traced")
    b_ref, ws_b = None, None
    if second is not None:
        _check_device(second, ws_second, "decode_traced")
        b = second.descriptor()
        b_ref, ws_b = ctypes.byref(b), ws_second.data_ptr()
    if expert_start is None or _is_wide(expert_start):
        raise ValueError("decode_traced takes an int32 expert_start")
    a = first.descriptor()
    es, h = _es_ptr(expert_start, first), _stream_handle(stream, first.device)
    groups = ctypes.c_uint32(0)
    lib = _lib()
    _check(lib.csf_decode_traced(ctypes.byref(a), ws_first.data_ptr(), b_ref, ws_b, es, None, 0,
                                 ctypes.byref(groups), h), "csf_decode_traced(groups)")
    stamps = torch.zeros(groups.value, STAMPS_PER_GROUP, dtype=torch.int64, device=first.device)
    _check(lib.csf_decode_traced(ctypes.byref(a), ws_first.data_ptr(), b_ref, ws_b, es, stamps.data_ptr(),
                                 stamps.numel(), ctypes.byref(groups), h), "csf_decode_traced")
    return stamps


def build_index(stack: CompressedStack, stream=None) -> torch.Tensor:
    """Enqueue the GPU construction of ``stack``'s tile index; returns the new
    int32 tensor (also attached to ``stack``)."""
    if stack.device.type != "cuda":
        raise ValueError("build_index: stack must be on a GPU")
    _check_stack_tensors(stack, "build_index")
    out = torch.empty(stack.E * stack.index_tiles + 1, dtype=torch.int32, device=stack.device)
    d = stack.descriptor()
    _check(_lib().csf_build_index(ctypes.byref(d), out.data_ptr(), _stream_handle(stream, stack.device)),
           "csf_build_index")
    stack.tile_index = out
    return out


def validate(stack: CompressedStack):
    """Check the layout invariants on a host copy; raises ``CsfError`` (CSF_E_CORRUPT)."""
    h = stack.to("cpu") if stack.device.type != "cpu" else stack
    _check_stack_tensors(h, "validate")
    d = h.descriptor()
    _check(_lib().csf_validate(ctypes.byref(d)), "csf_validate")
