"""Binding of ``libcsf_probe.so``: the measurement kernels the decoder's
timings are read against (``include/csf_probe.h``).  Argument marshalling
only; raises if the library is not built."""
from __future__ import annotations

import ctypes
import os

import torch

from . import _check, _lib, _stream_handle, csf_stack

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsf_probe.so")
EXPORTS = ("csf_probe_mix", "csf_probe_chain", "csf_probe_host_ns")
NT_ENTRIES = 1

_PLIB = None


def library():
    global _PLIB
    if _PLIB is None:
        _lib()  # libcsf.so first: the probe library links to it
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is not built; run `python -m moe_weight_decode_amd.build`")
        lib = ctypes.CDLL(LIBRARY)
        vp, u32, u64 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64
        lib.csf_probe_mix.restype = ctypes.c_int
        lib.csf_probe_mix.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(u64), u32, vp, u64, u32, u32, vp]
        lib.csf_probe_chain.restype = ctypes.c_int
        lib.csf_probe_chain.argtypes = [vp, u64, u32, u32, vp, u32, u32, vp]
        lib.csf_probe_host_ns.restype = ctypes.c_double
        lib.csf_probe_host_ns.argtypes = [ctypes.POINTER(csf_stack), vp, ctypes.POINTER(csf_stack), vp, vp, u32, vp]
        _PLIB = lib
    return _PLIB


class Mix:
    """One stream-mix launch (``csf_probe_mix``) with its arguments marshalled
    once: reads every tensor of ``srcs``, writes ``dst``."""

    def __init__(self, srcs, dst: torch.Tensor, grid: int, flags: int = 0, stream=None):
        self.keep = (tuple(srcs), dst)
        n = len(srcs)
        self.src = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in srcs])
        self.nbytes = (ctypes.c_uint64 * max(n, 1))(*[t.numel() * t.element_size() for t in srcs])
        self.n, self.dst, self.dst_bytes = n, dst.data_ptr(), dst.numel() * dst.element_size()
        self.grid, self.flags = grid, flags
        self.stream = _stream_handle(stream, dst.device)
        self.fn = library().csf_probe_mix

    def __call__(self):
        _check(self.fn(self.src, self.nbytes, self.n, self.dst, self.dst_bytes, self.grid, self.flags,
                       self.stream), "csf_probe_mix")


class Chain:
    """One ``csf_probe_chain`` launch: ``hops`` dependent loads per workgroup
    through ``buf`` (int32 tensor holding a permutation of its indices), then
    a 16-byte store per lane into ``out`` (or none)."""

    def __init__(self, buf, hops: int, out, grid: int, block: int = 256, seed: int = 0, stream=None):
        t = out if out is not None else buf
        dev = t.device if t is not None else torch.device("cuda", torch.cuda.current_device())
        self.keep = (buf, out)
        self.args = [buf.data_ptr() if buf is not None else None, buf.numel() if buf is not None else 0, seed,
                     hops, out.data_ptr() if out is not None else None, grid, block]
        self.dev = dev
        self.fixed = None if stream is None else _stream_handle(stream, dev)
        self.fn = library().csf_probe_chain

    @property
    def stream(self) -> int:
        """The launch stream: the one given, else the current stream at the call."""
        return self.fixed if self.fixed is not None else _stream_handle(None, self.dev)

    def __call__(self):
        _check(self.fn(*self.args, self.stream), "csf_probe_chain")


def host_ns(first, ws_first, second=None, ws_second=None, expert_start=None, calls: int = 200, stream=None) -> float:
    """Host nanoseconds per C call of csf_decode / csf_decode_paired
    (enqueue only)."""
    a = first.descriptor()
    b = second.descriptor() if second is not None else None
    v = library().csf_probe_host_ns(ctypes.byref(a), ws_first.data_ptr(), ctypes.byref(b) if b is not None else None,
                                    ws_second.data_ptr() if second is not None else None,
                                    expert_start.data_ptr() if expert_start is not None else None, calls,
                                    _stream_handle(stream, first.device))
    if v < 0:
        raise RuntimeError(f"csf_probe_host_ns failed ({v})")
    return v
