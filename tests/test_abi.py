"""Host-side tests of the C ABI (no GPU): exports, the library encoder against
the oracle encoder, the stream validator, and argument errors that must be
returned before anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import workloads

mwd = pytest.importorskip("moe_weight_decode_amd")

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(os.path.dirname(HERE), "include", "csf.h")


@pytest.fixture(scope="module")
def lib():
    return mwd.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csf_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(mwd.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_every_declared_symbol():
    from moe_weight_decode_amd import probe
    text = open(os.path.join(os.path.dirname(HERE), "include", "csf_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(csf_[a-z0-9_]+)\s*\(", text)))
    assert set(names) == set(probe.EXPORTS)
    plib = probe.library()
    for n in names:
        assert hasattr(plib, n), n


def test_probe_argument_errors():
    from moe_weight_decode_amd import probe
    plib = probe.library()
    u64 = ctypes.c_uint64
    srcs = (ctypes.c_void_p * 1)(0x1000)
    big = (u64 * 1)(1 << 30)
    # a read stream whose per-tile piece exceeds what a lane loads
    assert mwd.STATUS[plib.csf_probe_mix(srcs, big, 1, 0x2000, 16384, 1, 0, None)] == "CSF_E_SIZE"
    assert mwd.STATUS[plib.csf_probe_mix(srcs, big, 4, 0x2000, 16384, 1, 0, None)] == "CSF_E_SIZE"
    three = (ctypes.c_void_p * 3)(0x1000, 0x1000, 0x1000)
    sizes = (u64 * 3)(1 << 13, 1 << 13, 1 << 13)  # stream 2's piece above 4 KiB
    assert mwd.STATUS[plib.csf_probe_mix(three, sizes, 0, 0x2000, 16384, 1, 0, None)] == "CSF_E_SIZE"
    assert mwd.STATUS[plib.csf_probe_mix(three, sizes, 3, 0x2000, 16384, 1, 0, None)] == "CSF_E_SIZE"
    assert mwd.STATUS[plib.csf_probe_mix(None, None, 1, 0x2000, 16384, 1, 0, None)] == "CSF_E_NULL"
    assert mwd.STATUS[plib.csf_probe_chain(None, 0, 0, 3, None, 1, 64, None)] == "CSF_E_NULL"
    assert mwd.STATUS[plib.csf_probe_chain(0x1000, 16, 0, 3, None, 1, 100, None)] == "CSF_E_SIZE"
    assert mwd.STATUS[plib.csf_probe_chain(0x1000, 1 << 30, 0, 3, None, 1, 64, None)] == "CSF_E_SIZE"


def test_abi_version_and_status_strings(lib):
    assert lib.csf_abi_version() == 5
    for s in range(9):
        assert lib.csf_status_str(s)
    assert lib.csf_status_str(99) == b"unknown status"


def _same_stack(a: dict, b: dict):
    for k in ("fmt", "E", "R", "C", "stride"):
        assert a[k] == b[k], k
    for k in ("bases", "offsets", "exceptions", "prefix", "tile_index"):
        assert np.array_equal(np.asarray(a[k]).ravel(), np.asarray(b[k]).ravel()), k


ENCODE_CASES = [
    ("tiny", workloads.NVFP4, lambda: workloads.TINY.generate()),
    ("gate_slice", workloads.NVFP4, lambda: workloads.nvfp4_stack(6, 80, 128, 1, 0.03)),
    ("down_slice", workloads.NVFP4, lambda: workloads.nvfp4_stack(6, 200, 50, 2, 0.10, hot_row_frac=0.01)),
    ("mx_slice", workloads.MXFP4, lambda: workloads.mxfp4_stack(5, 100, 160, 4, 0.15)),
    ("uniform_nv", workloads.NVFP4, lambda: workloads.uniform_bytes(3, 31, 37, 8)),
    ("uniform_mx", workloads.MXFP4, lambda: workloads.uniform_bytes(3, 31, 37, 9)),
    ("one_col", workloads.NVFP4, lambda: workloads.uniform_bytes(2, 7, 1, 10)),
    ("c_eight", workloads.MXFP4, lambda: workloads.uniform_bytes(2, 3, 8, 11)),
]


@pytest.mark.parametrize("name,fmt,gen", ENCODE_CASES, ids=[c[0] for c in ENCODE_CASES])
def test_library_encoder_matches_oracle(orc, name, fmt, gen):
    x = gen()
    lib_stack = mwd.prepare(x, fmt).numpy()
    _same_stack(lib_stack, orc.encode(fmt, x))


def test_library_encoder_two_column_exhaustive(orc):
    a, b = np.meshgrid(np.arange(256), np.arange(256), indexing="ij")
    x = np.stack([a.ravel(), b.ravel()], axis=1).astype(np.uint8).reshape(4, 16384, 2)
    for fmt in (workloads.NVFP4, workloads.MXFP4):
        _same_stack(mwd.prepare(x, fmt).numpy(), orc.encode(fmt, x))


def test_prepare_sizes_closed_form():
    x = workloads.TINY.generate()
    st = mwd.prepare(x, workloads.NVFP4)
    assert st.stride == 256 and st.offsets.numel() == 4 * 256
    assert st.dense_bytes == 2048
    # 512 positions per plane: one index tile per expert
    assert st.tile_index.numel() == 4 * 1 + 1
    assert st.compressed_bytes == 4 * 64 + 4 * 256 + 4 * st.num_exceptions + 4 * 5 + 4 * 5
    assert mwd.prepare(x, workloads.NVFP4, index=False).tile_index is None


def test_validate_accepts_encoded_stacks():
    for _, fmt, gen in ENCODE_CASES:
        mwd.validate(mwd.prepare(gen(), fmt))


def _corrupt(st, what):
    st = st.clone()
    exc = st.exceptions.numpy().view(np.uint32)
    if what == "prefix_start":
        st.prefix[0] = 1
    elif what == "prefix_decreasing":
        st.prefix[2] = st.prefix[1] - 1
    elif what == "prefix_end":
        st.prefix[-1] = st.prefix[-1] - 1
    elif what == "unsorted":
        exc[[0, 1]] = exc[[1, 0]]
    elif what == "duplicate":
        exc[1] = (exc[0] & ~np.uint32(0xFF)) | (exc[1] & np.uint32(0xFF))
    elif what == "out_of_plane":
        exc[int(st.prefix[1]) - 1] = np.uint32((st.P << 8) | 0x99)
    elif what == "fits_window":
        p = int(exc[0] >> 8)
        base = int(st.bases[p // st.C])
        exc[0] = np.uint32((p << 8) | base)
    elif what == "index_shifted":
        st.tile_index[1] += 1
    elif what == "index_end":
        st.tile_index[-1] -= 1
    elif what == "field_at_exception":
        p = int(exc[0] >> 8)
        st.offsets[16 * (p // 32) + p % 16] |= np.uint8(1 << (4 * ((p % 32) // 16)))
    return st


@pytest.mark.parametrize("what", ["prefix_start", "prefix_decreasing", "prefix_end", "unsorted",
                                  "duplicate", "out_of_plane", "fits_window", "field_at_exception",
                                  "index_shifted", "index_end"])
def test_validate_rejects_corruption(what):
    x = workloads.TINY.generate()
    st = mwd.prepare(x, workloads.NVFP4)
    bad = _corrupt(st, what)
    with pytest.raises(mwd.CsfError) as ei:
        mwd.validate(bad)
    assert ei.value.name == "CSF_E_CORRUPT"


def test_validate_checks_prefix_before_entries():
    """A prefix that overshoots the entry count is rejected before any entry is
    read.  The entries sit at the end of a readable page followed by an
    inaccessible one, so a read past the last entry would fault the process."""
    import mmap
    x = np.full((2, 4, 8), 0x40, dtype=np.uint8)   # expert 0: no entries
    x[1, 0, 1] = x[1, 1, 3] = x[1, 2, 0] = x[1, 3, 5] = x[1, 3, 7] = 0x00   # expert 1: five
    st = mwd.prepare(x, workloads.NVFP4)
    mwd.validate(st)
    n = st.num_exceptions
    exc = np.ascontiguousarray(st.exceptions.numpy().view(np.uint32)[:n])
    assert n == 5 and list(st.prefix.numpy()) == [0, 0, 5]
    page = mmap.PAGESIZE
    buf = mmap.mmap(-1, 2 * page)
    base = ctypes.addressof(ctypes.c_char.from_buffer(buf))
    libc = ctypes.CDLL(None, use_errno=True)
    libc.mprotect.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    at = base + page - 4 * n
    ctypes.memmove(at, exc.ctypes.data, 4 * n)
    assert libc.mprotect(base + page, page, 0) == 0   # PROT_NONE
    try:
        st.prefix[1] = n + 1000
        d = st.descriptor()
        d.exceptions = at
        assert mwd.STATUS[mwd.library().csf_validate(ctypes.byref(d))] == "CSF_E_CORRUPT"
    finally:
        assert libc.mprotect(base + page, page, 3) == 0   # PROT_READ | PROT_WRITE


@pytest.mark.parametrize("what", ["bases", "offsets", "exceptions", "prefix", "tile_index"])
def test_binding_rejects_short_stack_tensors(what):
    """The library sees only pointers; the binding refuses a stack whose buffer
    is shorter than the layout addresses (or of another dtype) before any call."""
    st = mwd.prepare(workloads.TINY.generate(), workloads.NVFP4)
    mwd.validate(st)
    short = st.clone()
    t = getattr(short, what)
    setattr(short, what, t[: (t.numel() - 1) if what != "exceptions" else st.num_exceptions - 1])
    with pytest.raises(ValueError, match=what):
        mwd.validate(short)
    wrong = st.clone()
    setattr(wrong, what, getattr(wrong, what).to(torch.int64))
    with pytest.raises(ValueError, match=what):
        mwd.validate(wrong)


def test_validate_rejects_fields_past_plane():
    x = workloads.uniform_bytes(1, 5, 7, 3)  # P = 35: second group holds positions 32..63
    st = mwd.prepare(x, workloads.NVFP4)
    st.offsets[16 + 5] |= np.uint8(0x01)  # position 37
    with pytest.raises(mwd.CsfError):
        mwd.validate(st)


def test_validate_rejects_wrapping_field():
    x = np.full((1, 1, 4), 250, dtype=np.uint8)
    st = mwd.prepare(x, workloads.NVFP4)
    st.offsets[0] = 0x0F  # 250 + 15 > 255
    with pytest.raises(mwd.CsfError):
        mwd.validate(st)


# --- decode argument errors: rejected on the host, before any HIP call -------

def _fake(fmt=0, E=4, R=64, C=8, stride=256, n=10, bases=0x1000, offsets=0x2000, exc=0x3000,
          prefix=0x4000, tile_index=None):
    d = mwd.csf_stack()
    d.format, d.num_experts, d.rows, d.cols = fmt, E, R, C
    d.offsets_stride, d.num_exceptions = stride, n
    d.bases, d.offsets, d.exceptions, d.exc_prefix = bases, offsets, exc, prefix
    d.tile_index = tile_index
    return d


DECODE_ERRORS = [
    ("null_stack", None, 0x5000, "CSF_E_NULL"),
    ("null_ws", _fake(), None, "CSF_E_NULL"),
    ("null_offsets", _fake(offsets=None), 0x5000, "CSF_E_NULL"),
    ("null_exc_with_entries", _fake(exc=None), 0x5000, "CSF_E_NULL"),
    ("bad_format", _fake(fmt=5), 0x5000, "CSF_E_FORMAT"),
    ("zero_experts", _fake(E=0), 0x5000, "CSF_E_SHAPE"),
    ("negative_rows", _fake(R=-1), 0x5000, "CSF_E_SHAPE"),
    ("plane_too_big", _fake(R=4096, C=4096, stride=16 * 524288), 0x5000, "CSF_E_SHAPE"),
    ("too_many_experts", _fake(E=4096), 0x5000, "CSF_E_SHAPE"),
    ("short_stride", _fake(stride=240), 0x5000, "CSF_E_SIZE"),
    ("odd_stride", _fake(stride=264), 0x5000, "CSF_E_SIZE"),
    ("huge_stride", _fake(stride=1 << 31), 0x5000, "CSF_E_SIZE"),
    ("negative_entries", _fake(n=-1), 0x5000, "CSF_E_SIZE"),
    ("misaligned_offsets", _fake(offsets=0x2008), 0x5000, "CSF_E_ALIGN"),
    ("misaligned_prefix", _fake(prefix=0x4002), 0x5000, "CSF_E_ALIGN"),
    ("misaligned_exc", _fake(exc=0x3001), 0x5000, "CSF_E_ALIGN"),
    ("misaligned_index", _fake(tile_index=0x8002), 0x5000, "CSF_E_ALIGN"),
]


@pytest.mark.parametrize("name,desc,ws,want", DECODE_ERRORS, ids=[e[0] for e in DECODE_ERRORS])
def test_decode_rejects_bad_arguments(lib, name, desc, ws, want):
    ref = ctypes.byref(desc) if desc is not None else None
    st = lib.csf_decode(ref, ws, None, None)
    assert mwd.STATUS[st] == want


def test_paired_and_passes_errors(lib):
    a, b = _fake(E=4), _fake(E=5)
    assert mwd.STATUS[lib.csf_decode_paired(ctypes.byref(a), 0x5000, ctypes.byref(b), 0x6000, None,
                                            None)] == "CSF_E_MISMATCH"
    assert mwd.STATUS[lib.csf_decode_paired(ctypes.byref(a), 0x5000, None, 0x6000, None,
                                            None)] == "CSF_E_NULL"
    assert mwd.STATUS[lib.csf_decode_paired(ctypes.byref(a), 0x5000, ctypes.byref(a), None, None,
                                            None)] == "CSF_E_NULL"
    for passes in (0, 4, 7):
        assert mwd.STATUS[lib.csf_decode_passes(ctypes.byref(a), 0x5000, None, None, None, passes,
                                                None)] == "CSF_E_SIZE"
    assert mwd.STATUS[lib.csf_decode(ctypes.byref(a), 0x5000, 0x7002, None)] == "CSF_E_ALIGN"
    assert mwd.STATUS[lib.csf_decode_i64(ctypes.byref(a), 0x5000, None, None, 0x7004, None)] == "CSF_E_ALIGN"
    assert mwd.STATUS[lib.csf_decode_i64(ctypes.byref(a), 0x5000, ctypes.byref(b), 0x6000, 0x7000,
                                         None)] == "CSF_E_MISMATCH"
    assert mwd.STATUS[lib.csf_decode_i64(None, 0x5000, None, None, 0x7000, None)] == "CSF_E_NULL"
    assert mwd.STATUS[lib.csf_build_index(ctypes.byref(a), None, None)] == "CSF_E_NULL"
    assert mwd.STATUS[lib.csf_build_index(ctypes.byref(a), 0x9002, None)] == "CSF_E_ALIGN"
    assert mwd.STATUS[lib.csf_build_index(ctypes.byref(_fake(E=0)), 0x9000, None)] == "CSF_E_SHAPE"


def test_decode_rows_windows(lib):
    a, b = _fake(R=64), _fake(R=32)
    ws = 0x5000

    def call(ra, rb=None, second=None, passes=3):
        r1 = mwd.csf_rows(*ra) if ra is not None else None
        r2 = mwd.csf_rows(*rb) if rb is not None else None
        return mwd.STATUS[lib.csf_decode_rows(ctypes.byref(a), ws, None if r1 is None else ctypes.byref(r1),
                                              None if second is None else ctypes.byref(second),
                                              0x6000 if second is not None else None,
                                              None if r2 is None else ctypes.byref(r2), None, passes, None)]

    for bad in ((-1, 4), (5, 4), (0, 65), (64, 65)):
        assert call(bad) == "CSF_E_SHAPE", bad
        assert call((0, 0), bad, second=b) in ("CSF_E_SHAPE",), bad
    assert call((0, 64), (0, 33), second=b) == "CSF_E_SHAPE"
    assert call((0, 4), passes=0) == "CSF_E_SIZE"
    # empty windows launch nothing (no HIP call on this GPU-less host)
    assert call((0, 0)) == "CSF_OK"
    assert call((64, 64)) == "CSF_OK"
    assert call((7, 7), (32, 32), second=b) == "CSF_OK"
    assert mwd.STATUS[lib.csf_decode_rows(None, ws, None, None, None, None, None, 3, None)] == "CSF_E_NULL"


def test_moe_w4a16_errors(lib):
    def call(desc, dense=None, w=0x10000, x=0x20000, T=4, alpha=0x30000, es=0x40000, y=0x50000):
        return mwd.STATUS[lib.csf_moe_w4a16(ctypes.byref(desc) if desc is not None else None, dense, w, x, T,
                                            alpha, es, y, None)]
    ok = _fake(R=32, C=16, stride=16 * 16, tile_index=0x8000)
    assert call(_fake(fmt=5, R=32, C=16, stride=16 * 64, tile_index=0x8000)) == "CSF_E_FORMAT"
    assert call(_fake(fmt=1, R=32, C=257, stride=16 * 128, tile_index=0x8000)) == "CSF_E_SHAPE"  # MXFP4 K = 8224
    assert call(_fake(R=32, C=15, stride=16 * 15, tile_index=0x8000)) == "CSF_E_SHAPE"   # K = 240
    assert call(_fake(R=32, C=514, stride=16 * 514, tile_index=0x8000)) == "CSF_E_SHAPE"  # K > 8192
    assert call(_fake(R=32, C=16, stride=16 * 16)) == "CSF_E_NULL"        # no tile index, no dense scales
    assert call(ok, w=None) == "CSF_E_NULL"
    assert call(ok, alpha=None) == "CSF_E_NULL"
    assert call(ok, x=None) == "CSF_E_NULL"
    assert call(ok, T=-1) == "CSF_E_SIZE"
    assert call(ok, w=0x10008) == "CSF_E_ALIGN"
    assert call(ok, y=0x50002) == "CSF_E_ALIGN"
    assert call(ok, T=0, x=None, dense=0x60001) == "CSF_E_ALIGN"          # NVFP4 dense scales: 2 bytes
    mx = _fake(fmt=1, R=32, C=5, stride=16 * 2, tile_index=0x8000)      # MXFP4, K = 160, C odd
    assert call(mx, T=0, x=None, dense=0x60001) == "CSF_OK"               # MXFP4 dense scales: bytes
    assert call(None) == "CSF_E_NULL"
    assert call(ok, T=0, x=None) == "CSF_OK"                              # nothing to do, nothing launched
    assert call(ok, T=0, x=None, y=None) == "CSF_OK"                      # no tokens: no output rows either
    assert call(ok, y=None) == "CSF_E_NULL"


def test_encode_device_errors(lib):
    f = lib.csf_encode_device
    ok = dict(dense=0x1000, bases=0x2000, offsets=0x3000, exc=0x4000, prefix=0x5000, tidx=0x6000)

    def call(fmt=0, E=2, R=3, C=4, phase=1, **kw):
        p = dict(ok, **kw)
        return mwd.STATUS[f(fmt, E, R, C, p["dense"], p["bases"], p["offsets"], p["exc"], p["prefix"],
                            p["tidx"], phase, None)]
    assert call(fmt=3) == "CSF_E_FORMAT"
    assert call(R=0) == "CSF_E_SHAPE"
    assert call(phase=0) == "CSF_E_SIZE" and call(phase=3) == "CSF_E_SIZE"
    assert call(E=2048, R=1024, C=1024) == "CSF_E_SIZE"  # E*R*C >= 2^31
    assert call(dense=None) == "CSF_E_NULL"
    assert call(tidx=None) == "CSF_E_NULL"
    assert call(offsets=None) == "CSF_E_NULL"
    assert call(phase=2, exc=None) == "CSF_E_NULL"
    assert call(offsets=0x3004) == "CSF_E_ALIGN"
    assert call(prefix=0x5001) == "CSF_E_ALIGN"
    assert call(phase=2, exc=0x4002) == "CSF_E_ALIGN"


def test_prepare_errors(lib):
    sz = mwd.csf_sizes()
    x = np.zeros((2, 3, 4), dtype=np.uint8)
    st = lib.csf_prepare(9, 2, 3, 4, x.ctypes.data, ctypes.byref(sz), None, None, None, None, None)
    assert mwd.STATUS[st] == "CSF_E_FORMAT"
    st = lib.csf_prepare(0, 2, 0, 4, x.ctypes.data, ctypes.byref(sz), None, None, None, None, None)
    assert mwd.STATUS[st] == "CSF_E_SHAPE"
    st = lib.csf_prepare(0, 2, 3, 4, None, ctypes.byref(sz), None, None, None, None, None)
    assert mwd.STATUS[st] == "CSF_E_NULL"
    buf = np.zeros(64, dtype=np.uint8)
    st = lib.csf_prepare(0, 2, 3, 4, x.ctypes.data, ctypes.byref(sz), buf.ctypes.data, None, None, None,
                         None)
    assert mwd.STATUS[st] == "CSF_E_NULL"
    st = lib.csf_prepare(0, 2, 3, 4, x.ctypes.data, ctypes.byref(sz), None, None, None, None,
                         buf.ctypes.data)
    assert mwd.STATUS[st] == "CSF_E_NULL"


def test_traced_decode_host_checks(lib):
    """The traced decode's two-call pattern and errors, decided on the host
    before anything is launched (descriptors with fake device pointers)."""
    a = _fake(E=512, R=800, C=128, stride=51200, tile_index=0x9000)
    b = _fake(E=512, R=2048, C=50, stride=51200, tile_index=0xA000)
    groups = ctypes.c_uint32(0)
    args = (ctypes.byref(a), 0x5000, ctypes.byref(b), 0x6000)
    st = lib.csf_decode_traced(*args, 0x7000, None, 0, ctypes.byref(groups), None)
    assert mwd.STATUS[st] == "CSF_OK" and groups.value > 0
    st = lib.csf_decode_traced(*args, 0x7000, 0x8000, 8 * groups.value - 1, ctypes.byref(groups), None)
    assert mwd.STATUS[st] == "CSF_E_SIZE"
    assert mwd.STATUS[lib.csf_decode_traced(*args, None, None, 0, ctypes.byref(groups), None)] == "CSF_E_NULL"
    assert mwd.STATUS[lib.csf_decode_traced(*args, 0x7000, None, 0, None, None)] == "CSF_E_NULL"
    c = _fake(E=512, R=800, C=128, stride=51200)
    st = lib.csf_decode_traced(ctypes.byref(c), 0x5000, None, None, 0x7000, None, 0, ctypes.byref(groups), None)
    assert mwd.STATUS[st] == "CSF_E_NULL"


def test_prepare_many_on_host_arrays_equals_prepare():
    """Host arrays take the host encoder, stack by stack."""
    xs = [workloads.nvfp4_stack(2, 8, 20, 5, 0.1), workloads.mxfp4_stack(1, 4, 64, 6, 0.2)]
    fmts = [workloads.NVFP4, workloads.MXFP4]
    got = mwd.prepare_many(xs, fmts)
    for x, f, g in zip(xs, fmts, got):
        want = mwd.prepare(x, f).numpy()
        have = g.numpy()
        for k in ("bases", "offsets", "exceptions", "prefix", "tile_index"):
            assert np.array_equal(np.asarray(have[k]).ravel(), np.asarray(want[k]).ravel()), k
    with pytest.raises(ValueError):
        mwd.prepare_many(xs, fmts[:1])
