"""GPU parity: the HIP decoder, called through the C ABI, against the CPU oracle.

Every comparison is byte-exact over whole planes.  Inputs come from the seeded
generators; the compressed streams fed to the GPU are the oracle's encodings
(and, separately, the library encoder's), and the expected bytes are the
oracle's decode of the same stream (which the oracle pins tie to the input x).

Decode tests run twice: "fused" (stacks carry the tile index: one kernel
patches exceptions on chip) and "two_pass" (no index: fixed-stream kernel,
then the exception kernel).
"""
import numpy as np
import pytest
import torch

import workloads

mwd = pytest.importorskip("moe_weight_decode_amd")

pytestmark = pytest.mark.gpu

POISON = 0xA5
GUARD = 0x5A
GUARD_BYTES = 4096


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


MODES = ["fused", "two_pass"]


def upload(st: dict, dev, mode="fused") -> "mwd.CompressedStack":
    stack = mwd.from_numpy(st, dev)
    return stack.without_index() if mode == "two_pass" else stack


def run_decode(stack, dev, es=None, fill=POISON, offset=0):
    """Decode into a guarded workspace starting `offset` bytes into its buffer;
    returns the dense bytes and asserts the guard bands are intact."""
    n = stack.dense_bytes
    buf = torch.full((GUARD_BYTES + offset + n + GUARD_BYTES,), GUARD, dtype=torch.uint8, device=dev)
    ws = buf[GUARD_BYTES + offset: GUARD_BYTES + offset + n]
    ws.fill_(fill)
    es_t = None if es is None else torch.from_numpy(np.ascontiguousarray(es, dtype=np.int32)).to(dev)
    mwd.decode(stack, ws, es_t)
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    assert np.all(h[:GUARD_BYTES + offset] == GUARD), "write before the workspace"
    assert np.all(h[GUARD_BYTES + offset + n:] == GUARD), "write past the workspace"
    return h[GUARD_BYTES + offset: GUARD_BYTES + offset + n].reshape(stack.E, stack.R, stack.C)


def oracle_expect(orc, st: dict, es=None, fill=POISON):
    ws = np.full((st["E"], st["R"], st["C"]), fill, dtype=np.uint8)
    return orc.decode(st, es, ws)


def assert_bytes_equal(got, want, what=""):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        e, r, c = bad[0]
        raise AssertionError(f"{what}: {len(bad)} bytes differ; first at expert {e} row {r} col {c}: "
                             f"gpu {got[e, r, c]:#x} oracle {want[e, r, c]:#x}")


# -- full-size and small stacks ------------------------------------------------

_cache = {}


def stack_case(name, orc):
    if name not in _cache:
        spec = workloads.STACKS[name]
        x = spec.generate()
        _cache[name] = (spec, x, orc.encode(spec.fmt, x))
    return _cache[name]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", ["tiny_nvfp4", "gate_nvfp4", "down_nvfp4", "mxfp4"])
def test_full_decode_matches_oracle(orc, dev, name, mode):
    spec, x, st = stack_case(name, orc)
    print(f"[parity] full decode {name} {mode} {x.shape} entries={st['exceptions'].size}", flush=True)
    got = run_decode(upload(st, dev, mode), dev)
    want = oracle_expect(orc, st)
    assert_bytes_equal(got, want, name)
    assert_bytes_equal(got, x, name + " vs input")


@pytest.mark.parametrize("name", ["tiny_nvfp4", "down_nvfp4", "mxfp4"])
def test_library_encoded_stream_decodes(orc, dev, name):
    spec, x, st = stack_case(name, orc)
    lib_stack = mwd.prepare(torch.from_numpy(x).to(dev), spec.fmt)
    assert lib_stack.device.type == "cuda"  # preparation keeps the input's device
    for mode_stack in (lib_stack, lib_stack.without_index()):
        assert_bytes_equal(run_decode(mode_stack, dev), x, name)


@pytest.mark.parametrize("name", ["tiny_nvfp4", "gate_nvfp4", "down_nvfp4", "mxfp4"])
def test_gpu_index_matches_oracle(orc, dev, name):
    spec, x, st = stack_case(name, orc)
    stack = upload(st, dev).without_index()
    idx = mwd.build_index(stack)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), st["tile_index"])
    assert_bytes_equal(run_decode(stack, dev), x, name + " with the GPU-built index")


RAGGED = [
    # (fmt, E, R, C): plane sizes with tails, every row mode, tiny and wide planes
    (workloads.NVFP4, 3, 5, 7),
    (workloads.NVFP4, 2, 7, 50),
    (workloads.NVFP4, 5, 33, 17),
    (workloads.NVFP4, 4, 1, 1),
    (workloads.NVFP4, 2, 300, 1),
    (workloads.NVFP4, 3, 9, 8),
    (workloads.NVFP4, 2, 41, 16),
    (workloads.NVFP4, 1, 1000, 129),
    (workloads.MXFP4, 3, 5, 7),
    (workloads.MXFP4, 2, 65, 160),
    (workloads.MXFP4, 3, 17, 18),
    (workloads.MXFP4, 2, 700, 3),
    (workloads.MXFP4, 1, 1, 1),
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("fmt,E,R,C", RAGGED, ids=[f"f{c[0]}_{c[1]}x{c[2]}x{c[3]}" for c in RAGGED])
def test_ragged_uniform_bytes(orc, dev, fmt, E, R, C, mode):
    x = workloads.uniform_bytes(E, R, C, seed=E * 1000 + R * 10 + C)
    st = orc.encode(fmt, x)
    got = run_decode(upload(st, dev, mode), dev)
    assert_bytes_equal(got, oracle_expect(orc, st), "uniform")
    assert_bytes_equal(got, x, "uniform vs input")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("fmt,E,R,C", [(workloads.NVFP4, 3, 1000, 50), (workloads.MXFP4, 3, 800, 160),
                                       (workloads.NVFP4, 2, 64, 8), (workloads.NVFP4, 2, 250, 130)])
def test_generated_distributions_small(orc, dev, fmt, E, R, C, mode):
    if fmt == workloads.NVFP4:
        x = workloads.nvfp4_stack(E, R, C, 21, 0.10, hot_row_frac=0.02)
    else:
        x = workloads.mxfp4_stack(E, R, C, 22, 0.15)
    st = orc.encode(fmt, x)
    assert_bytes_equal(run_decode(upload(st, dev, mode), dev), x, "generated")


@pytest.mark.parametrize("mode", MODES)
def test_largest_plane(orc, dev, mode):
    # R*C = 2^24 - 16: the largest plane an entry's 24-bit position can address
    R, C = 1048575, 16
    x = workloads.nvfp4_stack(1, R, C, 31, 0.05)
    st = orc.encode(workloads.NVFP4, x)
    assert_bytes_equal(run_decode(upload(st, dev, mode), dev), x, "largest plane")


@pytest.mark.parametrize("mode", MODES)
def test_most_experts(orc, dev, mode):
    x = workloads.nvfp4_stack(mwd.MAX_EXPERTS, 4, 24, 32, 0.2)
    st = orc.encode(workloads.NVFP4, x)
    assert_bytes_equal(run_decode(upload(st, dev, mode), dev), x, "2048 experts")
    es = workloads.routing(mwd.MAX_EXPERTS, 300, 5, seed=33)
    got = run_decode(upload(st, dev, mode), dev, es=es)
    assert_bytes_equal(got, oracle_expect(orc, st, es), "2048 experts routed")


def test_many_tiles_per_workgroup(orc, dev):
    # A routed call decodes 4096-position tiles on 2 workgroups per CU with the
    # pipelined loop, which reads the tile index bounds of 64 tiles at a time.
    # With all 2048 experts routed in a paired call and enough tiles per plane,
    # every workgroup decodes more than 64 tiles and reads bounds in batches.
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    E, C = mwd.MAX_EXPERTS, 128
    tiles = -(-64 * 2 * cus // (2 * E)) + 1
    R = tiles * 4096 // C
    assert 2 * E * tiles > 64 * 2 * cus
    xg = workloads.nvfp4_stack(E, R, C, 41, 0.03)
    xd = workloads.nvfp4_stack(E, R, C, 42, 0.10)
    g = upload(orc.encode(workloads.NVFP4, xg), dev)
    d = upload(orc.encode(workloads.NVFP4, xd), dev)
    es = torch.from_numpy(workloads.expert_start_from_mask(np.ones(E, dtype=bool), tokens=2)).to(dev)
    wg = torch.full((g.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
    wd = torch.full((d.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
    mwd.decode_paired(g, wg, d, wd, es)
    torch.cuda.synchronize()
    assert_bytes_equal(wg.cpu().numpy().reshape(xg.shape), xg, "gate half, every expert routed")
    assert_bytes_equal(wd.cpu().numpy().reshape(xd.shape), xd, "down half, every expert routed")


@pytest.mark.parametrize("mode", MODES)
def test_no_exceptions(orc, dev, mode):
    x = workloads.nvfp4_stack(4, 64, 128, 5, 0.0)
    st = orc.encode(workloads.NVFP4, x)
    assert st["exceptions"].size == 0
    stack = upload(st, dev, mode)
    assert stack.num_exceptions == 0 and stack.descriptor().exceptions is None
    assert_bytes_equal(run_decode(stack, dev), x, "no exceptions")


@pytest.mark.parametrize("mode", MODES)
def test_alternative_bases(orc, dev, mode):
    rng = np.random.default_rng(41)
    for fmt in (workloads.NVFP4, workloads.MXFP4):
        x = workloads.uniform_bytes(3, 50, 50, 42 + fmt)
        st = orc.encode_with_bases(fmt, x, rng.integers(0, 256, (3, 50), dtype=np.uint8))
        assert_bytes_equal(run_decode(upload(st, dev, mode), dev), x, "random bases")


@pytest.mark.parametrize("mode", MODES)
def test_arbitrary_offset_fields(orc, dev, mode):
    """Streams the encoder never writes (random fields everywhere, wrapping
    sums, fields past the plane) still decode exactly as the oracle does."""
    rng = np.random.default_rng(43)
    for fmt, (E, R, C) in ((workloads.NVFP4, (3, 37, 50)), (workloads.MXFP4, (2, 21, 33))):
        st = orc.encode(fmt, workloads.uniform_bytes(E, R, C, 44))
        st = dict(st)
        st["offsets"] = rng.integers(0, 256, st["offsets"].size, dtype=np.uint8)
        st["bases"] = rng.integers(0, 256, st["bases"].size, dtype=np.uint8)
        assert_bytes_equal(run_decode(upload(st, dev, mode), dev), oracle_expect(orc, st), "random fields")


@pytest.mark.parametrize("mode", MODES)
def test_entries_outside_plane_are_dropped(orc, dev, mode):
    x = np.full((3, 2, 8), 0x40, dtype=np.uint8)
    st = dict(orc.encode(workloads.NVFP4, x))
    st["exceptions"] = np.array([(3 << 8) | 0x99, (16 << 8) | 0x77, (20 << 8) | 0x11,
                                 (15 << 8) | 0x33, (1 << 23 | 5) << 8 | 0x44], dtype=np.uint32)
    st["prefix"] = np.array([0, 3, 4, 5], dtype=np.int32)
    st["tile_index"] = orc.build_index(st)
    for es in (None, np.array([0, 1, 1, 2], dtype=np.int32)):
        got = run_decode(upload(st, dev, mode), dev, es=es)
        assert_bytes_equal(got, oracle_expect(orc, st, es), "out-of-plane entries")


# -- routing -------------------------------------------------------------------

@pytest.mark.parametrize("mode", MODES)
def test_tiny_every_routed_subset(orc, dev, mode):
    spec, x, st = stack_case("tiny_nvfp4", orc)
    stack = upload(st, dev, mode)
    for m in range(1 << spec.E):
        mask = np.array([(m >> e) & 1 for e in range(spec.E)])
        es = workloads.expert_start_from_mask(mask, tokens=2)
        got = run_decode(stack, dev, es=es)
        assert_bytes_equal(got, oracle_expect(orc, st, es), f"subset {mask}")


@pytest.mark.parametrize("mode", MODES)
def test_routed_garbage_expert_start(orc, dev, mode):
    spec, x, st = stack_case("tiny_nvfp4", orc)
    es = np.array([0, 5, 5, 3, -7], dtype=np.int32)  # only expert 0 has tokens
    got = run_decode(upload(st, dev, mode), dev, es=es)
    assert_bytes_equal(got, oracle_expect(orc, st, es), "garbage expert_start")


def _paired(orc, dev, es, mode, fill=POISON):
    _, xg, sg = stack_case("gate_nvfp4", orc)
    _, xd, sd = stack_case("down_nvfp4", orc)
    g, d = upload(sg, dev, mode), upload(sd, dev, mode)
    wg = torch.full((g.dense_bytes,), fill, dtype=torch.uint8, device=dev)
    wd = torch.full((d.dense_bytes,), fill, dtype=torch.uint8, device=dev)
    es_t = None if es is None else torch.from_numpy(es).to(dev)
    mwd.decode_paired(g, wg, d, wd, es_t)
    torch.cuda.synchronize()
    return (wg.cpu().numpy().reshape(xg.shape), wd.cpu().numpy().reshape(xd.shape),
            oracle_expect(orc, sg, es, fill), oracle_expect(orc, sd, es, fill))


@pytest.mark.parametrize("mode", MODES)
def test_routed_paired_gate_down(orc, dev, mode):
    es = workloads.ROUTED.expert_start()
    print(f"[parity] routed paired {mode}, active experts {np.nonzero(np.diff(es))[0].tolist()}", flush=True)
    gg, gd, wg, wd = _paired(orc, dev, es, mode)
    assert_bytes_equal(gg, wg, "routed gate")
    assert_bytes_equal(gd, wd, "routed down")
    inactive = np.diff(es) <= 0
    assert np.all(gg[inactive] == POISON) and np.all(gd[inactive] == POISON)


@pytest.mark.parametrize("n_active", [1, 60, 120, 250, 511])
def test_two_pass_routed_entry_spread(orc, dev, n_active):
    """Routed two-pass decodes of the gate stack with 1 to 511 of 512 experts
    routed: the exception pass spreads the routed entries over its grid in
    chunks of 1, 2, 4 or 8 entries per lane, and with most experts routed a
    workgroup takes several chunks."""
    _, _, st = stack_case("gate_nvfp4", orc)
    rng = np.random.default_rng(4100 + n_active)
    act = np.zeros(512, bool)
    act[rng.choice(512, n_active, replace=False)] = True
    es = workloads.expert_start_from_mask(act, tokens=3)
    print(f"[parity] two-pass routed gate, {n_active} experts routed", flush=True)
    got = run_decode(upload(st, dev, "two_pass"), dev, es)
    assert_bytes_equal(got, oracle_expect(orc, st, es), f"{n_active} routed")
    assert np.all(got[~act] == POISON), "unrouted planes written"


@pytest.mark.parametrize("mode", MODES)
def test_paired_full_and_all_inactive(orc, dev, mode):
    gg, gd, wg, wd = _paired(orc, dev, None, mode)
    assert_bytes_equal(gg, wg, "paired gate")
    assert_bytes_equal(gd, wd, "paired down")
    es = np.zeros(513, dtype=np.int32)
    gg, gd, _, _ = _paired(orc, dev, es, mode)
    assert np.all(gg == POISON) and np.all(gd == POISON), "no expert routed: nothing written"


@pytest.mark.parametrize("mode", MODES)
def test_paired_all_active_equals_full(orc, dev, mode):
    es = workloads.expert_start_from_mask(np.ones(512, dtype=np.int64), tokens=1)
    gg, gd, wg, wd = _paired(orc, dev, es, mode)
    _, xg, _ = stack_case("gate_nvfp4", orc)
    _, xd, _ = stack_case("down_nvfp4", orc)
    assert_bytes_equal(gg, xg, "all active gate")
    assert_bytes_equal(gd, xd, "all active down")


def _skewed_stack(E, R, C, seed, where):
    """NVFP4 planes with few outliers except a band of rows of uniform bytes
    (nearly all outliers) near the plane's start, middle or end."""
    x = workloads.nvfp4_stack(E, R, C, seed, 0.01)
    u = workloads.uniform_bytes(E, R, C, seed + 1)
    band = {"start": slice(0, R // 8), "middle": slice(R // 2 - R // 16, R // 2 + R // 16),
            "end": slice(R - R // 8, R)}[where]
    x[:, band, :] = u[:, band, :]
    return x


@pytest.mark.parametrize("where", ["start", "middle", "end"])
def test_routed_tiles_with_many_entries(orc, dev, where):
    """Routed tiles with more entries than a workgroup prefetches read the rest
    from the stream directly; the traced decode shows such tiles occurred and
    its output is the plain decode's."""
    E, R, C = 12, 2048, 50
    x = _skewed_stack(E, R, C, 91 + len(where), where)
    st = orc.encode(workloads.NVFP4, x)
    stack = upload(st, dev)
    es = workloads.expert_start_from_mask(np.array([1, 0, 1, 1, 0, 0, 1, 0, 0, 1, 1, 0]), tokens=3)
    print(f"[parity] routed tiles with many entries, band at {where}", flush=True)
    assert_bytes_equal(run_decode(stack, dev, es=es), oracle_expect(orc, st, es), f"routed, band at {where}")
    ws = torch.full((stack.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
    stamps = mwd.decode_traced(stack, ws, expert_start=torch.from_numpy(es).to(dev))
    torch.cuda.synchronize()
    assert_bytes_equal(ws.cpu().numpy().reshape(x.shape), oracle_expect(orc, st, es), "traced")
    tags = stamps[:, 7].cpu().numpy().astype(np.uint64)
    assert np.any(tags >> np.uint64(32) == 1), "no tile had more entries than prefetched: the case is not exercised"


def test_traced_decode_stamps(orc, dev):
    """The traced routed pair writes what csf_decode_paired writes, one tag
    per routed tile, and clock values in step order."""
    es = workloads.ROUTED.expert_start()
    _, xg, sg = stack_case("gate_nvfp4", orc)
    _, xd, sd = stack_case("down_nvfp4", orc)
    g, d = upload(sg, dev), upload(sd, dev)
    wg = torch.full((g.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
    wd = torch.full((d.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
    stamps = mwd.decode_traced(g, wg, d, wd, torch.from_numpy(es).to(dev))
    torch.cuda.synchronize()
    assert_bytes_equal(wg.cpu().numpy().reshape(xg.shape), oracle_expect(orc, sg, es), "traced gate")
    assert_bytes_equal(wd.cpu().numpy().reshape(xd.shape), oracle_expect(orc, sd, es), "traced down")
    t = stamps.cpu().numpy().astype(np.uint64)
    tags = t[:, 7]
    units = int(np.count_nonzero(np.diff(es) > 0)) * (g.tiles_per_plane(4096) + d.tiles_per_plane(4096))
    busy = (tags != 0) & (tags != np.uint64(0xFFFFFFFFFFFFFFFF))
    assert int(busy.sum()) == units
    assert sorted(int(v & np.uint64(0xFFFFFFFF)) - 1 for v in tags[busy]) == list(range(units))
    for row in t[busy]:
        assert all(row[i] <= row[i + 1] for i in range(6)), row
    assert np.all(t[:, 0] <= t[:, 1])


def test_routed_without_exceptions_and_empty_experts(orc, dev):
    """Routed stacks with no entry at all (no entry buffer), and experts
    without entries between experts with many."""
    x = workloads.nvfp4_stack(6, 300, 64, 95, 0.0)
    st = orc.encode(workloads.NVFP4, x)
    assert st["exceptions"].size == 0
    es = workloads.expert_start_from_mask(np.array([0, 1, 1, 0, 1, 1]), tokens=2)
    assert_bytes_equal(run_decode(upload(st, dev), dev, es=es), oracle_expect(orc, st, es), "no entries")
    x[1] = workloads.uniform_bytes(1, 300, 64, 96)[0]
    x[4] = workloads.uniform_bytes(1, 300, 64, 97)[0]
    st = orc.encode(workloads.NVFP4, x)
    es = workloads.expert_start_from_mask(np.array([1, 1, 1, 0, 1, 1]), tokens=2)
    assert_bytes_equal(run_decode(upload(st, dev), dev, es=es), oracle_expect(orc, st, es), "mixed")


@pytest.mark.parametrize("mode", MODES + ["one_indexed"])
def test_paired_mixed_formats(orc, dev, mode):
    xa = workloads.nvfp4_stack(16, 100, 50, 51, 0.1)
    xb = workloads.mxfp4_stack(16, 60, 160, 52, 0.15)
    sa, sb = orc.encode(workloads.NVFP4, xa), orc.encode(workloads.MXFP4, xb)
    a = upload(sa, dev, "two_pass" if mode == "two_pass" else "fused")
    b = upload(sb, dev, "fused" if mode == "fused" else "two_pass")
    es = workloads.routing(16, 5, 9, seed=53)
    wa = torch.full((a.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
    wb = torch.full((b.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
    mwd.decode_paired(a, wa, b, wb, torch.from_numpy(es).to(dev))
    torch.cuda.synchronize()
    assert_bytes_equal(wa.cpu().numpy().reshape(xa.shape), oracle_expect(orc, sa, es), "mixed a")
    assert_bytes_equal(wb.cpu().numpy().reshape(xb.shape), oracle_expect(orc, sb, es), "mixed b")


# -- workspace, passes, streams, graphs -----------------------------------------

@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("offset", [1, 3, 7, 15])
def test_odd_offset_workspace(orc, dev, offset, mode):
    for name in ("tiny_nvfp4", "mxfp4"):
        spec, x, st = stack_case(name, orc)
        got = run_decode(upload(st, dev, mode), dev, offset=offset)
        assert_bytes_equal(got, x, f"{name} at offset {offset}")
    es = workloads.expert_start_from_mask(np.array([1, 0, 1, 1]), tokens=1)
    spec, x, st = stack_case("tiny_nvfp4", orc)
    got = run_decode(upload(st, dev, mode), dev, es=es, offset=offset)
    assert_bytes_equal(got, oracle_expect(orc, st, es), "routed odd offset")


def test_passes_one_at_a_time(orc, dev):
    spec, x, st = stack_case("down_nvfp4", orc)
    stack = upload(st, dev)
    ws = torch.full((stack.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
    mwd.decode_passes(stack, ws, passes=mwd.PASS_FIXED)
    torch.cuda.synchronize()
    fixed_only = ws.cpu().numpy().reshape(x.shape)
    # after the fixed stream alone every exception position holds its row base
    no_exc = dict(st)
    no_exc["exceptions"] = np.zeros(0, dtype=np.uint32)
    no_exc["prefix"] = np.zeros(spec.E + 1, dtype=np.int32)
    assert_bytes_equal(fixed_only, orc.decode(no_exc), "fixed pass")
    mwd.decode_passes(stack, ws, passes=mwd.PASS_EXCEPTIONS)
    torch.cuda.synchronize()
    assert_bytes_equal(ws.cpu().numpy().reshape(x.shape), x, "fixed then exceptions")


@pytest.mark.parametrize("mode", MODES)
def test_repeat_is_deterministic(orc, dev, mode):
    spec, x, st = stack_case("mxfp4", orc)
    stack = upload(st, dev, mode)
    ws = torch.empty(stack.dense_bytes, dtype=torch.uint8, device=dev)
    ref = torch.from_numpy(x.reshape(-1)).to(dev)
    for i in range(20):
        ws.fill_(i)
        mwd.decode(stack, ws)
        assert torch.equal(ws, ref), f"repeat {i}"


def test_side_stream_ordering(orc, dev):
    spec, x, st = stack_case("gate_nvfp4", orc)
    stack = upload(st, dev)
    ws = torch.full((stack.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        mwd.decode(stack, ws)  # current stream is the side stream
        done = torch.cuda.Event()
        done.record(side)
    torch.cuda.current_stream(dev).wait_event(done)
    ref = torch.from_numpy(x.reshape(-1)).to(dev)
    assert torch.equal(ws, ref)


@pytest.mark.parametrize("mode", MODES)
def test_graph_replay_follows_routing(orc, dev, mode):
    """One captured paired decode replayed with three routings, poisoned
    workspaces in between; the library allocates nothing during capture."""
    _, xg, sg = stack_case("gate_nvfp4", orc)
    _, xd, sd = stack_case("down_nvfp4", orc)
    g, d = upload(sg, dev, mode), upload(sd, dev, mode)
    wg = torch.empty(g.dense_bytes, dtype=torch.uint8, device=dev)
    wd = torch.empty(d.dense_bytes, dtype=torch.uint8, device=dev)
    es_t = torch.zeros(513, dtype=torch.int32, device=dev)
    routings = [workloads.ROUTED.expert_start(), workloads.routing(512, 40, 3, seed=61),
                workloads.expert_start_from_mask(np.ones(512, dtype=np.int64))]
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):  # warm the launch path outside capture
        mwd.decode_paired(g, wg, d, wd, es_t)
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        # the capture context allocates graph-safe RNG state of its own; the
        # decode call itself must allocate nothing
        allocated, reserved = torch.cuda.memory_allocated(dev), torch.cuda.memory_reserved(dev)
        mwd.decode_paired(g, wg, d, wd, es_t)
        assert torch.cuda.memory_allocated(dev) == allocated
        assert torch.cuda.memory_reserved(dev) == reserved
    for rnd in range(2):
        for i, es in enumerate(routings):
            wg.fill_(POISON)
            wd.fill_(POISON)
            es_t.copy_(torch.from_numpy(es))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert_bytes_equal(wg.cpu().numpy().reshape(xg.shape), oracle_expect(orc, sg, es),
                               f"replay {rnd}.{i} gate")
            assert_bytes_equal(wd.cpu().numpy().reshape(xd.shape), oracle_expect(orc, sd, es),
                               f"replay {rnd}.{i} down")


# -- the GPU encoder ------------------------------------------------------------

def _same_streams(got: dict, want: dict, what: str):
    for k in ("fmt", "E", "R", "C", "stride"):
        assert got[k] == want[k], f"{what}: {k}"
    for k in ("bases", "offsets", "exceptions", "prefix", "tile_index"):
        g, w = np.asarray(got[k]).ravel(), np.asarray(want[k]).ravel()
        if not np.array_equal(g, w):
            bad = np.nonzero(g[:min(g.size, w.size)] != w[:min(g.size, w.size)])[0]
            raise AssertionError(f"{what}: {k} differs (sizes {g.size} vs {w.size}; first at {bad[:5]})")


@pytest.mark.parametrize("name", ["tiny_nvfp4", "gate_nvfp4", "down_nvfp4", "mxfp4"])
def test_gpu_encoder_matches_oracle(orc, dev, name):
    spec, x, st = stack_case(name, orc)
    print(f"[parity] gpu encode {name}", flush=True)
    got = mwd.prepare(torch.from_numpy(x).to(dev), spec.fmt)
    torch.cuda.synchronize()
    _same_streams(got.numpy(), st, name)
    assert_bytes_equal(run_decode(got, dev), x, name + " decoded")


ENCODE_SHAPES = RAGGED + [(workloads.NVFP4, 2, 3000, 50), (workloads.MXFP4, 2, 1500, 160),
                          (workloads.NVFP4, 1, 1048575, 16),
                          # stacks of a multiple of 4 bytes with rows of at most 255 columns (the
                          # 16-lanes-per-row base search), last group of 4 rows partial
                          (workloads.NVFP4, 3, 33, 12), (workloads.MXFP4, 1, 5, 4), (workloads.NVFP4, 2, 7, 254),
                          (workloads.MXFP4, 4, 7, 255), (workloads.NVFP4, 1, 255, 4), (workloads.MXFP4, 3, 100, 52),
                          # one column more than the byte-wide bins allow
                          (workloads.NVFP4, 4, 5, 256),
                          # more index tiles (E x tiles per plane) than the scan keeps in
                          # registers: its counts are read twice
                          (workloads.NVFP4, 40000, 3, 11), (workloads.MXFP4, 70001, 1, 3)]


@pytest.mark.parametrize("fmt,E,R,C", ENCODE_SHAPES, ids=[f"f{c[0]}_{c[1]}x{c[2]}x{c[3]}" for c in ENCODE_SHAPES])
def test_gpu_encoder_ragged(orc, dev, fmt, E, R, C):
    if R * C > 1 << 20:
        x = workloads.nvfp4_stack(E, R, C, 71, 0.05)
    else:
        x = workloads.uniform_bytes(E, R, C, seed=E * 7 + R * 3 + C)
    got = mwd.prepare(torch.from_numpy(x).to(dev), fmt)
    torch.cuda.synchronize()
    _same_streams(got.numpy(), orc.encode(fmt, x), f"{fmt} {E}x{R}x{C}")


def test_gpu_encoder_bases_above_256_minus_w(orc, dev):
    """A row's base is one of its values and may exceed 256 - W; bytes just
    above 0 then differ from it by less than W modulo 256 but lie below the
    window, so they are exceptions."""
    rng = np.random.default_rng(11)
    for fmt, top, low, C in ((workloads.NVFP4, 250, 6, 32), (workloads.NVFP4, 245, 10, 40),
                             (workloads.MXFP4, 255, 2, 32), (workloads.MXFP4, 255, 3, 17)):
        rows = []
        for _ in range(2 * 8):
            row = np.concatenate([np.full(C - low, top), np.arange(low)]).astype(np.uint8)
            rows.append(rng.permutation(row))
        x = np.stack(rows).reshape(2, 8, C)
        want = orc.encode(fmt, x)
        assert (want["bases"] == top).all() and len(want["exceptions"]) == 2 * 8 * low
        got = mwd.prepare(torch.from_numpy(x).to(dev), fmt)
        torch.cuda.synchronize()
        _same_streams(got.numpy(), want, f"high bases {fmt} C={C}")


@pytest.mark.parametrize("shift", [1, 4, 8])
def test_gpu_encoder_unaligned_dense(orc, dev, shift):
    """A stack that starts 1, 4 or 8 bytes past a 16-byte boundary: the row
    bases come from the kernel for any alignment, the offset and entry passes
    read the bytes one by one."""
    for fmt, E, R, C in ((workloads.NVFP4, 3, 33, 50), (workloads.MXFP4, 2, 17, 160), (workloads.NVFP4, 2, 9, 128)):
        x = workloads.nvfp4_stack(E, R, C, 13, 0.08) if fmt == workloads.NVFP4 else workloads.mxfp4_stack(E, R, C, 13, 0.15)
        buf = torch.empty(x.size + 32, dtype=torch.uint8, device=dev)
        xd = buf[shift:shift + x.size].view(E, R, C)
        xd.copy_(torch.from_numpy(x))
        assert xd.data_ptr() % 16 == shift % 16
        got = mwd.prepare(xd, fmt)
        torch.cuda.synchronize()
        _same_streams(got.numpy(), orc.encode(fmt, x), f"shift {shift} {fmt} {E}x{R}x{C}")


def test_gpu_prepare_many_equals_one_by_one(orc, dev):
    """Several stacks (both formats, one without exceptions, one with rows
    wider than 255) encoded with one read-back of their entry counts, on the
    current and on a side stream."""
    xs = [(workloads.nvfp4_stack(3, 40, 50, 21, 0.1), workloads.NVFP4),
          (workloads.mxfp4_stack(2, 33, 160, 22, 0.15), workloads.MXFP4),
          (workloads.nvfp4_stack(2, 16, 128, 23, 0.0), workloads.NVFP4),
          (workloads.uniform_bytes(2, 3, 300, 24), workloads.NVFP4)]
    side = torch.cuda.Stream(device=dev)
    for stream in (None, side):
        got = mwd.prepare_many([torch.from_numpy(x).to(dev) for x, _ in xs], [f for _, f in xs], stream=stream)
        if stream is not None:
            torch.cuda.current_stream(dev).wait_stream(stream)
        torch.cuda.synchronize()
        assert got[2].num_exceptions == 0
        for (x, f), g in zip(xs, got):
            _same_streams(g.numpy(), orc.encode(f, x), f"prepare_many {f} {x.shape}")


def test_gpu_encoder_two_column_exhaustive(orc, dev):
    a, b = np.meshgrid(np.arange(256), np.arange(256), indexing="ij")
    x = np.stack([a.ravel(), b.ravel()], axis=1).astype(np.uint8).reshape(4, 16384, 2)
    for fmt in (workloads.NVFP4, workloads.MXFP4):
        got = mwd.prepare(torch.from_numpy(x).to(dev), fmt)
        torch.cuda.synchronize()
        _same_streams(got.numpy(), orc.encode(fmt, x), f"two-column {fmt}")


def test_gpu_encoder_no_exceptions_and_side_stream(orc, dev):
    x = workloads.nvfp4_stack(3, 64, 128, 5, 0.0)
    side = torch.cuda.Stream(device=dev)
    xt = torch.from_numpy(x).to(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        got = mwd.prepare(xt, workloads.NVFP4, stream=side)
    torch.cuda.current_stream(dev).wait_stream(side)
    assert got.num_exceptions == 0
    _same_streams(got.numpy(), orc.encode(workloads.NVFP4, x), "no exceptions")


def test_gpu_encoder_on_a_stream_that_is_not_current(orc, dev):
    """Outputs allocated on the current stream, written on another: after the
    caller's wait the streams equal the oracle's encoding."""
    x = workloads.nvfp4_stack(3, 64, 128, 7, 0.05)
    side = torch.cuda.Stream(device=dev)
    xt = torch.from_numpy(x).to(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    got = mwd.prepare(xt, workloads.NVFP4, stream=side)
    torch.cuda.current_stream(dev).wait_stream(side)
    assert got.num_exceptions > 0
    _same_streams(got.numpy(), orc.encode(workloads.NVFP4, x), "encode on a side stream")


def test_gpu_encoder_side_stream_waits_for_freed_memory(orc, dev):
    """The current stream still writes memory freed just before the call, and
    the caller makes no wait: the encode on the side stream allocates its
    outputs from that memory and must still see none of those writes."""
    x = workloads.nvfp4_stack(64, 800, 128, 9, 0.03)
    xt = torch.from_numpy(x).to(dev)
    uploaded = torch.cuda.Event()
    uploaded.record(torch.cuda.current_stream(dev))
    side = torch.cuda.Stream(device=dev)
    side.wait_event(uploaded)  # the input is ready on the side stream; nothing else is ordered
    scratch = torch.empty(32 << 20, dtype=torch.uint8, device=dev)
    for i in range(200):  # queued work on the current stream, writing memory about to be freed
        scratch.fill_(i & 0xFF)
    del scratch
    got = mwd.prepare(xt, workloads.NVFP4, stream=side)
    torch.cuda.current_stream(dev).wait_stream(side)
    _same_streams(got.numpy(), orc.encode(workloads.NVFP4, x), "encode after freed memory")


def test_gpu_encoder_high_bases(orc, dev):
    """Rows whose base is above 240 next to small values: the window does not
    wrap past 255, so the small values are exceptions."""
    rng = np.random.default_rng(81)
    for fmt, W in ((workloads.NVFP4, 16), (workloads.MXFP4, 2)):
        base = rng.integers(241, 256, (3, 200), dtype=np.int64)
        off = rng.integers(0, W, (3, 200, 40))
        x = np.minimum(base[:, :, None] + off, 255)
        low = rng.random((3, 200, 40)) < 0.2
        x = np.where(low, rng.integers(0, 16, (3, 200, 40)), x).astype(np.uint8)
        want = orc.encode(fmt, x)
        got = mwd.prepare(torch.from_numpy(x).to(dev), fmt)
        torch.cuda.synchronize()
        _same_streams(got.numpy(), want, f"high bases {fmt}")
        assert_bytes_equal(run_decode(got, dev), x, "high bases decoded")


# -- int64 routing ----------------------------------------------------------------

@pytest.mark.parametrize("mode", MODES)
def test_routed_int64_expert_start(orc, dev, mode):
    """int64 expert_start with offsets beyond 2^32: the same planes as the
    int32 routing with the same token counts."""
    es32 = workloads.ROUTED.expert_start()
    es64 = es32.astype(np.int64) + (np.int64(5) << 40)
    _, xg, sg = stack_case("gate_nvfp4", orc)
    _, xd, sd = stack_case("down_nvfp4", orc)
    g, d = upload(sg, dev, mode), upload(sd, dev, mode)
    wg = torch.full((g.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
    wd = torch.full((d.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
    mwd.decode_paired(g, wg, d, wd, torch.from_numpy(es64).to(dev))
    torch.cuda.synchronize()
    assert_bytes_equal(wg.cpu().numpy().reshape(xg.shape), oracle_expect(orc, sg, es32), "int64 gate")
    assert_bytes_equal(wd.cpu().numpy().reshape(xd.shape), oracle_expect(orc, sd, es32), "int64 down")
    # single stack; the low 32 bits alone would say "no tokens" for expert 1
    spec, x, st = stack_case("tiny_nvfp4", orc)
    es = np.array([0, 1 << 33, (1 << 33) + 1, (1 << 33) + 1, (1 << 34)], dtype=np.int64)
    ws = torch.full((x.size,), POISON, dtype=torch.uint8, device=dev)
    mwd.decode(upload(st, dev, mode), ws, torch.from_numpy(es).to(dev))
    torch.cuda.synchronize()
    want = oracle_expect(orc, st, np.array([0, 1, 2, 2, 3], dtype=np.int32))
    assert_bytes_equal(ws.cpu().numpy().reshape(x.shape), want, "int64 single")


@pytest.mark.parametrize("wide", [False, True])
def test_two_pass_paired_many_experts(orc, dev, wide):
    """Two-pass paired decode of 600-expert NVFP4 and MXFP4 stacks with 300
    experts routed (int32, or int64 offsets beyond 2^32): the exception pass
    lists the routed experts in two steps of 512 and scans their entry counts
    in two steps of 256, for two stacks of different entry counts."""
    E = 600
    xa = workloads.nvfp4_stack(E, 40, 50, 8101, 0.10)
    xb = workloads.mxfp4_stack(E, 32, 40, 8102, 0.15)
    sa, sb = orc.encode(workloads.NVFP4, xa), orc.encode(workloads.MXFP4, xb)
    rng = np.random.default_rng(8103)
    act = np.zeros(E, bool)
    act[rng.choice(E, 300, replace=False)] = True
    es = workloads.expert_start_from_mask(act, tokens=2)
    es_dev = es.astype(np.int64) + (np.int64(3) << 36) if wide else es
    print(f"[parity] two-pass paired, 600 experts, 300 routed, wide {wide}", flush=True)
    a, b = upload(sa, dev, "two_pass"), upload(sb, dev, "two_pass")
    wa = torch.full((a.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
    wb = torch.full((b.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
    mwd.decode_paired(a, wa, b, wb, torch.from_numpy(es_dev).to(dev))
    torch.cuda.synchronize()
    assert_bytes_equal(wa.cpu().numpy().reshape(xa.shape), oracle_expect(orc, sa, es), "NVFP4 stack")
    assert_bytes_equal(wb.cpu().numpy().reshape(xb.shape), oracle_expect(orc, sb, es), "MXFP4 stack")


@pytest.mark.parametrize("mode", MODES)
def test_routed_expert_start_not_16_byte_aligned(orc, dev, mode):
    """expert_start tensors that start 4 or 12 (int32) or 8 (int64) bytes past
    a 16-byte boundary are read value by value instead of 16 bytes at a time:
    the same planes as from the aligned tensor."""
    es32 = workloads.ROUTED.expert_start()
    _, xg, sg = stack_case("gate_nvfp4", orc)
    _, xd, sd = stack_case("down_nvfp4", orc)
    g, d = upload(sg, dev, mode), upload(sd, dev, mode)
    want_g, want_d = oracle_expect(orc, sg, es32), oracle_expect(orc, sd, es32)
    for dtype, shift in ((torch.int32, 1), (torch.int32, 3), (torch.int64, 1)):
        print(f"[parity] routed pair, {dtype} expert_start {shift} elements past an aligned start", flush=True)
        buf = torch.zeros(len(es32) + 4, dtype=dtype, device=dev)
        es_t = buf[shift: shift + len(es32)]
        es_t.copy_(torch.from_numpy(es32).to(dev))
        assert es_t.data_ptr() % 16 != 0
        wg = torch.full((g.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
        wd = torch.full((d.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
        mwd.decode_paired(g, wg, d, wd, es_t)
        torch.cuda.synchronize()
        assert_bytes_equal(wg.cpu().numpy().reshape(xg.shape), want_g, f"gate, {dtype} shift {shift}")
        assert_bytes_equal(wd.cpu().numpy().reshape(xd.shape), want_d, f"down, {dtype} shift {shift}")


# -- row windows (decode only the rows a consumer reads) -----------------------

def run_decode_rows(stack, dev, rows, es=None, offset=0, second=None, rows_second=None):
    """csf_decode_rows into guarded, poisoned workspaces; returns the dense
    bytes of each stack and asserts the guard bands are intact."""
    stacks = [stack] + ([second] if second is not None else [])
    bufs, wss = [], []
    for s in stacks:
        n = s.dense_bytes
        buf = torch.full((GUARD_BYTES + offset + n + GUARD_BYTES,), GUARD, dtype=torch.uint8, device=dev)
        ws = buf[GUARD_BYTES + offset: GUARD_BYTES + offset + n]
        ws.fill_(POISON)
        bufs.append(buf)
        wss.append(ws)
    es_t = None if es is None else torch.from_numpy(np.ascontiguousarray(es, dtype=np.int32)).to(dev)
    mwd.decode_rows(stack, wss[0], rows, second, wss[1] if second is not None else None, rows_second, es_t)
    torch.cuda.synchronize()
    out = []
    for s, buf in zip(stacks, bufs):
        h = buf.cpu().numpy()
        n = s.dense_bytes
        assert np.all(h[:GUARD_BYTES + offset] == GUARD), "write before the workspace"
        assert np.all(h[GUARD_BYTES + offset + n:] == GUARD), "write past the workspace"
        out.append(h[GUARD_BYTES + offset: GUARD_BYTES + offset + n].reshape(s.E, s.R, s.C))
    return out


def oracle_rows(orc, st, rows, es=None):
    b, e = rows if rows is not None else (0, st["R"])
    return orc.decode_rows(st, b, e, es, np.full((st["E"], st["R"], st["C"]), POISON, dtype=np.uint8))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", ["gate_nvfp4", "down_nvfp4", "mxfp4"])
def test_row_window_full_stacks(orc, dev, name, mode):
    spec, x, st = stack_case(name, orc)
    R = spec.R
    stack = upload(st, dev, mode)
    for rows in ((0, R // 2), (R // 2, R), (37, R - 101)):
        got, = run_decode_rows(stack, dev, rows)
        assert_bytes_equal(got, oracle_rows(orc, st, rows), f"{name} rows {rows}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("fmt,E,R,C", [(workloads.NVFP4, 5, 300, 50), (workloads.MXFP4, 3, 200, 160),
                                       (workloads.NVFP4, 3, 2000, 7), (workloads.NVFP4, 4, 130, 128)],
                         ids=["nv_c50", "mx_c160", "nv_c7", "nv_c128"])
def test_row_window_small(orc, dev, fmt, E, R, C, mode):
    if fmt == workloads.NVFP4:
        x = workloads.nvfp4_stack(E, R, C, 61, 0.08, hot_row_frac=0.02)
    else:
        x = workloads.mxfp4_stack(E, R, C, 62, 0.15)
    st = orc.encode(fmt, x)
    stack = upload(st, dev, mode)
    rng = np.random.default_rng(R)
    windows = [(0, R), (0, R // 2), (R // 2, R), (0, 1), (R - 1, R), (0, 0), (R, R), (3, 4)]
    windows += [tuple(int(v) for v in sorted(rng.integers(0, R + 1, 2))) for _ in range(6)]
    es = workloads.expert_start_from_mask(np.arange(E) % 2 == 1, tokens=2)
    for rows in windows:
        got, = run_decode_rows(stack, dev, rows)
        assert_bytes_equal(got, oracle_rows(orc, st, rows), f"rows {rows}")
        got, = run_decode_rows(stack, dev, rows, es=es)
        assert_bytes_equal(got, oracle_rows(orc, st, rows, es), f"rows {rows} routed")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("offset", [1, 7])
def test_row_window_odd_offset_workspace(orc, dev, offset, mode):
    x = workloads.nvfp4_stack(3, 500, 50, 63, 0.05)
    st = orc.encode(workloads.NVFP4, x)
    stack = upload(st, dev, mode)
    for rows in ((0, 250), (123, 411)):
        got, = run_decode_rows(stack, dev, rows, offset=offset)
        assert_bytes_equal(got, oracle_rows(orc, st, rows), f"offset {offset} rows {rows}")


@pytest.mark.parametrize("mode", MODES)
def test_row_window_paired_gate_half(orc, dev, mode):
    # the gate half of the gate/up stack and every row of the down stack, routed
    _, xg, sg = stack_case("gate_nvfp4", orc)
    _, xd, sd = stack_case("down_nvfp4", orc)
    g, d = upload(sg, dev, mode), upload(sd, dev, mode)
    es = workloads.ROUTED.expert_start()
    half = (0, xg.shape[1] // 2)
    wg, wd = run_decode_rows(g, dev, half, es=es, second=d, rows_second=None)
    assert_bytes_equal(wg, oracle_rows(orc, sg, half, es), "gate half")
    assert_bytes_equal(wd, oracle_rows(orc, sd, None, es), "down, every row")
    # an empty first window leaves only the second stack to decode
    wg, wd = run_decode_rows(g, dev, (5, 5), es=es, second=d, rows_second=(100, 900))
    assert np.all(wg == POISON)
    assert_bytes_equal(wd, oracle_rows(orc, sd, (100, 900), es), "down rows 100..899")


def test_short_stack_tensors_refused_before_launch(dev):
    """A stack tensor shorter than the layout addresses is refused by the
    binding before any kernel is enqueued: the workspace keeps its poison."""
    st = mwd.prepare(workloads.TINY.generate(), workloads.NVFP4).to(dev)
    bad = st.clone()
    bad.offsets = bad.offsets[: st.E * st.stride - 16]
    ws = torch.full((st.dense_bytes,), POISON, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="offsets"):
        mwd.decode(bad, ws)
    with pytest.raises(ValueError, match="offsets"):
        mwd.Launch(bad, ws)
    with pytest.raises(ValueError, match="offsets"):
        mwd.build_index(bad)
    K = st.C * 16
    es = torch.tensor([0, 1, 1, 2, 2], dtype=torch.int32, device=dev)
    with pytest.raises(ValueError, match="offsets"):
        mwd.moe_w4a16(bad, torch.zeros(st.E * st.R * K // 2, dtype=torch.uint8, device=dev),
                      torch.zeros(2, K, dtype=torch.bfloat16, device=dev),
                      torch.ones(st.E, dtype=torch.float32, device=dev), es)
    torch.cuda.synchronize(dev)
    assert bool((ws == POISON).all())
    mwd.decode(st, ws)
    assert torch.equal(ws.cpu(), torch.from_numpy(workloads.TINY.generate().reshape(-1)))


# -- seeded random combinations -------------------------------------------------

def _random_case(rng, seed):
    E = int(rng.choice([1, 2, 3, 4, 5, 8, 31, 64, 100, 257, 511, 512, 513, 600]))
    fmt = int(rng.integers(0, 2))

    def shape():
        C = int(rng.choice([1, 2, 3, 7, 8, 15, 16, 17, 31, 32, 33, 50, 64, 100, 128, 129, 160, 200, 255, 256, 300]))
        return int(rng.integers(1, max(1, min(3000, 2_000_000 // (E * C))) + 1)), C

    def stack(f, R, C, s):
        k = rng.integers(0, 3)
        if k == 0:
            return workloads.uniform_bytes(E, R, C, s)
        if f == workloads.NVFP4:
            return workloads.nvfp4_stack(E, R, C, s, float(rng.uniform(0, 0.3)),
                                         hot_row_frac=float(rng.choice([0.0, 0.02])))
        return workloads.mxfp4_stack(E, R, C, s, float(rng.uniform(0, 0.3)))

    R, C = shape()
    return E, fmt, R, C, stack(fmt, R, C, seed), shape, stack


@pytest.mark.parametrize("block", range(4))
def test_random_feature_combinations(orc, dev, block):
    """60 seeded cases per block, each drawing a stack (uniform bytes or a
    generated distribution, either format, 1 to 600 experts, rows of 1 to 300
    columns) and a combination of: fused or two-pass decode, routing (active
    subsets, garbage values, int32 or int64, off a 16-byte boundary), a second
    stack of other shape and format in the same launch, row windows, workspace
    byte offsets, and a GPU encode of the same bytes off a 16-byte boundary.
    Every result is compared with the oracle, workspace guard bands included."""
    for i in range(60):
        seed = 7000 + 60 * block + i
        rng = np.random.default_rng(seed)
        E, fmt, R, C, x, shape, stack = _random_case(rng, 9000 + seed)
        st = orc.encode(fmt, x)
        mode = str(rng.choice(MODES))
        es = None
        if rng.random() < 0.6:
            if rng.random() < 0.1:
                es = rng.integers(-5, 50, E + 1).astype(np.int32)
            else:
                act = np.zeros(E, bool)
                act[rng.choice(E, int(rng.integers(0, min(E, 40) + 1)), replace=False)] = True
                es = workloads.expert_start_from_mask(act, tokens=int(rng.integers(1, 5)))
        paired = rng.random() < 0.4
        window = rng.random() < 0.3
        off = int(rng.choice([0, 0, 1, 7, 13]))
        wide = es is not None and not window and rng.random() < 0.3
        shift = int(rng.choice([0, 0, 1]))
        print(f"[parity] random case {seed}: fmt {fmt} E {E} R {R} C {C} {mode} routed {es is not None} "
              f"wide {wide} shift {shift} paired {paired} window {window} offset {off}", flush=True)
        stacks = [(st, upload(st, dev, mode), (E, R, C))]
        if paired:
            f2 = int(rng.integers(0, 2))
            R2, C2 = shape()
            st2 = orc.encode(f2, stack(f2, R2, C2, 19000 + seed))
            stacks.append((st2, upload(st2, dev, mode), (E, R2, C2)))
        es_t = None
        if es is not None:
            dt = torch.int64 if wide else torch.int32
            es_t = torch.zeros(E + 5, dtype=dt, device=dev)[shift: shift + E + 1]
            es_t.copy_(torch.from_numpy(es.astype(np.int64)).to(dev))
        bufs, wss, wants, rows = [], [], [], []
        for s_np, s_gpu, shp in stacks:
            n = s_gpu.dense_bytes
            buf = torch.full((GUARD_BYTES + off + n + GUARD_BYTES,), GUARD, dtype=torch.uint8, device=dev)
            ws = buf[GUARD_BYTES + off: GUARD_BYTES + off + n]
            ws.fill_(POISON)
            fill = np.full(shp, POISON, np.uint8)
            if window:
                b = int(rng.integers(0, shp[1] + 1))
                e = int(rng.integers(b, shp[1] + 1))
                rows.append((b, e))
                wants.append(orc.decode_rows(s_np, b, e, es, fill))
            else:
                wants.append(orc.decode(s_np, es, fill))
            bufs.append(buf)
            wss.append(ws)
        if window:
            second = (stacks[1][1], wss[1], rows[1]) if paired else (None, None, None)
            mwd.decode_rows(stacks[0][1], wss[0], rows[0], *second, es_t)
        elif paired:
            mwd.decode_paired(stacks[0][1], wss[0], stacks[1][1], wss[1], es_t)
        else:
            mwd.decode(stacks[0][1], wss[0], es_t)
        torch.cuda.synchronize()
        for (s_np, s_gpu, shp), buf, want in zip(stacks, bufs, wants):
            h = buf.cpu().numpy()
            n = s_gpu.dense_bytes
            assert np.all(h[:GUARD_BYTES + off] == GUARD), f"case {seed}: write before the workspace"
            assert np.all(h[GUARD_BYTES + off + n:] == GUARD), f"case {seed}: write past the workspace"
            assert_bytes_equal(h[GUARD_BYTES + off: GUARD_BYTES + off + n].reshape(shp), want, f"case {seed}")
        if rng.random() < 0.3:
            sh = int(rng.choice([0, 1, 4]))
            xd = torch.empty(x.size + 16, dtype=torch.uint8, device=dev)[sh: sh + x.size].view(E, R, C)
            xd.copy_(torch.from_numpy(x).to(dev))
            _same_streams(mwd.prepare(xd, fmt).numpy(), st, f"case {seed} GPU encode")


def test_gpu_encoder_random_value_patterns(orc, dev):
    """150 seeded stacks whose values stress the base search: a few values
    anywhere, most values in the top 16 bytes with the rest just above 0 (a
    base above 256 - W, and bytes within W of it modulo 256), two equal
    clusters (ties), uniform bytes, and constant planes with a few stray
    bytes; rows of 1 to 400 columns, both formats, dense bytes 0 to 8 bytes
    past a 16-byte boundary.  The GPU encoder's streams equal the oracle's."""
    for i in range(150):
        seed = 500000 + i
        rng = np.random.default_rng(seed)
        E = int(rng.choice([1, 2, 3, 7, 64, 300]))
        C = int(rng.choice([1, 2, 3, 4, 5, 15, 16, 17, 31, 32, 33, 48, 50, 64, 100, 128, 160, 200, 254, 255, 256,
                            257, 400]))
        R = int(rng.integers(1, max(1, min(500, 1_000_000 // (E * C))) + 1))
        kind = int(rng.integers(0, 5))
        shp = (E, R, C)
        if kind == 0:
            x = rng.choice(rng.integers(0, 256, int(rng.integers(1, 6))), shp).astype(np.uint8)
        elif kind == 1:
            x = np.where(rng.random(shp) < 0.8, rng.integers(240, 256, shp), rng.integers(0, 20, shp)).astype(np.uint8)
        elif kind == 2:
            a, b = rng.integers(0, 256, 2)
            x = np.clip(np.where(rng.random(shp) < 0.5, a + rng.integers(0, 2, shp), b + rng.integers(0, 2, shp)),
                        0, 255).astype(np.uint8)
        elif kind == 3:
            x = workloads.uniform_bytes(E, R, C, seed)
        else:
            x = np.full(shp, int(rng.integers(0, 256)), np.uint8)
            k = max(1, x.size // 50)
            x.reshape(-1)[rng.integers(0, x.size, k)] = rng.integers(0, 256, k)
        fmt = int(rng.integers(0, 2))
        sh = int(rng.choice([0, 0, 1, 3, 8]))
        print(f"[parity] encoder pattern {kind} case {seed}: fmt {fmt} {shp} shift {sh}", flush=True)
        xd = torch.empty(x.size + 16, dtype=torch.uint8, device=dev)[sh: sh + x.size].view(*shp)
        xd.copy_(torch.from_numpy(x).to(dev))
        _same_streams(mwd.prepare(xd, fmt).numpy(), orc.encode(fmt, x), f"encoder case {seed}")
