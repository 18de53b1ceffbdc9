"""GPU parity of the W4A16 consumer (csf_moe_w4a16) against its oracle.

The kernel reads the block scales (E4M3 per 16 weights for NVFP4, UE8M0 per 32
for MXFP4) either straight from the CSF streams (expanded into LDS per unit of
32 rows) or from a dense scale workspace; both must
give the same float32 outputs bit for bit, and both must match the float64
oracle within the fp32 accumulation bound

    |y - y_ref| <= (K + 8) * 2^-24 * |alpha| * sum_k |x_k w_k|

(every product x*w is exact in fp32; each of the at most K + 8 roundings of
the sums and of the alpha scaling adds at most 2^-24 of the running magnitude).
A wrong operand layout or a wrong scale gives errors of the order of the
outputs themselves."""
import numpy as np
import pytest
import torch

import workloads
from oracle import w4a16 as ref

mwd = pytest.importorskip("moe_weight_decode_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


FMT_NAME = {workloads.NVFP4: "nvfp4", workloads.MXFP4: "mxfp4"}


def run(orc, dev, inp: workloads.W4A16Inputs, dense: bool, dense_offset: int = 0):
    st = orc.encode(inp.fmt, inp.scales)
    stack = mwd.from_numpy(st, dev)
    w = torch.from_numpy(inp.w_packed).to(dev)
    x = torch.from_numpy(inp.x_bits.view(np.int16)).to(dev)
    alpha = torch.from_numpy(inp.alpha).to(dev)
    es = torch.from_numpy(inp.expert_start).to(dev)
    out = torch.full((x.shape[0], inp.w_packed.shape[1]), float("nan"), dtype=torch.float32, device=dev)
    dense_t = None
    if dense:
        buf = torch.full((stack.dense_bytes + dense_offset,), 0xA5, dtype=torch.uint8, device=dev)
        dense_t = buf[dense_offset:]
        mwd.decode(stack, dense_t, es)
    mwd.moe_w4a16(stack, w, x, alpha, es, out=out, dense_scales=dense_t)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(inp, got, what):
    K = inp.x_bits.shape[1]
    y, mag = ref.moe_w4a16(inp.x_bits, inp.w_packed, inp.scales, inp.alpha, inp.expert_start,
                           fmt=FMT_NAME[inp.fmt])
    tol = (K + 8) * 2.0 ** -24 * mag
    err = np.abs(got.astype(np.float64) - y)
    bad = ~(err <= tol)
    if bad.any():
        t, n = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} outputs outside the bound; first token {t} row {n}: "
                             f"gpu {got[t, n]!r} oracle {y[t, n]!r} bound {tol[t, n]!r}")
    return y


@pytest.mark.parametrize("E,N,K,counts", [
    (4, 48, 256, [0, 1, 17, 70]),
    (3, 40, 96, [5, 0, 64]),
    (2, 16, 2048, [3, 33]),
    (5, 7, 32, [1, 2, 0, 16, 15]),
    (3, 70, 160, [40, 1, 7]),
    (2, 40, 2080, [17, 5]),
    (2, 33, 4096, [1, 50]),
    (2, 48, 7168, [70, 3]),
    (2, 40, 8192, [33, 20]),
], ids=["mixed_counts", "ragged_rows", "k2048", "tiny", "k160_rows70", "k2080", "k4096", "k7168_two_passes",
        "k8192_max"])
def test_small_shapes(orc, dev, E, N, K, counts):
    es = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    inp = workloads.w4a16_inputs(E, N, K, es, seed=E * 100 + N, exc_rate=0.08)
    got_csf = run(orc, dev, inp, dense=False)
    got_dense = run(orc, dev, inp, dense=True)
    check(inp, got_csf, "scales from CSF")
    assert np.array_equal(got_csf, got_dense)


@pytest.mark.parametrize("name,N,K", [("gate", 800, 2048), ("down", 2048, 800)])
def test_routed_full_shapes(orc, dev, name, N, K):
    # 8 of 512 experts routed with 1..64 tokens each (the routed workload)
    es = workloads.ROUTED.expert_start()
    inp = workloads.w4a16_inputs(512, N, K, es, seed=7 if name == "gate" else 8,
                                 exc_rate=0.03 if name == "gate" else 0.10)
    got_csf = run(orc, dev, inp, dense=False)
    got_dense = run(orc, dev, inp, dense=True)
    check(inp, got_csf, f"{name} scales from CSF")
    assert np.array_equal(got_csf, got_dense)


def test_unit_weights_give_activation_sums(orc, dev):
    # every code 1.0 and every scale 1.0 (0x38): y = alpha * sum_k x
    es = np.array([0, 9, 9, 40], dtype=np.int32)
    inp = workloads.w4a16_inputs(3, 32, 512, es, seed=3)
    inp.w_packed[:] = 0x22
    inp.scales[:] = 0x38
    got = run(orc, dev, inp, dense=False)
    check(inp, got, "unit weights")


def _routing(counts, T):
    es = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    assert es[-1] <= T
    return es


def test_graph_replay_follows_routing_and_activations(orc, dev):
    """One captured call replayed with three routings and fresh activations:
    the library allocates nothing during capture, every replay equals an
    eager call bit for bit and the oracle within the bound, and the outputs
    of tokens a routing leaves out stay untouched."""
    E, N, K, T = 24, 80, 512, 160
    routings = [_routing([0, 9, 0, 33, 1, 0, 64, 5] + [0] * 16, T),      # 112 of 160 tokens routed
                _routing([0] * 10 + [150] + [0] * 13, T),                 # one expert, several passes
                _routing([T // E + (i < T % E) for i in range(E)], T)]    # every expert, every token
    inp = workloads.w4a16_inputs(E, N, K, routings[0], seed=91, exc_rate=0.08)
    stack = mwd.from_numpy(orc.encode(workloads.NVFP4, inp.scales), dev)
    w = torch.from_numpy(inp.w_packed).to(dev)
    alpha = torch.from_numpy(inp.alpha).to(dev)
    x = torch.zeros((T, K), dtype=torch.int16, device=dev)
    y = torch.empty((T, N), dtype=torch.float32, device=dev)
    es_t = torch.zeros(E + 1, dtype=torch.int32, device=dev)
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):  # warm the launch path outside capture
        mwd.moe_w4a16(stack, w, x, alpha, es_t, out=y)
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        allocated, reserved = torch.cuda.memory_allocated(dev), torch.cuda.memory_reserved(dev)
        mwd.moe_w4a16(stack, w, x, alpha, es_t, out=y)
        assert torch.cuda.memory_allocated(dev) == allocated
        assert torch.cuda.memory_reserved(dev) == reserved
    rng = np.random.default_rng(92)
    for rnd in range(2):
        for i, es in enumerate(routings):
            xb = workloads.bf16_bits(T, K, rng)
            x.copy_(torch.from_numpy(xb.view(np.int16)))
            es_t.copy_(torch.from_numpy(es))
            y.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = y.cpu().numpy()
            eager = mwd.moe_w4a16(stack, w, x, alpha, es_t).cpu().numpy()
            routed = int(es[-1])
            assert np.array_equal(got[:routed], eager[:routed]), f"replay {rnd}/{i} differs from an eager call"
            assert np.isnan(got[routed:]).all(), f"replay {rnd}/{i} wrote outputs of unrouted tokens"
            if rnd == 0:
                ref, mag = ref_moe(xb, inp, es)
                err = np.abs(got[:routed].astype(np.float64) - ref[:routed])
                assert np.all(err <= (K + 8) * 2.0 ** -24 * mag[:routed]), f"replay {i} outside the bound"


def ref_moe(x_bits, inp, es):
    return ref.moe_w4a16(x_bits, inp.w_packed, inp.scales, inp.alpha, es)


def test_side_stream_ordering(orc, dev):
    es = _routing([3, 0, 40, 17], 60)
    inp = workloads.w4a16_inputs(4, 48, 256, es, seed=93)
    stack = mwd.from_numpy(orc.encode(workloads.NVFP4, inp.scales), dev)
    w = torch.from_numpy(inp.w_packed).to(dev)
    x = torch.from_numpy(inp.x_bits.view(np.int16)).to(dev)
    alpha = torch.from_numpy(inp.alpha).to(dev)
    es_t = torch.from_numpy(inp.expert_start).to(dev)
    y = torch.full((60, 48), float("nan"), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        mwd.moe_w4a16(stack, w, x, alpha, es_t, out=y)  # the current stream is the side stream
        done = torch.cuda.Event()
        done.record(side)
    torch.cuda.current_stream(dev).wait_event(done)
    check(inp, y.cpu().numpy(), "side stream")


def check_non_finite(inp, got, what):
    """Like check(), where the oracle's output is NaN or infinite: the GPU
    output must be NaN at exactly the same places and the same infinity
    elsewhere; finite outputs keep the float32 bound."""
    K = inp.x_bits.shape[1]
    with np.errstate(invalid="ignore"):  # inf * 0 in the oracle is meant to give NaN
        y, mag = ref.moe_w4a16(inp.x_bits, inp.w_packed, inp.scales, inp.alpha, inp.expert_start,
                               fmt=FMT_NAME[inp.fmt])
    got = got.astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(y)), f"{what}: NaN pattern differs"
    inf = np.isinf(y)
    assert np.array_equal(got[inf], y[inf]), f"{what}: infinities differ"
    fin = np.isfinite(y)
    assert np.isfinite(got[fin]).all(), f"{what}: non-finite output where the oracle's is finite"
    assert np.all(np.abs(got[fin] - y[fin]) <= (K + 8) * 2.0 ** -24 * mag[fin]), f"{what}: outside the bound"
    return y


@pytest.mark.parametrize("K", [160, 2048, 4096])
def test_non_finite_values_stay_in_their_outputs(orc, dev, K):
    """A NaN scale byte (E4M3 S.1111.111) makes exactly its row's outputs NaN
    for the expert's tokens; an infinite or NaN activation reaches only its own
    token's outputs (K = 160 leaves part of a chunk past K: no lane may read
    the next token's row there; K = 4096 runs the K-tile path, which keeps its
    scales as float16 patterns)."""
    es = _routing([5, 6], 11)
    inp = workloads.w4a16_inputs(2, 40, K, es, seed=94 + K, exc_rate=0.05)
    inp.scales[1, 33, 3] = 0x7F                          # expert 1 (tokens 5..10), row 33
    inp.x_bits[2, K - 1] = 0x7F80                        # +inf, last k of token 2
    inp.x_bits[3, 0] = 0x7FC0                            # NaN, first k of token 3
    inp.x_bits[8, K // 2] = 0xFF80                       # -inf, token 8 (expert 1)
    for dense in (False, True):
        got = run(orc, dev, inp, dense=dense)
        y = check_non_finite(inp, got, f"non-finite inputs, {'dense' if dense else 'CSF'} scales")
    assert np.isnan(y[5:11, 33]).all() and np.isfinite(y[[0, 1, 4]]).all()


# -- MXFP4: UE8M0 scale per 32 weights, 1-bit CSF offsets ----------------------

@pytest.mark.parametrize("E,N,K,counts", [
    (3, 40, 96, [5, 0, 64]),
    (5, 7, 32, [1, 2, 0, 16, 15]),
    (3, 70, 160, [40, 1, 7]),
    (2, 16, 2048, [3, 33]),
    (2, 40, 2080, [17, 5]),
    (2, 33, 5120, [1, 50]),
    (2, 48, 8192, [70, 3]),
], ids=["k96", "tiny", "k160_rows70", "k2048", "k2080", "k5120", "k8192_two_passes"])
def test_mxfp4_small_shapes(orc, dev, E, N, K, counts):
    es = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    inp = workloads.w4a16_inputs(E, N, K, es, seed=E * 100 + N + 1, exc_rate=0.15, fmt=workloads.MXFP4)
    got_csf = run(orc, dev, inp, dense=False)
    got_dense = run(orc, dev, inp, dense=True)
    check(inp, got_csf, "MXFP4 scales from CSF")
    assert np.array_equal(got_csf, got_dense)


@pytest.mark.parametrize("fmt,K,offset", [
    (workloads.MXFP4, 160, 1), (workloads.MXFP4, 5120, 3),
    (workloads.NVFP4, 256, 2), (workloads.NVFP4, 4096, 6),
], ids=["mx_k160_odd", "mx_k5120_odd", "nv_k256_2", "nv_k4096_6"])
def test_dense_scales_at_unaligned_addresses(orc, dev, fmt, K, offset):
    """Dense scales need no alignment for MXFP4 (byte loads) and two bytes for
    NVFP4 (16-bit loads): a workspace starting at such an address gives the
    same outputs as the scales expanded from the CSF streams."""
    es = np.array([0, 19, 19, 60], dtype=np.int32)
    inp = workloads.w4a16_inputs(3, 45, K, es, seed=K + offset, exc_rate=0.15 if fmt else 0.03, fmt=fmt)
    got_csf = run(orc, dev, inp, dense=False)
    got_dense = run(orc, dev, inp, dense=True, dense_offset=offset)
    check(inp, got_csf, "scales from CSF")
    assert np.array_equal(got_csf, got_dense)


def test_mxfp4_routed_full_shape(orc, dev):
    # the MXFP4 stack's shape (384 experts x 1024 rows, K = 5120), 8 experts routed
    es = workloads.routing(384, 8, 64, 4)
    inp = workloads.w4a16_inputs(384, 1024, 5120, es, seed=4, exc_rate=0.15, fmt=workloads.MXFP4)
    got_csf = run(orc, dev, inp, dense=False)
    got_dense = run(orc, dev, inp, dense=True)
    check(inp, got_csf, "MXFP4 routed scales from CSF")
    assert np.array_equal(got_csf, got_dense)


@pytest.mark.parametrize("K", [160, 5120])
def test_mxfp4_scale_extremes_and_nan(orc, dev, K):
    """UE8M0 bytes far from 127 scale by their exponent alone (rows whose
    blocks carry 20 and 230, products still inside float32's normal range,
    stay within the bound), and byte 255 (NaN) makes
    exactly its row's outputs NaN for the expert's tokens (K = 5120: the
    K-tile path)."""
    es = _routing([6, 5], 11)
    inp = workloads.w4a16_inputs(2, 40, K, es, seed=95, exc_rate=0.05, fmt=workloads.MXFP4)
    inp.scales[0, 3, :] = 20
    inp.scales[0, 4, 1] = 230
    inp.scales[1, 9, :5] = np.array([20, 230, 127, 100, 200], dtype=np.uint8)
    inp.scales[1, 21, 4] = 0xFF
    inp.scales[1, 22, K // 32 - 1] = 0xFF                # the last scale column (last K-tile)
    for dense in (False, True):
        got = run(orc, dev, inp, dense=dense)
        y = check_non_finite(inp, got, f"MXFP4 extremes, {'dense' if dense else 'CSF'} scales")
    assert np.isnan(y[6:11, 21:23]).all() and np.isfinite(y[:6]).all()


@pytest.mark.parametrize("fmt,K", [(workloads.NVFP4, 256), (workloads.MXFP4, 5120)])
def test_no_routed_tokens_writes_nothing(orc, dev, fmt, K):
    """expert_start with no expert holding a token (all equal), and one whose
    ranges all lie past num_tokens: the call writes no output."""
    E, N, T = 5, 48, 12
    inp = workloads.w4a16_inputs(E, N, K, _routing([3, 0, 9, 0, 0], T), seed=96, fmt=fmt)
    stack = mwd.from_numpy(orc.encode(fmt, inp.scales), dev)
    w = torch.from_numpy(inp.w_packed).to(dev)
    x = torch.from_numpy(inp.x_bits.view(np.int16)).to(dev)
    alpha = torch.from_numpy(inp.alpha).to(dev)
    for es in (np.full(E + 1, 7, dtype=np.int32),                      # no expert has tokens
               np.array([T, T, T + 5, T + 9, T + 9, T + 9], dtype=np.int32)):  # all past num_tokens
        y = torch.full((T, N), float("nan"), dtype=torch.float32, device=dev)
        mwd.moe_w4a16(stack, w, x, alpha, torch.from_numpy(es).to(dev), out=y)
        torch.cuda.synchronize()
        assert torch.isnan(y).all()


def test_ahead_of_call_expansion_on_a_side_stream(orc, dev):
    """The pages' ahead-of-call flow: the routed experts' scales are expanded
    into a dense workspace on a side stream, and the projection on the main
    stream waits for that stream's event before reading them.  Equal, bit for
    bit, to the projection that expands its scales in LDS."""
    es = _routing([0, 21, 0, 40, 3, 0], 64)
    inp = workloads.w4a16_inputs(6, 72, 1024, es, seed=97, exc_rate=0.06)
    stack = mwd.from_numpy(orc.encode(workloads.NVFP4, inp.scales), dev)
    w = torch.from_numpy(inp.w_packed).to(dev)
    x = torch.from_numpy(inp.x_bits.view(np.int16)).to(dev)
    alpha = torch.from_numpy(inp.alpha).to(dev)
    es_t = torch.from_numpy(es).to(dev)
    stage = mwd.moe_w4a16(stack, w, x, alpha, es_t)
    ws = torch.full((stack.dense_bytes,), 0xA5, dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        mwd.decode(stack, ws, es_t)
        expanded = torch.cuda.Event()
        expanded.record(side)
    torch.cuda.current_stream(dev).wait_event(expanded)
    y = mwd.moe_w4a16(stack, w, x, alpha, es_t, dense_scales=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, stage)
    check(inp, y.cpu().numpy(), "ahead-of-call expansion")


def test_no_routed_tokens(orc, dev):
    """A routing with no tokens at all: an empty output, nothing launched,
    for both scale sources and formats."""
    for fmt in (workloads.NVFP4, workloads.MXFP4):
        inp = workloads.w4a16_inputs(3, 40, 256, np.zeros(4, dtype=np.int32), seed=5, fmt=fmt)
        for dense in (False, True):
            got = run(orc, dev, inp, dense=dense)
            assert got.shape == (0, 40)
