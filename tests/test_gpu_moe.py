"""GPU parity of the W4A16 consumer (csf_moe_w4a16) against its oracle.

The kernel reads the E4M3 scales either straight from the CSF streams
(expanded into LDS per 16-row unit) or from a dense scale workspace; both must
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


def run(orc, dev, inp: workloads.W4A16Inputs, dense: bool):
    st = orc.encode(workloads.NVFP4, inp.scales)
    stack = mwd.from_numpy(st, dev)
    w = torch.from_numpy(inp.w_packed).to(dev)
    x = torch.from_numpy(inp.x_bits.view(np.int16)).to(dev)
    alpha = torch.from_numpy(inp.alpha).to(dev)
    es = torch.from_numpy(inp.expert_start).to(dev)
    out = torch.full((x.shape[0], inp.w_packed.shape[1]), float("nan"), dtype=torch.float32, device=dev)
    dense_t = None
    if dense:
        dense_t = torch.full((stack.dense_bytes,), 0xA5, dtype=torch.uint8, device=dev)
        mwd.decode(stack, dense_t, es)
    mwd.moe_w4a16(stack, w, x, alpha, es, out=out, dense_scales=dense_t)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(inp, got, what):
    K = inp.x_bits.shape[1]
    y, mag = ref.moe_w4a16(inp.x_bits, inp.w_packed, inp.scales, inp.alpha, inp.expert_start)
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
], ids=["mixed_counts", "ragged_rows", "k2048", "tiny", "k160_rows70"])
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
