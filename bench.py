"""Benchmark of the CSF block-scale decoder on one MI355X.

One step = one full decode of the 512-expert gate-like NVFP4 stack (512 x 800
x 128 E4M3 scale bytes, 3 % outliers, with its tile index) into its dense
workspace: a single launch of the fused kernel (fixed stream + exceptions
patched on chip).  Steps rotate over several device copies of the compressed
stack and workspace (together larger than the 256 MB Infinity Cache), so
every step reads and writes HBM.

Prints ONE JSON line on stdout:
  value       whole-run throughput, GB/s = (compressed bytes read + dense
              bytes written) per step x steps / elapsed time
  roofline    the fused kernel (the only kernel of a step): its algorithmic
              bytes per launch / its mean launch time, from two HIP events on
              its stream bracketing the back-to-back launches of the timed
              region (no event sits between two launches), against the MI355X
              HBM3E peak (8 TB/s)
  cpu_baseline the CPU oracle decoding the same stack on one host core

  python bench.py [--steps K] [--warmup W] [--sets N] [--workload NAME] [--all] [--no-cpu]

--workload picks another timed workload (down_nvfp4, mxfp4, tiny_nvfp4,
routed_paired, routed_moe, routed_moe_mx) for profiling; the default is the
gate-like stack.  routed_moe times the W4A16 consumer that expands its scales
in LDS from the CSF streams (csf_moe_w4a16) on the gate-like projection with 8
of 512 experts routed, next to a routed decode followed by the same GEMM on
dense scales; routed_moe_mx does the same on the MXFP4 stack's projection
(384 x 1024, K = 5120, 8 of 384 experts routed).

--all also measures the other workloads (down-like, MXFP4, routed paired,
tiny), the two-pass decode of each (fixed-stream kernel, then exception
kernel), warm and cache-flushed single calls, the floor of two dependent tiny
launches, and a plain copy; one line each on stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "CSF decode GB/s (compressed read + dense write) and µs per 512-expert stack"
MOE_METRIC = ("routed W4A16 MoE projection with stage-local CSF scale decode: algorithmic GB/s (weights, "
              "compressed scales, activations read; outputs written) and µs per call")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t timing through the HIP runtime torch already loaded."""

    def __init__(self):
        path = None
        for line in open("/proc/self/maps"):
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
        self.hip = ctypes.CDLL(path or "libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.record = self.hip.hipEventRecord

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), 0) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            evs.append(e.value)
        return evs

    def ms(self, a, b) -> float:
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def stack_bytes(stack, active=None):
    """Algorithmic bytes of one decode: (fixed-stream bytes read, exception
    bytes read, dense bytes written).  Exception bytes include the prefix and,
    for an indexed stack, the tile index (a routed decode reads only the
    index segments of its routed experts).  active: boolean mask of routed
    experts, or None for all."""
    import numpy as np
    E = stack.E
    n_act = E if active is None else int(np.count_nonzero(active))
    prefix = stack.prefix.cpu().numpy()
    if active is None:
        entries = stack.num_exceptions
    else:
        entries = int(np.diff(prefix)[np.asarray(active, dtype=bool)].sum())
    fixed = n_act * (stack.R + stack.stride)          # bases + offsets
    exc = 4 * entries + 4 * (E + 1)                   # entries + prefix
    if stack.tile_index is not None:
        exc += 4 * (E * stack.index_tiles + 1) if active is None else 4 * n_act * (stack.index_tiles + 1)
    dense = n_act * stack.P
    return fixed, exc, dense


_KERNEL_SOURCES = {
    "csf_fused_kernel": ("csf_kernels.hip",),
    "csf_moe_w4a16_kernel": ("csf_moe.hip",),
}


def source_hash(kernel: str = "csf_fused_kernel", csrc: str | None = None) -> str:
    """Fingerprint of the code a kernel is built and launched from (its own
    source plus the shared device helpers, launch structs and host planner):
    comments and whitespace are dropped, so only a change to the code itself
    invalidates that kernel's counter records."""
    import re
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "moe_weight_decode_amd", "csrc")
    for name in _KERNEL_SOURCES[kernel] + ("csf_launch.h", "csf_api.cpp", "csf_device.h"):
        text = open(os.path.join(csrc, name)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def pmc_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    data = json.load(open(path))
    rec = data.get(f"{kernel}/{workload}")
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def make_sets(mwd, torch, stack, nsets, dev):
    sets = []
    for i in range(nsets):
        s = stack if i == 0 else stack.clone()
        ws = torch.empty(stack.dense_bytes, dtype=torch.uint8, device=dev)
        sets.append((s, ws))
    return sets


def timed_loop(torch, ev, calls, steps, warmup):
    """Run `steps` calls (after `warmup`), rotating over `calls`, with one HIP
    event before and one after the whole run on the launch stream.  Returns
    (wall-clock ms per step, event ms per step)."""
    stream = calls[0].stream
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    evs = ev.create(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(evs[0], stream)
    n = len(calls)
    for i in range(steps):
        calls[i % n]()
    ev.record(evs[1], stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    total_ms = ev.ms(evs[0], evs[1])
    ev.destroy(evs)
    return wall_ms / steps, total_ms / steps


def flushed_call_ms(torch, ev, launch, dev, reps=30, flush_bytes=1 << 30):
    """Latency of one call on cold caches: a 1 GiB buffer (more than the MALL
    and every L2 together) is written on the call's stream before each call,
    and one event pair brackets the call alone.  Median over `reps` calls."""
    if torch.cuda.current_stream(dev).cuda_stream != launch.stream:
        raise RuntimeError("flushed_call_ms: the call must run on the current stream")
    buf = torch.empty(flush_bytes, dtype=torch.uint8, device=dev)
    evs = ev.create(2 * reps)
    for i in range(reps):
        buf.fill_(i & 0xFF)
        ev.record(evs[2 * i], launch.stream)
        launch()
        ev.record(evs[2 * i + 1], launch.stream)
    torch.cuda.synchronize()
    t = [ev.ms(evs[2 * i], evs[2 * i + 1]) for i in range(reps)]
    ev.destroy(evs)
    del buf
    return statistics.median(t)


class Passes:
    """A Launch restricted to some passes (for the two-pass split)."""

    def __init__(self, launch, passes):
        self.launch, self.passes, self.stream = launch, passes, launch.stream

    def __call__(self):
        self.launch(self.passes)


def check_equal(torch, ws, x, what):
    import numpy as np
    got = ws.cpu().numpy().reshape(x.shape)
    if not np.array_equal(got, x):
        raise SystemExit(f"{what}: GPU decode differs from the input in {(got != x).sum()} bytes")


def bench_stack(mwd, torch, ev, spec, steps, warmup, nsets, dev, split=False):
    """Time the full decode of `spec` (fused, indexed stack); with `split`
    also the two-pass decode of the same stack and its fixed pass alone, one
    stack decoded over and over (warm: its 85-109 MB stay in the MALL), and
    single calls on flushed caches."""
    x = spec.generate()
    stack = mwd.prepare(x, spec.fmt).to(dev)
    sets = make_sets(mwd, torch, stack, nsets, dev)
    launches = [mwd.Launch(s, ws) for s, ws in sets]
    launches[0]()
    torch.cuda.synchronize()
    check_equal(torch, sets[0][1], x, spec.name)
    wall, evt = timed_loop(torch, ev, launches, steps, warmup)
    fb, eb, db = stack_bytes(stack)
    out = dict(x=x, stack=stack, fixed_bytes=fb, exc_bytes=eb, dense_bytes=db,
               step_ms=max(wall, evt), wall_ms=wall, event_ms=evt)
    if split:
        two = [mwd.Launch(s.without_index(), ws) for s, ws in sets]
        two[0]()
        torch.cuda.synchronize()
        check_equal(torch, sets[0][1], x, spec.name + " two-pass")
        w2, e2 = timed_loop(torch, ev, two, steps, warmup)
        wf, ef = timed_loop(torch, ev, [Passes(L, mwd.PASS_FIXED) for L in two], steps, warmup)
        ww, we = timed_loop(torch, ev, [launches[0]], steps, warmup)
        out.update(two_pass_ms=max(w2, e2), fixed_only_ms=max(wf, ef), warm_ms=max(ww, we),
                   flushed_ms=flushed_call_ms(torch, ev, launches[0], dev))
    return out


def _repeat(fn, budget_s):
    times = []
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or len(times) < 3:
        t = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t)
    return statistics.median(times), len(times)


def cpu_baseline(spec, x, budget_s=10.0):
    """The oracle (plain C, one thread) decoding the whole stack, repeated for
    about `budget_s` seconds; GB/s on the same byte formula as the GPU."""
    import oracle
    orc = oracle.load()
    st = orc.encode(spec.fmt, x)
    ws = orc.decode(st)
    if not (ws == x).all():
        raise SystemExit("oracle round trip failed")
    sec, n = _repeat(lambda: orc.decode(st, None, ws), budget_s)
    E = spec.E
    comp = E * spec.R + E * st["stride"] + 4 * st["exceptions"].size + 4 * (E + 1)
    return dict(value=round((comp + x.size) / sec / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                us_per_stack=round(sec * 1e6, 1),
                sample=f"whole {spec.name} stack ({spec.E}x{spec.R}x{spec.C}), decoded {n} "
                       f"times on one host core, median")


def cpu_baseline_routed(workloads, budget_s=10.0):
    """The oracle's routed decode of the gate and down stacks (8 of 512
    experts), one host core; GB/s on the GPU's byte formula."""
    import numpy as np
    import oracle
    orc = oracle.load()
    gspec, dspec = workloads.ROUTED.stacks
    es = workloads.ROUTED.expert_start()
    act = np.diff(es) > 0
    sts, wss, nbytes = [], [], 4 * len(es)
    for spec in (gspec, dspec):
        x = spec.generate()
        st = orc.encode(spec.fmt, x)
        sts.append(st)
        wss.append(np.zeros(x.shape, dtype=np.uint8))
        ent = int(np.diff(st["prefix"])[act].sum())
        nbytes += int(act.sum()) * (spec.R + st["stride"] + spec.R * spec.C) + 4 * ent + 4 * (spec.E + 1)
    sec, n = _repeat(lambda: [orc.decode(st, es, ws) for st, ws in zip(sts, wss)], budget_s)
    return dict(value=round(nbytes / sec / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                us_per_stack=round(sec * 1e6, 1),
                sample=f"routed paired decode (8 of 512 experts) of the gate and down stacks, "
                       f"{n} times on one host core, median")


def routed_sets(workloads, E, n_active, max_tokens, seed, count):
    """`count` routings whose active experts are disjoint groups of a seeded
    permutation (each expert routed in turn), U{1..max_tokens} tokens each."""
    import numpy as np
    rng = np.random.default_rng(seed)
    perm = rng.permutation(E)
    out = []
    for i in range(count):
        act = perm[(i * n_active) % E:(i * n_active) % E + n_active]
        counts = np.zeros(E, dtype=np.int64)
        counts[act] = rng.integers(1, max_tokens, n_active, endpoint=True)
        out.append(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
    return out


def bench_routed(mwd, torch, ev, workloads, steps, warmup, dev, indexed=True, copies=2, routings=64,
                 gate_only=False):
    """Paired gate + down decode of 8 routed experts (with gate_only, the gate
    stack alone: the pages' routed figure).  Checks the configured routing
    first.  Then times graph replays (no per-launch CPU cost) of
    `copies` device copies of both stacks x `routings` disjoint routings, so
    consecutive steps touch different planes, and of the configured routing
    alone (warm)."""
    import numpy as np
    gspec, dspec = workloads.ROUTED.stacks
    xg, xd = gspec.generate(), dspec.generate()
    g = mwd.prepare(xg, gspec.fmt, index=indexed).to(dev)
    d = mwd.prepare(xd, dspec.fmt, index=indexed).to(dev)
    es = workloads.ROUTED.expert_start()
    es_t = torch.from_numpy(es).to(dev)
    wg = torch.full((g.dense_bytes,), 0xA5, dtype=torch.uint8, device=dev)
    wd = torch.full((d.dense_bytes,), 0xA5, dtype=torch.uint8, device=dev)
    mwd.decode_paired(g, wg, d, wd, es_t)
    torch.cuda.synchronize()
    active = np.diff(es) > 0
    hg = wg.cpu().numpy().reshape(xg.shape)
    hd = wd.cpu().numpy().reshape(xd.shape)
    if not (np.array_equal(hg[active], xg[active]) and np.all(hg[~active] == 0xA5)
            and np.array_equal(hd[active], xd[active]) and np.all(hd[~active] == 0xA5)):
        raise SystemExit("routed paired decode is wrong")
    spec = workloads.ROUTED
    rs = routed_sets(workloads, gspec.E, spec.n_active, spec.max_tokens, spec.seed + 100, routings)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    calls, nbytes, keep = [], [], []
    with torch.cuda.stream(side):
        for c in range(copies):
            gc, dc = (g, d) if c == 0 else (g.clone(), d.clone())
            wgc = torch.empty(g.dense_bytes, dtype=torch.uint8, device=dev)
            wdc = torch.empty(d.dense_bytes, dtype=torch.uint8, device=dev)
            for r in rs:
                rt = torch.from_numpy(r).to(dev)
                act = np.diff(r) > 0
                if gate_only:
                    calls.append(mwd.Launch(gc, wgc, expert_start=rt))
                    nbytes.append(sum(stack_bytes(gc, act)) + 4 * len(r))
                else:
                    calls.append(mwd.Launch(gc, wgc, dc, wdc, rt))
                    nbytes.append(sum(sum(stack_bytes(s, act)) for s in (gc, dc)) + 4 * len(r))
        warm = [mwd.Launch(g, wg, expert_start=es_t) if gate_only else mwd.Launch(g, wg, d, wd, es_t)] * len(calls)
        for L in calls + warm:  # warm the launch path outside capture
            L()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for seq in (calls, warm):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=side):
            for L in seq:
                L()
        graphs.append(gr)
    torch.cuda.synchronize()

    class Replay:
        stream = torch.cuda.current_stream(dev).cuda_stream

        def __init__(self, gr):
            self.gr = gr

        def __call__(self):
            self.gr.replay()

    reps = max(1, steps // len(calls))
    wall, evt = timed_loop(torch, ev, [Replay(graphs[0])], reps, max(1, warmup // len(calls)))
    wwall, wevt = timed_loop(torch, ev, [Replay(graphs[1])], reps, max(1, warmup // len(calls)))
    single = mwd.Launch(g, wg, expert_start=es_t) if gate_only else mwd.Launch(g, wg, d, wd, es_t)
    flushed = flushed_call_ms(torch, ev, single, dev)
    n = len(calls)
    b = [stack_bytes(s, active) for s in ((g,) if gate_only else (g, d))]
    return dict(step_ms=max(wall, evt) / n, event_ms=evt / n, wall_ms=wall / n,
                bytes=sum(nbytes) / len(nbytes), warm_ms=max(wwall, wevt) / n,
                warm_bytes=sum(sum(x) for x in b) + 4 * len(es), active=int(active.sum()), flushed_ms=flushed,
                sets=n, steps=reps * n)


def bench_moe(mwd, torch, ev, workloads, steps, warmup, dev, routings=64, spec=None):
    """Routed W4A16 projection of a stack's shape with its scales: the
    gate-like NVFP4 stack (512 experts x 800 rows x K = 2048) by default, or
    the MXFP4 stack (384 x 1024 x K = 5120); 8 experts routed per call with
    1..64 tokens each; `routings` disjoint routings cover every expert at least
    once, so each replay of the call sequence reads every expert's weights from HBM.
    Times, from HIP-graph replays: the stage-local consumer (scales expanded in
    LDS from the CSF streams), a routed decode into a dense workspace followed
    by the same GEMM on the dense scales, and the GEMM alone on scales decoded
    beforehand.  Checks first that the stage-local and dense-scale variants
    agree bit for bit on the first routing; the CPU baseline leg compares that
    routing's output with the oracle."""
    import numpy as np
    spec = spec or workloads.GATE
    E, N, K = spec.E, spec.R, spec.K
    fmt = "nvfp4" if spec.fmt == workloads.NVFP4 else "mxfp4"
    xs = spec.generate()
    stack = mwd.prepare(xs, spec.fmt).to(dev)
    rng = np.random.default_rng(77)
    w_host = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    w = torch.from_numpy(w_host).to(dev)
    alpha_host = rng.uniform(0.5, 2.0, E).astype(np.float32)
    alpha = torch.from_numpy(alpha_host).to(dev)
    full = torch.empty(stack.dense_bytes, dtype=torch.uint8, device=dev)
    mwd.decode(stack, full)
    ws = torch.empty(stack.dense_bytes, dtype=torch.uint8, device=dev)
    rs = routed_sets(workloads, E, workloads.ROUTED.n_active, workloads.ROUTED.max_tokens, 177, routings)
    cases, nbytes, extra_bytes = [], [], []
    pfx = stack.prefix.cpu().numpy()
    for i, es in enumerate(rs):
        T = int(es[-1])
        xb = workloads.bf16_bits(T, K, rng)
        x = torch.from_numpy(xb.view(np.int16)).to(dev)
        y = torch.empty(T, N, dtype=torch.float32, device=dev)
        es_t = torch.from_numpy(es).to(dev)
        act = np.flatnonzero(np.diff(es) > 0)
        entries = int(sum(pfx[e + 1] - pfx[e] for e in act))
        scales = len(act) * (stack.R + stack.stride) + 4 * entries + 4 * len(act) * (stack.index_tiles + 1)
        nbytes.append(len(act) * N * K // 2 + scales + T * K * 2 + T * N * 4 + 4 * (E + 1) + 4 * len(act))
        extra_bytes.append(2 * len(act) * stack.P)
        cases.append((x, y, es_t))
        if i == 0:
            y0 = mwd.moe_w4a16(stack, w, x, alpha, es_t, out=y)
            torch.cuda.synchronize()
            got = y0.cpu().numpy()
            y1 = torch.empty_like(y)
            mwd.decode(stack, ws, es_t)
            mwd.moe_w4a16(stack, w, x, alpha, es_t, out=y1, dense_scales=ws)
            torch.cuda.synchronize()
            if not torch.equal(y0, y1):
                raise SystemExit("stage-local and dense-scale projections differ")
            first = (xb, es, act)

    def seq(kind):
        for x, y, es_t in cases:
            if kind == "stage":
                mwd.moe_w4a16(stack, w, x, alpha, es_t, out=y)
            elif kind == "decode_then_gemm":
                mwd.decode(stack, ws, es_t)
                mwd.moe_w4a16(stack, w, x, alpha, es_t, out=y, dense_scales=ws)
            else:
                mwd.moe_w4a16(stack, w, x, alpha, es_t, out=y, dense_scales=full)

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    graphs = {}
    with torch.cuda.stream(side):
        for kind in ("stage", "decode_then_gemm", "dense_gemm"):
            seq(kind)  # warm the launch path outside capture
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    for kind in ("stage", "decode_then_gemm", "dense_gemm"):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=side):
            seq(kind)
        graphs[kind] = gr
    torch.cuda.synchronize()

    class Replay:
        stream = torch.cuda.current_stream(dev).cuda_stream

        def __init__(self, gr):
            self.gr = gr

        def __call__(self):
            self.gr.replay()

    n = len(cases)
    reps = max(1, steps // n)
    out = dict(bytes=sum(nbytes) / n, extra_bytes=sum(extra_bytes) / n, calls=n, steps=reps * n,
               tokens=sum(int(c[2][-1]) for c in cases) / n, first=first, w_host=w_host, xs=xs,
               alpha_host=alpha_host, first_bytes=nbytes[0], fmt=fmt, first_y=got, K=K)
    for kind, gr in graphs.items():
        wall, evt = timed_loop(torch, ev, [Replay(gr)], reps, max(1, warmup // n))
        out[kind + "_ms"] = max(wall, evt) / n
        out[kind + "_event_ms"] = evt / n
    return out


def cpu_baseline_moe(mr, budget_s=10.0):
    """The W4A16 oracle (numpy float64) computing the first routing's
    projection; its result must bound the GPU's output of that routing."""
    import numpy as np
    from oracle import w4a16 as ref
    xb, es, act = mr["first"]
    sec, n = _repeat(lambda: ref.moe_w4a16(xb, mr["w_host"], mr["xs"], mr["alpha_host"], es, experts=act,
                                           fmt=mr["fmt"]), budget_s)
    yr, mag = ref.moe_w4a16(xb, mr["w_host"], mr["xs"], mr["alpha_host"], es, experts=act, fmt=mr["fmt"])
    if not np.all(np.abs(mr["first_y"] - yr) <= (mr["K"] + 8) * 2.0 ** -24 * mag):
        raise SystemExit("routed W4A16 projection differs from the oracle")
    return dict(value=round(mr["first_bytes"] / sec / 1e9, 4), unit="GB/s", cores=_blas_threads(),
                kind="oracle", us_per_call=round(sec * 1e6, 1),
                sample=f"one routed call ({len(act)} experts, {int(es[-1])} tokens) of the W4A16 "
                       f"oracle, repeated {n} times, median")


def _blas_threads() -> int:
    """Threads numpy's BLAS may use (the float64 matmuls of the W4A16 oracle)."""
    for var in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS"):
        v = os.environ.get(var)
        if v and v.isdigit():
            return int(v)
    return len(os.sched_getaffinity(0))


def launch_floor(torch, ev, dev, steps=2000):
    """The floor under a decode call of two dependent launches: two tiny
    kernels (one-element adds) per step, launched directly and replayed from
    a HIP graph of 64 steps; µs per step."""
    t = torch.zeros(1, dtype=torch.int32, device=dev)

    class Pair:
        stream = torch.cuda.current_stream(dev).cuda_stream

        def __call__(self):
            t.add_(1)
            t.add_(1)

    wall, evt = timed_loop(torch, ev, [Pair()], steps, 100)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        Pair()()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=side):
        for _ in range(64):
            Pair()()

    class Replay:
        stream = torch.cuda.current_stream(dev).cuda_stream

        def __call__(self):
            gr.replay()

    gw, ge = timed_loop(torch, ev, [Replay()], max(1, steps // 64), 2)
    return dict(direct_us=round(max(wall, evt) * 1e3, 2), graph_us=round(max(gw, ge) / 64 * 1e3, 2))


def bench_copy(torch, ev, mwd, dev, nbytes, nsets, steps):
    srcs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(nsets)]
    dsts = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(nsets)]
    for i in range(10):
        dsts[i % nsets].copy_(srcs[i % nsets])
    torch.cuda.synchronize()
    t = time.perf_counter()
    for i in range(steps):
        dsts[i % nsets].copy_(srcs[i % nsets])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t) * 1e3 / steps
    return 2 * nbytes / (ms * 1e-3) / 1e9, ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--sets", type=int, default=8, help="rotating device copies (HBM, not cache)")
    ap.add_argument("--all", action="store_true", help="also time the other workloads on stderr")
    ap.add_argument("--all-json", default=None, metavar="PATH", help="with --all: also write those timings as JSON")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="N",
                    help="after the timed run, N plain 256 MiB device copies (reference for "
                         "hardware byte counters)")
    ap.add_argument("--workload", default="gate_nvfp4",
                    choices=["gate_nvfp4", "down_nvfp4", "mxfp4", "tiny_nvfp4", "routed_paired", "routed_moe",
                             "routed_moe_mx"],
                    help="timed workload (default: the 512-expert gate-like stack)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the CSF decode path is rank-local and has no "
              "multi-GPU mode (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_weight_decode_amd as mwd
    import workloads

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    ev = HipEvents()
    moe = args.workload.startswith("routed_moe")
    if moe:
        mx = args.workload == "routed_moe_mx"
        mr = bench_moe(mwd, torch, ev, workloads, args.steps, args.warmup, dev,
                       spec=workloads.MX if mx else workloads.GATE)
        step_bytes = mr["bytes"]
        r = dict(step_ms=mr["stage_ms"], event_ms=mr["stage_event_ms"], wall_ms=mr["stage_ms"])
        shape = ("the MXFP4 stack's shape (384 experts x 1024 rows x K=5120, MXFP4 weights, CSF scales of "
                 "the MXFP4 stack) with 8 of 384 experts" if mx else
                 "the gate-like shape (512 experts x 800 rows x K=2048, NVFP4 weights, CSF scales of the "
                 "gate-like stack) with 8 of 512 experts")
        config = {
            "workload": f"{args.workload}: W4A16 projection of {shape} routed (1..64 tokens each); scales "
                        "expanded in LDS from the CSF streams",
            "decode": "stage-local (csf_moe_w4a16 reading the CSF streams); steps replayed from a HIP "
                      "graph of all rotating routings",
            "bytes_per_step": round(step_bytes),
            "mean_tokens": mr["tokens"],
            "rotating_sets": mr["calls"],
            "timed_steps": mr["steps"],
            "decode_then_gemm_us": round(mr["decode_then_gemm_ms"] * 1e3, 3),
            "dense_scale_gemm_us": round(mr["dense_gemm_ms"] * 1e3, 3),
            "decode_then_gemm_extra_bytes": round(mr["extra_bytes"]),
        }
        x_head = None
    elif args.workload == "routed_paired":
        rr = bench_routed(mwd, torch, ev, workloads, args.steps, args.warmup, dev)
        gs, ds = workloads.ROUTED.stacks
        step_bytes = rr["bytes"]
        r = dict(step_ms=rr["step_ms"], event_ms=rr["event_ms"], wall_ms=rr["wall_ms"])
        config = {
            "workload": f"routed_paired: one paired decode of the {gs.name} ({gs.E}x{gs.R}x{gs.C}) and "
                        f"{ds.name} ({ds.E}x{ds.R}x{ds.C}) stacks with {rr['active']} of {gs.E} experts "
                        f"routed (1..64 tokens each), int32 expert_start read on the device",
            "decode": "single pass (fused kernel, tile index), routed; steps replayed from a "
                      "HIP graph of all rotating sets",
            "bytes_per_step": round(step_bytes),
            "rotating_sets": rr["sets"],
            "timed_steps": rr["steps"],
            "warm_us_same_routing": round(rr["warm_ms"] * 1e3, 3),
        }
        x_head = None
    else:
        spec = workloads.STACKS[args.workload]
        log(f"[bench] {spec.name}: generating and encoding {spec.E}x{spec.R}x{spec.C}")
        r = bench_stack(mwd, torch, ev, spec, args.steps, args.warmup,
                        args.sets if spec.E > 4 else 2, dev)
        stack = r["stack"]
        step_bytes = r["fixed_bytes"] + r["exc_bytes"] + r["dense_bytes"]
        fmt = "NVFP4 (E4M3 scales)" if spec.fmt == workloads.NVFP4 else "MXFP4 (UE8M0 scales)"
        config = {
            "workload": f"{spec.name}: full-stack CSF decode of {spec.E} experts x {spec.R} rows x "
                        f"{spec.C} scale columns (K={spec.K}), {spec.desc.split(', ', 1)[-1]}, "
                        f"seed {spec.seed}",
            "experts": spec.E, "rows": spec.R, "cols": spec.C, "format": fmt,
            "decode": "single pass (fused kernel, tile index)",
            "exception_entries": stack.num_exceptions,
            "compressed_bytes": r["fixed_bytes"] + r["exc_bytes"],
            "dense_bytes": r["dense_bytes"],
            "bytes_per_step": step_bytes,
            "rotating_sets": args.sets if spec.E > 4 else 2,
        }
        x_head = r["x"]
    gbps = step_bytes / (r["step_ms"] * 1e-3) / 1e9
    launch_us = r["event_ms"] * 1e3
    achieved = step_bytes / (r["event_ms"] * 1e-3) / 1e9
    log(f"[bench] step {r['step_ms'] * 1e3:.2f} us (wall {r['wall_ms'] * 1e3:.2f}, events "
        f"{r['event_ms'] * 1e3:.2f}); {gbps:.1f} GB/s")
    kernel = "csf_moe_w4a16_kernel" if moe else "csf_fused_kernel"
    traffic = pmc_traffic(kernel, args.workload)
    out = {
        "metric": MOE_METRIC if moe else METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["step_ms"], 6),
        ("us_per_call" if args.workload.startswith("routed") else "us_per_stack"): round(r["step_ms"] * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if moe else "u8",
        "data": "synthetic",
        "config": config,
        "roofline": {
            "kernel": kernel,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": round(step_bytes),
            "mean_launch_us": round(launch_us, 3),
        },
    }
    if args.all:
        extra = {}
        del r
        for name in ("gate_nvfp4", "down_nvfp4", "mxfp4", "tiny_nvfp4"):
            s = workloads.STACKS[name]
            log(f"[bench] {name}")
            rr = bench_stack(mwd, torch, ev, s, min(args.steps, 2000), args.warmup,
                             args.sets if s.E > 4 else 2, dev, split=True)
            b = rr["fixed_bytes"] + rr["exc_bytes"] + rr["dense_bytes"]
            extra[name] = dict(us=round(rr["step_ms"] * 1e3, 2),
                               gbps=round(b / (rr["step_ms"] * 1e-3) / 1e9, 1),
                               two_pass_us=round(rr["two_pass_ms"] * 1e3, 2),
                               fixed_only_us=round(rr["fixed_only_ms"] * 1e3, 2),
                               warm_us=round(rr["warm_ms"] * 1e3, 2),
                               flushed_us=round(rr["flushed_ms"] * 1e3, 2),
                               bytes=b, entries=rr["stack"].num_exceptions)
            xd = torch.from_numpy(rr["x"]).to(dev)
            enc = []
            for i in range(12):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                mwd.prepare(xd, s.fmt)  # device encode; reads back the entry count once
                torch.cuda.synchronize()
                enc.append(time.perf_counter() - t0)
            extra[name]["gpu_encode_us"] = round(statistics.median(enc[2:]) * 1e6, 1)
            log(f"[bench] {name}: {extra[name]}")
            del rr, xd
            torch.cuda.empty_cache()
        for indexed, gate_only in ((True, False), (False, False), (True, True)):
            key = ("routed_gate" if gate_only else "routed_paired") + ("" if indexed else "_two_pass")
            log(f"[bench] {key}")
            rr = bench_routed(mwd, torch, ev, workloads, min(args.steps, 2000), args.warmup, dev, indexed,
                              gate_only=gate_only)
            extra[key] = dict(us=round(rr["step_ms"] * 1e3, 2),
                              gbps=round(rr["bytes"] / (rr["step_ms"] * 1e-3) / 1e9, 1),
                              warm_us=round(rr["warm_ms"] * 1e3, 2), flushed_us=round(rr["flushed_ms"] * 1e3, 2),
                              bytes=round(rr["bytes"]),
                              active=rr["active"], sets=rr["sets"])
            log(f"[bench] {key}: {extra[key]}")
        extra["launch_floor"] = launch_floor(torch, ev, dev)
        log(f"[bench] launch floor: {extra['launch_floor']}")
        cg, cms = bench_copy(torch, ev, mwd, dev, 64 << 20, 8, 500)
        extra["copy_64MiB"] = dict(gbps=round(cg, 1), us=round(cms * 1e3, 2))
        log(f"[bench] plain copy 64 MiB: {extra['copy_64MiB']}")
        if args.all_json:
            os.makedirs(os.path.dirname(os.path.abspath(args.all_json)), exist_ok=True)
            json.dump(extra, open(args.all_json, "w"), indent=1)
    if args.calibrate_copy:
        # an elementwise kernel (a large device-to-device copy_ may go to a DMA
        # engine, which the counters do not see): 256 MiB read, 256 MiB written
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.calibrate_copy):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] {args.calibrate_copy} calibration kernels reading and writing 268435456 bytes")
        del src, dst
    if not args.no_cpu:
        log(f"[bench] cpu oracle baseline (~{args.cpu_seconds:.0f} s)")
        if args.workload == "routed_paired":
            out["cpu_baseline"] = cpu_baseline_routed(workloads, args.cpu_seconds)
        elif moe:
            out["cpu_baseline"] = cpu_baseline_moe(mr, args.cpu_seconds)
        else:
            out["cpu_baseline"] = cpu_baseline(spec, x_head, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
