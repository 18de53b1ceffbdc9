"""Benchmark of the CSF block-scale decoder on one MI355X.

One step = one full decode of the 512-expert gate-like NVFP4 stack (512 x 800
x 128 E4M3 scale bytes, 3 % outliers, with its tile index) into its dense
workspace: a single launch of the fused kernel (fixed stream + exceptions
patched on chip).  Steps rotate over several device copies of the compressed
stack and workspace (together larger than the 256 MB Infinity Cache), so
every step reads and writes HBM.

Prints ONE JSON line on stdout:
  value        whole-run throughput, GB/s = algorithmic bytes per step (the
               compressed streams read: bases, offsets, exception entries,
               entry prefix; the dense bytes written) x steps / elapsed time
  roofline     the fused kernel (the only kernel of a step): the same bytes
               per launch / its mean launch time, from two HIP events on its
               stream bracketing a second run of the same back-to-back steps
               (the wall-clock run has no events in it), against the MI355X
               HBM3E peak (8 TB/s); next to it the
               kernel average of the committed rocprofv3 trace of the same
               sources, and the plain stream-mix kernel's rate on the same
               buffers (the ceiling of this access pattern on this chip)
  cpu_baseline the CPU oracle decoding the same stack on the host's cores (one
               thread, and threads over disjoint expert ranges)

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
kernel), warm and cache-flushed single calls, the stream-mix ceiling of each
stack, the launch floors (an empty kernel and kernels with 0-3 dependent
round trips to memory at the routed decode's grid), the host cost of a
decode call (C and Python), the per-step timestamps of the routed decode and
the GPU encode; one line each on stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import subprocess
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


class StackBytes(tuple):
    """Algorithmic bytes of one decode of a stack: ``fixed`` (bases and
    offset segments read), ``exc`` (exception entries and the entry prefix
    read), ``dense`` (bytes written) and, apart, ``index`` (the tile index
    this build adds to the format; a routed decode reads only its routed
    experts' segments).  ``metric`` = fixed + exc + dense, the compressed
    bytes read plus the dense bytes written."""

    def __new__(cls, fixed, exc, dense, index):
        return super().__new__(cls, (fixed, exc, dense, index))

    fixed = property(lambda self: self[0])
    exc = property(lambda self: self[1])
    dense = property(lambda self: self[2])
    index = property(lambda self: self[3])
    metric = property(lambda self: self[0] + self[1] + self[2])


def stack_bytes(stack, active=None) -> StackBytes:
    """Bytes one decode of ``stack`` reads and writes; ``active`` is a boolean
    mask of routed experts, or None for all."""
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
    index = 0
    if stack.tile_index is not None:
        index = 4 * (E * stack.index_tiles + 1) if active is None else 4 * n_act * (stack.index_tiles + 1)
    return StackBytes(fixed, exc, n_act * stack.P, index)


_KERNEL_SOURCES = {
    "csf_fused_kernel": ("csf_kernels.hip",),
    "csf_routed_kernel": ("csf_kernels.hip",),
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


def profile_time(kernel: str, workload: str):
    """Average kernel duration (ns) from the committed rocprofv3 kernel trace
    of this workload, if it was taken on the current kernel sources; else
    None."""
    path = os.path.join(ROOT, "profiles", "kernel_times.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{kernel}/{workload}")
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec


def make_sets(mwd, torch, stack, nsets, dev):
    sets = []
    for i in range(nsets):
        s = stack if i == 0 else stack.clone()
        ws = torch.empty(stack.dense_bytes, dtype=torch.uint8, device=dev)
        sets.append((s, ws))
    return sets


def timed_loop(torch, ev, calls, steps, warmup):
    """Run `steps` calls (after `warmup`), rotating over `calls`, twice: once
    bracketed by torch.cuda.synchronize() alone (the wall clock of exactly
    those steps), once with one HIP event before and one after the run on
    the launch stream (an event record costs the stream a few µs and the host
    more, so it stays out of the wall-clock run).  Returns (wall-clock ms per
    step, event ms per step)."""
    stream = calls[0].stream
    n = len(calls)
    for i in range(warmup):
        calls[i % n]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        calls[i % n]()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    evs = ev.create(2)
    torch.cuda.synchronize()
    ev.record(evs[0], stream)
    for i in range(steps):
        calls[i % n]()
    ev.record(evs[1], stream)
    torch.cuda.synchronize()
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


def bench_stack(mwd, torch, ev, spec, steps, warmup, nsets, dev, split=False, ceiling=True, two_pass=False):
    """Time the full decode of `spec` (fused, indexed stack; with `two_pass`
    the two-pass decode of the stack without its index) and, with `ceiling`,
    the stream-mix kernel on the same buffers; with `split` also the two-pass
    decode of the same stack and its fixed pass alone, one stack decoded over
    and over (warm: its 85-109 MB stay in the MALL), and single calls on
    flushed caches."""
    x = spec.generate()
    stack = mwd.prepare(x, spec.fmt).to(dev)
    sets = make_sets(mwd, torch, stack, nsets, dev)
    launches = [mwd.Launch(s.without_index() if two_pass else s, ws) for s, ws in sets]
    launches[0]()
    torch.cuda.synchronize()
    check_equal(torch, sets[0][1], x, spec.name)
    wall, evt = timed_loop(torch, ev, launches, steps, warmup)
    out = dict(x=x, stack=stack, bytes=stack_bytes(stack.without_index() if two_pass else stack),
               step_ms=max(wall, evt), wall_ms=wall, event_ms=evt)
    if ceiling and spec.E > 4:
        out["ceiling"] = bench_ceiling(mwd, torch, ev, sets, min(steps, 2000), warmup, dev)
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


def bench_ceiling(mwd, torch, ev, sets, steps, warmup, dev):
    """The stream-mix kernel (csf_probe_mix) on each rotating set's own
    buffers: it reads the offset segments, the exception entries and the row
    bases and writes the workspace, the bytes and access shape of the decode
    without its work.  Best of 4, 6 and 8 workgroups per CU, with cached and
    with non-temporal entry loads; also the same without the entry stream.
    Event time per step (ms) and the configuration of the best."""
    from moe_weight_decode_amd import probe
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    best, best_cfg = None, None
    for wg in (4, 6, 8):
        for flags in (0, probe.NT_ENTRIES):
            mixes = [probe.Mix([s.offsets, s.exceptions[:s.num_exceptions], s.bases], ws, cus * wg, flags)
                     for s, ws in sets]
            _, evt = timed_loop(torch, ev, mixes, steps, warmup)
            if best is None or evt < best:
                best, best_cfg = evt, dict(wg_per_cu=wg, entry_loads="nt" if flags else "cached")
    two = [probe.Mix([s.offsets, s.bases], ws, cus * best_cfg["wg_per_cu"]) for s, ws in sets]
    _, evt2 = timed_loop(torch, ev, two, steps, warmup)
    return dict(event_ms=best, config=best_cfg, without_entries_ms=evt2)


def _repeat(fn, budget_s):
    times = []
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or len(times) < 3:
        t = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t)
    return statistics.median(times), len(times)


def cpu_info():
    """The host CPU: model, sockets and the threads this process may run on."""
    model, sockets = None, None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() == "Model name" and model is None:
                model = v.strip()
            elif k.strip() == "Socket(s)":
                sockets = int(v.strip()) if v.strip().isdigit() else v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None and os.path.exists("/proc/cpuinfo"):
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    return dict(model=model, sockets=sockets, affinity=len(os.sched_getaffinity(0)))


def cpu_threads() -> int:
    """Threads of the threaded oracle runs: the process's CPUs, at most the
    OMP_NUM_THREADS share when it is set."""
    n = len(os.sched_getaffinity(0))
    v = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(v))) if v.isdigit() else n


def _slices(E, n):
    step = (E + n - 1) // n
    return [(e, min(E, e + step)) for e in range(0, E, step)]


def oracle_runs(orc, jobs, budget_s):
    """Median seconds of one round of `jobs` (callables decoding disjoint
    expert ranges, each from one thread per job), about budget_s / 2 seconds
    on one thread and as much on len(jobs) threads."""
    from concurrent.futures import ThreadPoolExecutor
    one, n1 = _repeat(lambda: [j() for j in jobs], budget_s / 2)
    with ThreadPoolExecutor(len(jobs)) as pool:
        many, nn = _repeat(lambda: list(pool.map(lambda j: j(), jobs)), budget_s / 2)
    return one, n1, many, nn


def cpu_baseline(spec, x, budget_s=10.0):
    """The oracle (plain C) decoding the whole stack on one host thread, and
    on N threads over disjoint expert ranges (the same C function per range),
    each repeated for about budget_s / 2 seconds; GB/s on the GPU's byte
    formula.  The oracle's encode of the stack (one thread) is timed once, as
    context."""
    import numpy as np
    import oracle
    orc = oracle.load()
    t = time.perf_counter()
    st = orc.encode(spec.fmt, x)
    encode_s = time.perf_counter() - t
    ws = np.empty_like(x)
    n = cpu_threads()
    jobs = [lambda a=a, b=b: orc.decode_experts(st, a, b, ws) for a, b in _slices(spec.E, n)]
    for j in jobs:
        j()
    if not np.array_equal(ws, x):
        raise SystemExit("oracle round trip failed")
    one, n1, many, nn = oracle_runs(orc, jobs, budget_s)
    if not np.array_equal(ws, x):
        raise SystemExit("threaded oracle decode failed")
    E = spec.E
    nbytes = E * spec.R + E * st["stride"] + 4 * st["exceptions"].size + 4 * (E + 1) + x.size
    return dict(value=round(nbytes / many / 1e9, 4), unit="GB/s", cores=len(jobs), kind="oracle",
                us_per_stack=round(many * 1e6, 1),
                single_thread=dict(value=round(nbytes / one / 1e9, 4), us_per_stack=round(one * 1e6, 1), runs=n1),
                cpu=cpu_info(), oracle_encode_s=round(encode_s, 3),
                sample=f"whole {spec.name} stack ({spec.E}x{spec.R}x{spec.C}) decoded {nn} times on {len(jobs)} "
                       f"threads (disjoint expert ranges) and {n1} times on one thread, median of each")


def cpu_baseline_routed(workloads, budget_s=10.0):
    """The oracle's routed decode of the gate and down stacks (8 of 512
    experts), on one host thread and on N threads over disjoint expert
    ranges; GB/s on the GPU's byte formula."""
    import numpy as np
    import oracle
    orc = oracle.load()
    gspec, dspec = workloads.ROUTED.stacks
    es = workloads.ROUTED.expert_start()
    act = np.diff(es) > 0
    jobs, nbytes = [], 4 * len(es)
    n = cpu_threads()
    for spec in (gspec, dspec):
        x = spec.generate()
        st = orc.encode(spec.fmt, x)
        ws = np.zeros(x.shape, dtype=np.uint8)
        jobs += [lambda a=a, b=b, st=st, ws=ws: orc.decode_experts(st, a, b, ws, es)
                 for a, b in _slices(spec.E, max(1, n // 2))]
        ent = int(np.diff(st["prefix"])[act].sum())
        nbytes += int(act.sum()) * (spec.R + st["stride"] + spec.R * spec.C) + 4 * ent + 4 * (spec.E + 1)
    one, n1, many, nn = oracle_runs(orc, jobs, budget_s)
    return dict(value=round(nbytes / many / 1e9, 4), unit="GB/s", cores=len(jobs), kind="oracle",
                us_per_call=round(many * 1e6, 1),
                single_thread=dict(value=round(nbytes / one / 1e9, 4), us_per_call=round(one * 1e6, 1), runs=n1),
                cpu=cpu_info(),
                sample=f"routed paired decode (8 of 512 experts) of the gate and down stacks, {nn} times on "
                       f"{len(jobs)} threads (disjoint expert ranges) and {n1} times on one thread, median of each")


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
    calls, nbytes, index_bytes = [], [], []
    with torch.cuda.stream(side):
        for c in range(copies):
            gc, dc = (g, d) if c == 0 else (g.clone(), d.clone())
            wgc = torch.empty(g.dense_bytes, dtype=torch.uint8, device=dev)
            wdc = torch.empty(d.dense_bytes, dtype=torch.uint8, device=dev)
            for r in rs:
                rt = torch.from_numpy(r).to(dev)
                act = np.diff(r) > 0
                stacks = (gc,) if gate_only else (gc, dc)
                if gate_only:
                    calls.append(mwd.Launch(gc, wgc, expert_start=rt))
                else:
                    calls.append(mwd.Launch(gc, wgc, dc, wdc, rt))
                b = [stack_bytes(s, act) for s in stacks]
                nbytes.append(sum(x.metric for x in b) + 4 * len(r))  # + expert_start
                index_bytes.append(sum(x.index for x in b))
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
                bytes=sum(nbytes) / len(nbytes), index_bytes=sum(index_bytes) / len(index_bytes),
                warm_ms=max(wwall, wevt) / n,
                warm_bytes=sum(x.metric for x in b) + 4 * len(es), active=int(active.sum()), flushed_ms=flushed,
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


def bench_encode(mwd, torch, workloads, name, steps, warmup, dev):
    """GPU encodes (csf_encode_device through prepare) of a workload stack
    already in device memory, checked once against the host encoder; wall
    time per encode (with its one read-back of the entry count).  name
    "layer" encodes the gate-like and down-like stacks together (one layer's
    two projections, prepare_many: one read-back for both)."""
    import numpy as np
    specs = [workloads.GATE, workloads.DOWN] if name == "layer" else [workloads.STACKS[name]]
    xs = [s.generate() for s in specs]
    xds = [torch.from_numpy(x).to(dev) for x in xs]
    fmts = [s.fmt for s in specs]
    wants = [mwd.prepare(x, f).numpy() for x, f in zip(xs, fmts)]
    gots = [g.numpy() for g in mwd.prepare_many(xds, fmts)]
    for spec, got, want in zip(specs, gots, wants):
        for k in ("bases", "offsets", "exceptions", "prefix", "tile_index"):
            if not np.array_equal(np.asarray(got[k]).ravel(), np.asarray(want[k]).ravel()):
                raise SystemExit(f"GPU encode of {spec.name} differs from the host encoder in {k}")
    for _ in range(warmup):
        mwd.prepare_many(xds, fmts)
    torch.cuda.synchronize()
    t = []
    for _ in range(steps):
        t0 = time.perf_counter()
        mwd.prepare_many(xds, fmts)
        torch.cuda.synchronize()
        t.append(time.perf_counter() - t0)
    return dict(encode=name, shapes=[[s.E, s.R, s.C] for s in specs], dense_bytes=int(sum(x.size for x in xs)),
                steps=steps, us_per_encode=round(statistics.median(t) * 1e6, 1))


def graph_of(torch, dev, calls):
    """A HIP graph of `calls` in order (warmed outside capture), replayed on
    the current stream: returns a callable with the replay stream's handle."""
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for c in calls:
            c()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=side):
        for c in calls:
            c()
    torch.cuda.synchronize()

    class Replay:
        stream = torch.cuda.current_stream(dev).cuda_stream

        def __call__(self):
            gr.replay()

    r = Replay()
    r.graph = gr
    return r


def launch_floors(torch, ev, dev, grid, reps=40, per_graph=64):
    """Floors under a routed decode call, from graph replays of per_graph
    launches (µs per launch): an empty one-wave kernel; an empty kernel at
    the routed decode's grid (grid x 256 lanes); the same storing 16 bytes
    per lane; and with 1, 2, 3 dependent round trips to memory before the
    stores (csf_probe_chain: each workgroup follows a chain of 4-byte loads
    through 1 GiB, from a start set by the workgroup and the launch, so the
    loads miss the caches); and the latency of one dependent load, from a
    chain of 64 links through 1 GiB with cold caches (HBM) and again warm
    (L2)."""
    from moe_weight_decode_amd import probe
    words = 1 << 28
    i = torch.arange(words, dtype=torch.int64, device=dev)
    buf = ((i * 0x9E3779B1 + 12345) & (words - 1)).to(torch.int32)  # a permutation of 0 .. words-1
    del i
    outs = [torch.empty(grid * 256 * 16, dtype=torch.uint8, device=dev) for _ in range(8)]
    cases = {"empty_1wave": (0, False, 1, 64), "empty_grid": (0, False, grid, 256),
             "store_grid": (0, True, grid, 256), "chain1_store": (1, True, grid, 256),
             "chain2_store": (2, True, grid, 256), "chain3_store": (3, True, grid, 256)}
    out = {}
    for name, (hops, store, g, block) in cases.items():
        calls = [probe.Chain(buf if hops else None, hops, outs[k % len(outs)] if store else None, g, block,
                             seed=k + 1) for k in range(per_graph)]
        rep = graph_of(torch, dev, calls)
        wall, evt = timed_loop(torch, ev, [rep], reps, 3)
        out[name + "_us"] = round(max(wall, evt) / per_graph * 1e3, 3)
    # latency of one dependent load: one wave following 0 and 64 links of the
    # 1 GiB chain after a 512 MiB write has evicted it from the caches (HBM),
    # and the same chain again right after (L2); event pairs around the
    # launch alone, median of 15
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    evs = ev.create(2)
    stream = torch.cuda.current_stream(dev).cuda_stream
    lat = {"hbm": {}, "l2": {}}
    for hops in (0, 64):
        for name in ("hbm", "l2"):
            lat[name][hops] = []
        for r in range(15):
            call = probe.Chain(buf, hops, None, 1, 64, seed=1000 + r)
            flush.fill_(r & 0xFF)
            for name in ("hbm", "l2"):
                ev.record(evs[0], stream)
                call()
                ev.record(evs[1], stream)
                torch.cuda.synchronize()
                lat[name][hops].append(ev.ms(evs[0], evs[1]) * 1e6)
    ev.destroy(evs)
    for name in ("hbm", "l2"):
        out[f"load_latency_{name}_ns"] = round(
            (statistics.median(lat[name][64]) - statistics.median(lat[name][0])) / 64, 1)
    del buf, outs, flush
    torch.cuda.empty_cache()
    out["grid"] = grid
    return out


def host_cost(mwd, torch, dev, g, d, es_t, calls=300):
    """Host time per decode call, enqueue only: the C ABI called from C
    (csf_probe_host_ns) and from Python through the binding's Launch; full
    gate-stack decode and routed paired decode (µs)."""
    from moe_weight_decode_amd import probe
    wg = torch.empty(g.dense_bytes, dtype=torch.uint8, device=dev)
    wd = torch.empty(d.dense_bytes, dtype=torch.uint8, device=dev)
    out = {}
    for name, args in (("full_gate", (g, wg, None, None, None)), ("routed_paired", (g, wg, d, wd, es_t))):
        probe.host_ns(*args, calls=20)
        torch.cuda.synchronize()
        c_ns = probe.host_ns(*args, calls=calls)
        torch.cuda.synchronize()
        L = mwd.Launch(*args)
        for _ in range(20):
            L()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(calls):
            L()
        py_ns = (time.perf_counter() - t) / calls * 1e9
        torch.cuda.synchronize()
        out[name] = dict(c_call_us=round(c_ns / 1e3, 3), python_launch_us=round(py_ns / 1e3, 3))
    return out


def clock_hz(mwd, torch, g, dev, wait_s=0.25):
    """Rate of the clock the traced decode reads: the earliest start stamp of
    two traced calls wait_s seconds apart, against the host's clock."""
    import numpy as np
    es = torch.zeros(g.E + 1, dtype=torch.int32, device=dev)
    es[1:] = 1  # expert 0 routed
    ws = torch.empty(g.dense_bytes, dtype=torch.uint8, device=dev)
    a = mwd.decode_traced(g, ws, expert_start=es)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    time.sleep(wait_s)
    b = mwd.decode_traced(g, ws, expert_start=es)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ticks = int(b[:, 0].cpu().numpy().view(np.uint64).min()) - int(a[:, 0].cpu().numpy().view(np.uint64).min())
    return ticks / (t1 - t0)


def trace_routed(mwd, torch, dev, g, d, routings, copies=2):
    """Per-step timestamps of routed paired decodes (csf_decode_traced), one
    call per routing and stack copy, launched one by one; medians over the
    workgroups that decoded a tile, in ns from the call's first workgroup
    start (the clock is the device's constant-rate wall clock)."""
    import numpy as np
    ns_per_tick = 1e9 / clock_hz(mwd, torch, g, dev)
    stacks = [(g, d)] + [(g.clone(), d.clone()) for _ in range(copies - 1)]
    wss = [(torch.empty(g.dense_bytes, dtype=torch.uint8, device=dev),
            torch.empty(d.dense_bytes, dtype=torch.uint8, device=dev)) for _ in stacks]
    rts = [torch.from_numpy(r).to(dev) for r in routings]
    names = ["routing", "loads", "expand", "patch", "store_issue", "store_done"]
    rows, spans, long_tiles, units = [], [], 0, 0
    for k in range(2 + len(rts) * len(stacks)):
        (gc, dc), (wg, wd) = stacks[k % len(stacks)], wss[k % len(stacks)]
        st = mwd.decode_traced(gc, wg, dc, wd, rts[k % len(rts)])
        torch.cuda.synchronize()
        if k < 2:
            continue  # warm the launch path
        t = st.cpu().numpy().view(np.uint64).astype(np.float64)
        tags = st[:, 7].cpu().numpy().view(np.uint64)
        busy = (tags != 0) & (tags != np.uint64(0xFFFFFFFFFFFFFFFF))
        t0 = t[:, 0].min()
        rel = (t[busy, :7] - t0) * ns_per_tick
        rows.append(rel)
        spans.append((t[busy, 6].max() - t0) * ns_per_tick)
        long_tiles += int(np.count_nonzero((tags[busy] >> np.uint64(32)) & np.uint64(1)))
        units += int(busy.sum())
    rel = np.concatenate(rows)
    steps = np.diff(rel, axis=1)
    out = dict(start_ns_median=round(float(np.median(rel[:, 0])), 1),
               start_ns_p90=round(float(np.percentile(rel[:, 0], 90)), 1),
               done_ns_median=round(float(np.median(rel[:, 6])), 1),
               span_ns_median=round(float(np.median(spans)), 1),
               calls=len(spans), tiles=units, tiles_beyond_prefetch=long_tiles, ns_per_tick=ns_per_tick)
    for i, n in enumerate(names):
        out[n + "_ns_median"] = round(float(np.median(steps[:, i])), 1)
        out[n + "_ns_p90"] = round(float(np.percentile(steps[:, i], 90)), 1)
    return out


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
    ap.add_argument("--encode", default=None, metavar="STACK",
                    help="instead: time the GPU encoder (csf_encode_device) on a workload stack (or 'layer': "
                         "the gate-like and down-like stacks together), --steps times, and print one JSON line")
    ap.add_argument("--two-pass", action="store_true",
                    help="full-stack workloads: time the two-pass decode (fixed-stream kernel, then exception "
                         "kernel) of the stack without its tile index")
    ap.add_argument("--workload", default="gate_nvfp4",
                    choices=["gate_nvfp4", "down_nvfp4", "mxfp4", "tiny_nvfp4", "routed_paired", "routed_moe",
                             "routed_moe_mx"],
                    help="timed workload (default: the 512-expert gate-like stack)")
    args = ap.parse_args()
    if args.two_pass and (args.workload.startswith("routed") or args.encode):
        raise SystemExit("--two-pass applies to the full-stack workloads")
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
    if args.encode:
        print(json.dumps(bench_encode(mwd, torch, workloads, args.encode, args.steps, args.warmup, dev)), flush=True)
        return
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
            "index_bytes_per_step": round(rr["index_bytes"]),
            "rotating_sets": rr["sets"],
            "timed_steps": rr["steps"],
            "warm_us_same_routing": round(rr["warm_ms"] * 1e3, 3),
        }
        x_head = None
    else:
        spec = workloads.STACKS[args.workload]
        log(f"[bench] {spec.name}: generating and encoding {spec.E}x{spec.R}x{spec.C}")
        r = bench_stack(mwd, torch, ev, spec, args.steps, args.warmup,
                        args.sets if spec.E > 4 else 2, dev, two_pass=args.two_pass)
        stack, b = r["stack"], r["bytes"]
        step_bytes = b.metric
        fmt = "NVFP4 (E4M3 scales)" if spec.fmt == workloads.NVFP4 else "MXFP4 (UE8M0 scales)"
        config = {
            "workload": f"{spec.name}: full-stack CSF decode of {spec.E} experts x {spec.R} rows x "
                        f"{spec.C} scale columns (K={spec.K}), {spec.desc.split(', ', 1)[-1]}, "
                        f"seed {spec.seed}",
            "experts": spec.E, "rows": spec.R, "cols": spec.C, "format": fmt,
            "decode": ("two-pass (csf_fixed_kernel, then csf_exc_kernel; no tile index)" if args.two_pass
                       else "single pass (fused kernel, tile index)"),
            "exception_entries": stack.num_exceptions,
            "compressed_bytes": b.fixed + b.exc,
            "dense_bytes": b.dense,
            "bytes_per_step": step_bytes,
            "index_bytes_per_step": b.index,
            "rotating_sets": args.sets if spec.E > 4 else 2,
        }
        if args.two_pass:
            # per pass: the fixed stream reads bases and offsets and writes the
            # dense bytes; the exception pass reads the entries and prefix
            config.update(fixed_pass_bytes=b.fixed + b.dense, exception_pass_bytes=b.exc)
        x_head = r["x"]
    gbps = step_bytes / (r["step_ms"] * 1e-3) / 1e9
    launch_us = r["event_ms"] * 1e3
    achieved = step_bytes / (r["event_ms"] * 1e-3) / 1e9
    log(f"[bench] step {r['step_ms'] * 1e3:.2f} us (wall {r['wall_ms'] * 1e3:.2f}, events "
        f"{r['event_ms'] * 1e3:.2f}); {gbps:.1f} GB/s")
    kernel = ("csf_moe_w4a16_kernel" if moe else
              "csf_routed_kernel" if args.workload == "routed_paired" else
              "csf_fixed_kernel + csf_exc_kernel" if args.two_pass else "csf_fused_kernel")
    traffic = pmc_traffic(kernel, args.workload)
    roof = {
        "kernel": kernel,
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "algorithmic_bytes_per_launch": round(step_bytes),
        "mean_launch_us": round(launch_us, 3),
        "timing": "mean launch time from HIP events on the launch stream around the timed launches",
    }
    prof = profile_time(kernel, args.workload)
    if prof is not None:
        roof["profile"] = {"avg_us": round(prof["avg_ns"] / 1e3, 3), "calls": prof["calls"],
                           "frac": round(step_bytes / (prof["avg_ns"] * 1e-9) / 1e9 / HBM_PEAK_GBPS, 4),
                           "source": "profiles/kernel_times.json (rocprofv3 --kernel-trace --stats, same sources)"}
    if not moe and "ceiling" in r:
        c = r["ceiling"]
        cg = step_bytes / (c["event_ms"] * 1e-3) / 1e9
        roof["ceiling"] = {"gbps": round(cg, 1), "frac": round(achieved / cg, 4), **c["config"],
                           "kind": "csf_probe_mix on the same buffers: the decode's streams and access shape "
                                   "without its work"}
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
        "roofline": roof,
    }
    if args.all:
        out_all = run_all(mwd, torch, ev, workloads, args, dev)
        if args.all_json:
            os.makedirs(os.path.dirname(os.path.abspath(args.all_json)), exist_ok=True)
            json.dump(out_all, open(args.all_json, "w"), indent=1)
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


def run_all(mwd, torch, ev, workloads, args, dev):
    """The --all measurements; one line each on stderr; returns them."""
    import numpy as np
    extra = {}
    for name in ("gate_nvfp4", "down_nvfp4", "mxfp4", "tiny_nvfp4"):
        s = workloads.STACKS[name]
        log(f"[bench] {name}")
        rr = bench_stack(mwd, torch, ev, s, min(args.steps, 2000), args.warmup,
                         args.sets if s.E > 4 else 2, dev, split=True)
        b = rr["bytes"]
        e = dict(us=round(rr["step_ms"] * 1e3, 2), event_us=round(rr["event_ms"] * 1e3, 2),
                 gbps=round(b.metric / (rr["step_ms"] * 1e-3) / 1e9, 1),
                 event_gbps=round(b.metric / (rr["event_ms"] * 1e-3) / 1e9, 1),
                 two_pass_us=round(rr["two_pass_ms"] * 1e3, 2),
                 fixed_only_us=round(rr["fixed_only_ms"] * 1e3, 2),
                 warm_us=round(rr["warm_ms"] * 1e3, 2),
                 flushed_us=round(rr["flushed_ms"] * 1e3, 2),
                 bytes=b.metric, index_bytes=b.index, entries=rr["stack"].num_exceptions)
        if "ceiling" in rr:
            c = rr["ceiling"]
            cg = b.metric / (c["event_ms"] * 1e-3) / 1e9
            e.update(ceiling_us=round(c["event_ms"] * 1e3, 2), ceiling_gbps=round(cg, 1),
                     frac_of_ceiling=round(c["event_ms"] / rr["event_ms"], 4), ceiling_config=c["config"],
                     ceiling_without_entries_gbps=round((b.metric - b.exc) / (c["without_entries_ms"] * 1e-3) / 1e9,
                                                        1))
        xd = torch.from_numpy(rr["x"]).to(dev)
        enc = []
        for i in range(12):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            mwd.prepare(xd, s.fmt)  # device encode; reads back the entry count once
            torch.cuda.synchronize()
            enc.append(time.perf_counter() - t0)
        e["gpu_encode_us"] = round(statistics.median(enc[2:]) * 1e6, 1)
        extra[name] = e
        log(f"[bench] {name}: {e}")
        del rr, xd
        torch.cuda.empty_cache()
    le = bench_encode(mwd, torch, workloads, "layer", 20, 3, dev)
    extra["layer_encode"] = dict(us=le["us_per_encode"], dense_bytes=le["dense_bytes"], shapes=le["shapes"])
    log(f"[bench] layer_encode (gate-like + down-like stacks, one prepare_many): {extra['layer_encode']}")
    for indexed, gate_only in ((True, False), (False, False), (True, True)):
        key = ("routed_gate" if gate_only else "routed_paired") + ("" if indexed else "_two_pass")
        log(f"[bench] {key}")
        rr = bench_routed(mwd, torch, ev, workloads, min(args.steps, 2000), args.warmup, dev, indexed,
                          gate_only=gate_only)
        extra[key] = dict(us=round(rr["step_ms"] * 1e3, 2), event_us=round(rr["event_ms"] * 1e3, 3),
                          gbps=round(rr["bytes"] / (rr["step_ms"] * 1e-3) / 1e9, 1),
                          warm_us=round(rr["warm_ms"] * 1e3, 2), flushed_us=round(rr["flushed_ms"] * 1e3, 2),
                          bytes=round(rr["bytes"]), index_bytes=round(rr["index_bytes"]),
                          active=rr["active"], sets=rr["sets"])
        log(f"[bench] {key}: {extra[key]}")
    gspec, dspec = workloads.ROUTED.stacks
    g = mwd.prepare(gspec.generate(), gspec.fmt).to(dev)
    d = mwd.prepare(dspec.generate(), dspec.fmt).to(dev)
    es_t = torch.from_numpy(workloads.ROUTED.expert_start()).to(dev)
    groups = mwd.decode_traced(g, torch.empty(g.dense_bytes, dtype=torch.uint8, device=dev), d,
                               torch.empty(d.dense_bytes, dtype=torch.uint8, device=dev), es_t).shape[0]
    torch.cuda.synchronize()
    extra["launch_floors"] = launch_floors(torch, ev, dev, groups)
    log(f"[bench] launch floors: {extra['launch_floors']}")
    extra["host_cost"] = host_cost(mwd, torch, dev, g, d, es_t)
    log(f"[bench] host cost per call: {extra['host_cost']}")
    spec = workloads.ROUTED
    rs = routed_sets(workloads, gspec.E, spec.n_active, spec.max_tokens, spec.seed + 100, 64)
    extra["routed_trace"] = trace_routed(mwd, torch, dev, g, d, rs)
    log(f"[bench] routed paired decode, per-step timestamps: {extra['routed_trace']}")
    del g, d
    torch.cuda.empty_cache()
    return extra


if __name__ == "__main__":
    main()
