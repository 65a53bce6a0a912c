"""Decode-step benchmark on one GPU: Whisper-large-v2-shaped greedy decoding
(the headline), with speculative verification, beam search and the GQA LM as
sub-records of the same line.

Headline step = for each of the 32 decoder layers: append the new token's K/V
to the self cache and attend the token's query over it (decode_step_self: the
append and the self attention in one launch; --unfused: kv_append then
decode_attn_self), then cross attention over the 1500-frame cache built once
before timing (decode_attn_cross). B=1, 20 heads of 64, fp16 storage, fp32
accumulation. One captured graph per step.

The timed region replays exactly --steps step graphs whose self lengths are
spread evenly over the whole 1..448 sweep: step i runs at length
floor((i + 1/2) * 448 / steps) + 1, so --steps 448 is the sweep itself and
fewer steps are an even sample of it. The line names every length timed.

Prints one JSON line. `value` is decode steps/s over the timed steps (inputs
resident in HBM). Also: effective KV GB/s and its fraction of the 8 TB/s HBM
peak, a full-sweep replay beside the timed region, the dominant kernel's
roofline (cross attention, HIP events on its stream), the attainable read of
the same bytes, cold (Infinity-Cache-evicted) figures, the CPU oracle at one
thread and on every host core, and `configs`: verification of 5 drafts, beam
search with 5 beams and the GQA LM (prefill + decode), each with its own
steps/s and dominant-kernel roofline.

    python bench.py [--gpus 1] [--steps 448] [--warmup 64] [--no-cpu] [--headline-only]
    python bench.py --workload verify|beam|gqa|ragged|specloop|prefill   (one line each)
    python bench.py --workload kernels   (a few eager launches of each hot kernel,
                                          for hardware-counter runs)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
LAYERS, H, D, S_MAX, FRAMES = 32, 20, 64, 448, 1500
ROW_BYTES = H * D * 2                      # one position of one layer, K or V, fp16
CROSS_BYTES = 2 * FRAMES * ROW_BYTES       # K+V read by one cross-attention launch
METRIC = "decode-attn steps/s + effective KV GB/s (% HBM peak), large-v2 shape, 1 GPU"
WORKLOAD = ("whisper-large-v2 greedy decode step: 32 layers x [append T=1 + self attention "
            "N=1 over len 1..448, cross attention over 1500 frames], B1, 20 heads x 64, fp16 "
            "storage / fp32 accumulate")
KERNEL_SOURCES = ["kv_cached_decode_amd/csrc/kvd_attn.hip", "kv_cached_decode_amd/csrc/kvd_attn_common.hpp",
                  "kv_cached_decode_amd/csrc/kvd_device.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_cross_attention.json")


def log(msg: str):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def kv_bytes_per_step(L: int) -> int:
    """Algorithmic KV bytes of one step at self length L (after the append):
    self K+V read, cross K+V read, new K+V written, over every layer."""
    return LAYERS * (2 * L * ROW_BYTES + CROSS_BYTES + 2 * ROW_BYTES)


def sweep_sample(steps: int, length: int = S_MAX) -> list[int]:
    """Step indices (0-based; the self length is index + 1) spread evenly
    over the sweep 0 .. length-1: index i is floor((i + 1/2) * length /
    steps). steps == length gives every index once, in order."""
    return [int((i + 0.5) * length / steps) for i in range(steps)]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per cross-attention launch from the committed rocprofv3
    counter runs, if they were taken on the current kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def roof(nbytes: float, seconds: float, what: str) -> dict:
    """HBM roofline record of one kernel: algorithmic bytes per launch over
    its time per launch."""
    gbps = nbytes / seconds / 1e9
    return {"bound": "hbm", "kernel": what, "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "bytes_per_launch": int(nbytes),
            "avg_launch_us": round(seconds * 1e6, 3)}


class Engine:
    """Device state of the headline: caches, per-step inputs, outputs."""

    def __init__(self, torch, kb, I):
        self.torch, self.kb = torch, kb
        w = I.WHISPER_GREEDY
        self.w = w
        dev = "cuda"
        self.scale = w.attn_scale
        self.self_c, self.cross_c = [], []
        self.k_new, self.v_new, self.q_self, self.q_cross = [], [], [], []
        g = np.random.default_rng([w.seed, 77])
        for l in range(LAYERS):
            k_all, v_all = I.self_kv(w, l)                          # [1, 20, 448, 64]
            # token-major so that token t's [1, 20, 1, 64] rows are contiguous
            self.k_new.append(torch.from_numpy(np.ascontiguousarray(
                k_all.transpose(2, 0, 1, 3)[:, :, :, None, :])).to(dev))
            self.v_new.append(torch.from_numpy(np.ascontiguousarray(
                v_all.transpose(2, 0, 1, 3)[:, :, :, None, :])).to(dev))
            xk, xv = I.cross_kv(w, l)
            xc = kb.Cache(1, H, FRAMES, torch.float16, dev)
            kb.kv_append(xc, torch.from_numpy(xk).to(dev), torch.from_numpy(xv).to(dev), 0)
            self.cross_c.append(xc)
            self.self_c.append(kb.Cache(1, H, S_MAX, torch.float16, dev))
            qs = I.to_storage(g.standard_normal((S_MAX, 1, H, 1, D), dtype=np.float32) / 8, "f16")
            qx = I.to_storage(g.standard_normal((S_MAX, 1, H, 1, D), dtype=np.float32) / 8, "f16")
            self.q_self.append(torch.from_numpy(qs).to(dev))
            self.q_cross.append(torch.from_numpy(qx).to(dev))
        self.out_self = [torch.empty((1, H, 1, D), dtype=torch.float32, device=dev) for _ in range(LAYERS)]
        self.out_cross = [torch.empty((1, H, 1, D), dtype=torch.float32, device=dev) for _ in range(LAYERS)]
        self.ws = kb.workspace(max(kb.attn_workspace_bytes(1, H, 1, S_MAX),
                                   kb.attn_workspace_bytes(1, H, 1, FRAMES)), dev)
        torch.cuda.synchronize()

    def step(self, s: int, fused: bool = True):
        """Decode step s: the self cache grows to length s + 1. Fused: the
        append runs inside the self-attention launch (decode_step_self);
        otherwise kv_append then decode_attn_self."""
        kb = self.kb
        L = s + 1
        for l in range(LAYERS):
            if fused:
                kb.decode_step_self(self.q_self[l][s], self.k_new[l][s], self.v_new[l][s],
                                    self.self_c[l], L, self.scale, out=self.out_self[l], ws=self.ws)
            else:
                kb.kv_append(self.self_c[l], self.k_new[l][s], self.v_new[l][s], s)
                kb.decode_attn_self(self.q_self[l][s], self.self_c[l], L, self.scale,
                                    out=self.out_self[l], ws=self.ws)
            kb.decode_attn_cross(self.q_cross[l][s], self.cross_c[l], FRAMES, self.scale,
                                 out=self.out_cross[l], ws=self.ws)

    def cross(self, l: int, s: int):
        self.kb.decode_attn_cross(self.q_cross[l][s], self.cross_c[l], FRAMES, self.scale,
                                  out=self.out_cross[l], ws=self.ws)


def _graph_steps(torch, fn, steps):
    """One captured graph per step index."""
    graphs = []
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for s in steps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                fn(s)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    return graphs


def _time_graphs(torch, graphs, reps):
    """Seconds per graph, replaying the list `reps` times back to back."""
    for g in graphs[: min(len(graphs), 16)]:
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        for g in graphs:
            g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / (reps * len(graphs))


def _event_durations(torch, kb, calls):
    """Mean kernel duration of calls() (each makes exactly one launch), with
    HIP events recorded at kernel begin and end on the launch stream."""
    stream = torch.cuda.current_stream()
    pairs = []
    for fn in calls:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)   # creates the events
        b.record(stream)
        kb.time_next_launch(a, b)
        fn()
        pairs.append((a, b))
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in pairs])) * 1e-3


def _kernel_us(torch, kb, launch, n=64):
    """Mean kernel duration of `launch(i)` in microseconds (HIP events at
    kernel begin / end), over n launches."""
    return _event_durations(torch, kb, [lambda i=i: launch(i) for i in range(n)]) * 1e6


# GPU clock cycles (about 4 ms at 2.3 GHz) the stream spins before a timed
# region whose launches the host queues one by one
GPU_QUEUE_SLEEP_CYCLES = 10_000_000


def _graph_period(torch, calls, reps: int = 20):
    """Seconds per call when calls() run back to back inside one captured
    graph (as in a decode step); HIP events on the replay stream."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for fn in calls:   # warm: plans, code objects
            fn()
        with torch.cuda.graph(g, stream=stream):
            for fn in calls:
                fn()
    torch.cuda.current_stream().wait_stream(stream)
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    # the GPU spins (outside the timed region) while the host queues every
    # replay, so that no replay waits for the host: timed replays run back
    # to back (without it the beam workload's cross period read 15 us
    # against 6.7 on the same kernel). Three such rounds, the fastest kept:
    # a round the host still fell behind in (19.7 us once, in the full run's
    # beam record) is not a period of the kernels.
    best = None
    for _ in range(3):
        torch.cuda._sleep(GPU_QUEUE_SLEEP_CYCLES)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b) * 1e-3 / (reps * len(calls))
        best = t if best is None else min(best, t)
    return best


def time_cross_kernel(torch, kb, eng: Engine, reps: int = 8):
    """Cross-attention kernel: mean duration (HIP events at kernel begin and
    end on the launch stream, kvd_time_next_launch) over launches that cycle
    through the 32 layers, so none re-reads the cache the previous one read;
    and the period of back-to-back launches over the 32 layers in a graph."""
    calls = [lambda l=l, r=r: eng.cross(l, (r * 37 + l) % S_MAX)
             for r in range(reps) for l in range(LAYERS)]
    dur = _event_durations(torch, kb, calls)
    period = _graph_period(torch, [lambda l=l: eng.cross(l, l) for l in range(LAYERS)])
    return dur, period


PROBE_SHAPES = [(4, 0), (8, 0), (16, 0), (1, 0), (2, 0), (4, 1024), (8, 1024), (16, 256), (4, 256)]


def attainable(torch, kb, eng: Engine, reps: int = 8):
    """The same bytes read by a plain streaming-read kernel (kvd_read_probe_ex),
    timed the same way: K and V of the 32 layers' cross caches in turn, for
    several loads-in-flight / grid shapes (the best is the yardstick); plus
    the rate of the best shape at other sizes (working sets cycled through a
    1 GiB buffer)."""
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    half = CROSS_BYTES // 2

    def probe(l, u, nb):
        kb.read_probe(eng.cross_c[l].k, eng.cross_c[l].v, half, sink, unroll=u, blocks=nb)

    shapes = {}
    for u, nb in PROBE_SHAPES:
        period = _graph_period(torch, [lambda l=l: probe(l, u, nb) for l in range(LAYERS)])
        shapes[f"unroll{u}_blocks{nb or 'auto'}"] = round(period * 1e6, 3)
    best = min(shapes, key=shapes.get)
    bu, bnb = next((u, nb) for u, nb in PROBE_SHAPES if f"unroll{u}_blocks{nb or 'auto'}" == best)
    dur = _event_durations(torch, kb, [lambda l=l: probe(l, bu, bnb)
                                       for _ in range(reps) for l in range(LAYERS)])
    period = shapes[best] * 1e-6
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    curve = {}
    for mb in (1, 2, 4, 8, 16, 64, 512):
        n = mb << 20
        regions = max(1, min(32, (1 << 30) // n))
        best_t = None
        for u, nb in ((bu, bnb), (4, 0), (8, 0), (16, 0)):
            calls = [lambda i=i: kb.read_probe(buf[i * n:(i + 1) * n], None, n, sink, unroll=u, blocks=nb)
                     for _ in range(2) for i in range(regions)]
            t = _event_durations(torch, kb, calls)
            best_t = t if best_t is None else min(best_t, t)
        curve[f"{mb}MB"] = round(n / best_t / 1e9, 1)
    del buf
    return {"best_shape": best, "period_us_by_shape": shapes, "period": period, "alone": dur,
            "curve": curve, "best": (bu, bnb)}


def cold_numbers(torch, kb, eng: Engine, graphs, probe_shape, every: int = 7):
    """The same work with the 256 MB Infinity Cache evicted first: a 512 MB
    device write (outside the timed region) before each sampled decode step
    (one graph replay, HIP events around it on the replay stream) and before
    each cross-attention and read-probe launch (events at kernel begin and
    end)."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sampled = list(range(0, S_MAX, every))
    pairs = []
    for i, s in enumerate(sampled):
        flush.fill_(i & 0xFF)
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        graphs[s].replay()
        e.record(stream)
        pairs.append((a, e))
    torch.cuda.synchronize()
    step_s = float(np.mean([a.elapsed_time(e) for a, e in pairs])) * 1e-3
    kv = float(np.mean([kv_bytes_per_step(s + 1) for s in sampled]))
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    half = CROSS_BYTES // 2
    u, nb = probe_shape

    def flushed(fn, i):
        flush.fill_(i & 0xFF)
        fn()
    cross = _event_durations(torch, kb, [lambda l=l: flushed(lambda: eng.cross(l, l), l)
                                         for _ in range(2) for l in range(LAYERS)])
    probe = _event_durations(torch, kb, [lambda l=l: flushed(
        lambda: kb.read_probe(eng.cross_c[l].k, eng.cross_c[l].v, half, sink, unroll=u, blocks=nb), l)
        for _ in range(2) for l in range(LAYERS)])
    del flush
    return {"what": "512 MB written before each timed unit (outside it), evicting the 256 MB "
                    "Infinity Cache",
            "steps_per_s": round(1 / step_s, 2), "ms_per_step": round(step_s * 1e3, 5),
            "effective_kv_gbps": round(kv / step_s / 1e9, 1),
            "hbm_peak_frac": round(kv / step_s / 1e9 / HBM_PEAK_GBPS, 4),
            "sample": f"{len(sampled)} decode steps (every {every}th length of the 1..448 sweep), "
                      "each timed alone from its graph launch",
            "cross_kernel_us": round(cross * 1e6, 3),
            "cross_gbps": round(CROSS_BYTES / cross / 1e9, 1),
            "cross_frac": round(CROSS_BYTES / cross / 1e9 / HBM_PEAK_GBPS, 4),
            "probe_us": round(probe * 1e6, 3),
            "probe_gbps": round(CROSS_BYTES / probe / 1e9, 1),
            "cross_frac_of_attainable": round(probe / cross, 4)}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on the host cores.
# ---------------------------------------------------------------------------


def _oracle_state():
    """Cross caches of the 32 layers and every layer's self K/V, in the
    oracle's own containers."""
    import oracle as O
    from kv_cached_decode_amd import inputs as I
    w = I.WHISPER_GREEDY
    xcs = []
    for l in range(LAYERS):
        xk, xv = I.cross_kv(w, l)
        c = O.ConcatCache(1, H, D, "f16")
        c.set_once(xk, xv)
        xcs.append(c)
    kv = [I.self_kv(w, l) for l in range(LAYERS)]
    return xcs, kv


def _oracle_step(xcs, kv, L):
    """One full 32-layer oracle decode step at self length L; returns its
    seconds (the cache and query set-up is outside the timing)."""
    import oracle as O
    from kv_cached_decode_amd import inputs as I
    w = I.WHISPER_GREEDY
    caches = []
    for l in range(LAYERS):
        c = O.ConcatCache(1, H, D, "f16")
        c.append(kv[l][0][:, :, :L - 1], kv[l][1][:, :, :L - 1])
        caches.append(c)
    q = [I.queries(w, l, L) for l in range(LAYERS)]
    qx = [I.queries(w, l, L, cross=True) for l in range(LAYERS)]
    kn = [kv[l][0][:, :, L - 1:L] for l in range(LAYERS)]
    vn = [kv[l][1][:, :, L - 1:L] for l in range(LAYERS)]
    t0 = time.perf_counter()
    O.decode_step(q, qx, kn, vn, caches, xcs, w.attn_scale)
    return time.perf_counter() - t0


CPU_LENGTHS = [1, 112, 224, 336, 448, 56, 168, 280, 392, 28, 140, 252, 364, 420]


def _cpu_worker(wid, nworkers, seconds, barrier, results):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        xcs, kv = _oracle_state()
        barrier.wait()
        t0 = time.perf_counter()
        busy, used = 0.0, []
        n = wid
        while time.perf_counter() - t0 < seconds:
            L = CPU_LENGTHS[n % len(CPU_LENGTHS)]
            busy += _oracle_step(xcs, kv, L)
            used.append(L)
            n += nworkers
        results.put((wid, used, busy, time.perf_counter() - t0))


def cpu_baseline(seconds: float = 10.0) -> dict:
    """The CPU oracle (numpy, float64) on a bounded sample of the headline's
    steps: full 32-layer decode steps at lengths spread over 1..448.

    Two legs, both before the GPU is touched: one process with BLAS held to
    one thread, then one single-threaded oracle process per host core (the
    box's CPU share, at most 16), forked after a barrier and run for the
    same time; their steps add up (each step is independent work)."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    model = ""
    try:
        info = {}
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ":" in ln:
                    k, v = (x.strip() for x in ln.split(":", 1))
                    if k in ("model name", "cpu family", "model", "stepping", "cache size") and k not in info:
                        info[k] = v
        model = (f"{info.get('model name', '')} (family {info.get('cpu family', '?')}, model "
                 f"{info.get('model', '?')}, stepping {info.get('stepping', '?')}, cache "
                 f"{info.get('cache size', '?')})")
    except OSError:
        pass
    ncpu = len(os.sched_getaffinity(0))
    log("CPU oracle, one thread")
    with threadpool_limits(limits=1):
        xcs, kv = _oracle_state()
        spent, used, n = 0.0, [], 0
        while spent < seconds:
            L = CPU_LENGTHS[n % len(CPU_LENGTHS)]
            spent += _oracle_step(xcs, kv, L)
            used.append(L)
            n += 1
    single = len(used) / spent
    del xcs, kv
    workers = max(1, min(16, ncpu))
    log(f"CPU oracle, {workers} processes")
    ctx = mp.get_context("fork")
    barrier, results = ctx.Barrier(workers), ctx.Queue()
    procs = [ctx.Process(target=_cpu_worker, args=(w, workers, seconds, barrier, results))
             for w in range(workers)]
    for p in procs:
        p.start()
    got = [results.get() for _ in procs]
    for p in procs:
        p.join()
    steps = sum(len(u) for _, u, _, _ in got)
    wall = max(t for _, _, _, t in got)
    lengths = sorted({L for _, u, _, _ in got for L in u})
    return {"value": round(steps / wall, 3), "unit": "steps/s", "cores": workers, "kind": "oracle",
            "sample": (f"{steps} full 32-layer decode steps at self lengths {lengths}, "
                       f"{workers} single-threaded oracle processes (numpy float64) for "
                       f"{wall:.1f} s wall"),
            "single_thread": {"value": round(single, 3), "unit": "steps/s", "cores": 1,
                              "sample": f"{len(used)} steps at lengths {sorted(set(used))}, "
                                        f"{spent:.1f} s, BLAS held to one thread"},
            "cpu_model": model, "host_cpus_visible": ncpu}


# ---------------------------------------------------------------------------
# The headline.
# ---------------------------------------------------------------------------


def headline(torch, kb, I, args) -> dict:
    log("building device state")
    eng = Engine(torch, kb, I)
    fused = not args.unfused
    log("capturing 448 step graphs")
    graphs = _graph_steps(torch, lambda s: eng.step(s, fused), range(S_MAX))

    # warmup: whole sweeps (every cache row gets written) until the GPU has
    # been busy for 2 s (after the idle CPU-baseline legs its clocks need that
    # long to come back: a 20-step region timed right after one sweep ran 6%
    # slower than the same steps later), then --warmup more steps spread over
    # the sweep
    t_warm = time.perf_counter()
    while True:
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t_warm > 2.0:
            break
    for s in sweep_sample(args.warmup) if args.warmup > 0 else []:
        graphs[s].replay()
    torch.cuda.synchronize()

    # timed region: exactly --steps steps, lengths spread over 1..448 (HIP
    # events on the replay stream beside the host clock: the GPU's own time
    # for the same replays)
    seq = sweep_sample(args.steps)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for s in seq:
        graphs[s].replay()
    ev1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gpu_elapsed = ev0.elapsed_time(ev1) * 1e-3
    kv_bytes = sum(kv_bytes_per_step(s + 1) for s in seq)

    # beside it: the whole sweep, once
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    sweep_s = time.perf_counter() - t1
    sweep_kv = sum(kv_bytes_per_step(s + 1) for s in range(S_MAX))

    eager = None
    if args.eager:
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for s in seq:
            eng.step(s, fused)
        torch.cuda.synchronize()
        eager = args.steps / (time.perf_counter() - t2)

    log("timing the cross-attention kernel and the read probe")
    k_avg, k_period = time_cross_kernel(torch, kb, eng)
    att = attainable(torch, kb, eng)
    cold = cold_numbers(torch, kb, eng, graphs, att["best"])
    del graphs

    steps_per_s = args.steps / elapsed
    gbps = kv_bytes / elapsed / 1e9
    r = roof(CROSS_BYTES, k_period, "decode_attn_cross (attn_kernel<f16, 1 row, 4 waves>, 12 splits x 20 heads)")
    r["traffic"] = measured_traffic()
    r["timing"] = ("per-launch time of 32 back-to-back launches (one per layer) in a hipGraph, "
                   "HIP events on the replay stream, 20 replays, fastest of 3 rounds; the same kernel launched alone, "
                   f"HIP events at its begin/end (hipExtLaunchKernel, 256 launches): {k_avg * 1e6:.3f} us")
    lengths = [s + 1 for s in seq]
    return {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "layers": LAYERS, "batch": 1, "heads": H,
                   "head_dim": D, "cross_frames": FRAMES,
                   "self_len_timed": (f"{len(lengths)} steps at lengths spread evenly over 1..448: "
                                      + ",".join(map(str, lengths))),
                   "launch": ("one hipGraph per step, "
                              + ("64 kernels per step (append fused into self attention)"
                                 if fused else "96 kernels per step"))},
        "effective_kv_gbps": round(gbps, 1),
        "hbm_peak_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "timed_region_gpu_ms": round(gpu_elapsed * 1e3, 4),
        "full_sweep": {"steps_per_s": round(S_MAX / sweep_s, 2),
                       "ms_per_step": round(sweep_s / S_MAX * 1e3, 5),
                       "effective_kv_gbps": round(sweep_kv / sweep_s / 1e9, 1),
                       "what": "all 448 step graphs (lengths 1..448) replayed once, after the timed region"},
        "roofline": r,
        "attainable": {"probe": "kvd_read_probe_ex: plain streaming read of the same K/V bytes in one "
                                "launch, timed the same way, over loads-in-flight / grid shapes",
                       "best_shape": att["best_shape"],
                       "avg_launch_us": round(att["period"] * 1e6, 3),
                       "gbps": round(CROSS_BYTES / att["period"] / 1e9, 1),
                       "alone_launch_us": round(att["alone"] * 1e6, 3),
                       "period_us_by_shape": att["period_us_by_shape"],
                       "cross_frac_of_attainable": round(att["period"] / k_period, 4),
                       "probe_gbps_by_size_alone": att["curve"]},
        "cold": cold,
        **({"eager_steps_per_s": round(eager, 2)} if eager is not None else {}),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=448)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="seconds of oracle work per CPU-baseline leg")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the verify / beam / GQA sub-records")
    ap.add_argument("--eager", action="store_true", help="also time eager (no graph) launches")
    ap.add_argument("--workload", default="greedy",
                    choices=["greedy", "verify", "beam", "gqa", "ragged", "specloop", "prefill", "kernels"],
                    help="greedy (the headline line) or one further workload alone")
    ap.add_argument("--unfused", action="store_true",
                    help="separate kv_append and decode_attn_self launches (96 per step)")
    ap.add_argument("--reps", type=int, default=4, help="replays of each sub-record's graphs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the decode step runs on a single GPU)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        print("--steps must be at least 1", file=sys.stderr)
        sys.exit(2)

    # the CPU legs fork worker processes, so they run before the GPU is touched
    cpu = None
    if args.workload == "greedy" and not args.no_cpu:
        cpu = cpu_baseline(args.cpu_seconds)

    import torch
    from kv_cached_decode_amd import binding as kb
    from kv_cached_decode_amd import inputs as I
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kb.lib()

    if args.workload != "greedy":
        fn = {"verify": workload_verify, "beam": workload_beam, "gqa": workload_gqa,
              "ragged": workload_ragged, "specloop": workload_specloop,
              "prefill": workload_prefill, "kernels": workload_kernels}[args.workload]
        line = fn(torch, kb, args.reps)
        line.update({"n_gpus": 1, "data": "synthetic", "higher_is_better": True})
        print(json.dumps(line), flush=True)
        return

    line = headline(torch, kb, I, args)
    if not args.headline_only:
        configs = {}
        for name, fn in (("verify_n5", workload_verify), ("beam5", workload_beam),
                         ("gqa_prefill_decode", workload_gqa)):
            log(f"sub-record {name}")
            configs[name] = fn(torch, kb, args.reps)
            torch.cuda.empty_cache()
        line["configs"] = configs
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# Further workloads: sub-records of the default line, or one line each with
# --workload. Inputs are seeded torch draws on the device; the parity tests
# check these shapes against the oracle.
# ---------------------------------------------------------------------------


def workload_verify(torch, kb, reps):
    """Speculative verification at the large-v2 shape: per step, 32 layers of
    [append 5 draft rows + self attention of 5 causal queries, cross attention
    of 5 queries over 1500 frames], then verify_accept over [1, 5, 51865];
    one graph per length before the step, 64, 128, ..., 443."""
    g = torch.Generator(device="cuda").manual_seed(3)
    rn = lambda *sh: (torch.randn(*sh, generator=g, device="cuda") / 8).half()
    N, V = 5, 51865
    self_c, cross_c = [], []
    for _ in range(LAYERS):
        c = kb.Cache(1, H, S_MAX, torch.float16)
        c.k.copy_(rn(1, H, S_MAX, D)); c.v.copy_(rn(1, H, S_MAX, D))
        self_c.append(c)
        x = kb.Cache(1, H, FRAMES, torch.float16)
        x.k.copy_(rn(1, H, FRAMES, D)); x.v.copy_(rn(1, H, FRAMES, D))
        cross_c.append(x)
    q, qx = rn(LAYERS, 1, H, N, D), rn(LAYERS, 1, H, N, D)
    kn, vn = rn(LAYERS, 1, H, N, D), rn(LAYERS, 1, H, N, D)
    out = torch.empty((LAYERS, 1, H, N, D), dtype=torch.float32, device="cuda")
    outx = torch.empty_like(out)
    logits = torch.randn(1, N, V, generator=g, device="cuda") * 2
    draft = torch.randint(0, V, (1, N), generator=g, device="cuda", dtype=torch.int32)
    acc = torch.empty(1, dtype=torch.int32, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = kb.workspace(max(kb.attn_workspace_bytes(1, H, N, FRAMES), kb.verify_workspace_bytes(1, N, V)))
    lens = [64, 128, 192, 256, 320, 384, 443]

    def step(i):
        L = lens[i] + N
        for l in range(LAYERS):
            kb.decode_step_self(q[l], kn[l], vn[l], self_c[l], L, 1 / 8, out=out[l], ws=ws)
            kb.decode_attn_cross(qx[l], cross_c[l], FRAMES, 1 / 8, out=outx[l], ws=ws)
        kb.verify_accept(logits, draft, ws=ws, accept_len=acc, next_token=nxt)

    graphs = _graph_steps(torch, step, range(len(lens)))
    sec = _time_graphs(torch, graphs, reps * 8)
    del graphs
    kv = sum(LAYERS * (2 * (L + N) * ROW_BYTES + CROSS_BYTES + 2 * N * ROW_BYTES) for L in lens) / len(lens)
    cross_period = _graph_period(torch, [lambda l=l: kb.decode_attn_cross(
        qx[l], cross_c[l], FRAMES, 1 / 8, out=outx[l], ws=ws) for l in range(LAYERS)])
    self_period = _graph_period(torch, [lambda l=l: kb.decode_step_self(
        q[l], kn[l], vn[l], self_c[l], 448, 1 / 8, out=out[l], ws=ws) for l in range(LAYERS)])
    self_us = _kernel_us(torch, kb, lambda i: kb.decode_step_self(q[i % LAYERS], kn[i % LAYERS], vn[i % LAYERS], self_c[i % LAYERS], 448, 1 / 8, out=out[0], ws=ws))
    cross_us = _kernel_us(torch, kb, lambda i: kb.decode_attn_cross(qx[i % LAYERS], cross_c[i % LAYERS], FRAMES, 1 / 8, out=outx[0], ws=ws))
    verify_us = _kernel_us(torch, kb, lambda i: kb.verify_accept(logits, draft, ws=ws, accept_len=acc, next_token=nxt))
    # the same with the logit filters: 90 suppressed tokens on every row, blank
    # and end-of-text on the first row
    sup = kb.token_bitmap(range(50358, 50448), V)
    first = kb.token_bitmap([220, 50256], V)
    masked_us = _kernel_us(torch, kb, lambda i: kb.verify_accept_masked(
        logits, draft, sup, first, ws=ws, accept_len=acc, next_token=nxt))
    p = [0.75 ** k * 0.25 for k in range(5)] + [0.75 ** 5]
    tokens = sum(pk * t for pk, t in zip(p, [1, 2, 3, 4, 5, 5]))
    return {"metric": "speculative verify steps/s (N=5 drafts), large-v2 shape, 1 GPU",
            "value": round(1 / sec, 2), "unit": "verify steps/s", "ms_per_step": round(sec * 1e3, 4),
            "dtype": "f16",
            "effective_kv_gbps": round(kv / sec / 1e9, 1),
            "hbm_peak_frac": round(kv / sec / 1e9 / HBM_PEAK_GBPS, 4),
            "tokens_per_s_at_p075": round(tokens / sec, 1),
            "roofline": roof(CROSS_BYTES, cross_period,
                             "decode_attn_cross, 5 query rows per head (matrix-core tile), "
                             "32 back-to-back launches in a graph"),
            "self_step_len453_roofline": roof(2 * 448 * ROW_BYTES, self_period,
                                              "decode_step_self N=5 at len 448 (matrix-core tile), "
                                              "32 back-to-back launches in a graph"),
            "kernels_us_alone": {"step_self_N5_len448": round(self_us, 3),
                                 "cross_N5": round(cross_us, 3), "verify_accept_V51865": round(verify_us, 3),
                                 "verify_accept_masked_V51865": round(masked_us, 3)},
            "config": {"workload": "whisper-large-v2 verify: 32 layers x [append 5 + self N=5, cross N=5 "
                                   "over 1500] + verify_accept [1, 5, 51865]",
                       "len_before": lens, "timed": f"{len(lens)} step graphs x {reps * 8} replays"}}


def workload_ragged(torch, kb, reps):
    """Batched speculative verification with ragged rows at the large-v2
    shape: 4 sequences, each with its own self and cross caches and its own
    length (drawn per step in [32, 443]); per step, 32 layers of [append 5
    draft rows per sequence at its own length + self attention of its 5 causal
    queries (one ragged launch), cross attention of 5 queries per sequence over
    its 1500 frames], then verify_accept over [4, 5, 51865]."""
    g = torch.Generator(device="cuda").manual_seed(6)
    rn = lambda *sh: (torch.randn(*sh, generator=g, device="cuda") / 8).half()
    B, N, V, steps = 4, 5, 51865, 7
    self_c, cross_c = [], []
    for _ in range(LAYERS):
        c = kb.Cache(B, H, S_MAX, torch.float16)
        c.k.copy_(rn(B, H, S_MAX, D)); c.v.copy_(rn(B, H, S_MAX, D))
        self_c.append(c)
        x = kb.Cache(B, H, FRAMES, torch.float16)
        x.k.copy_(rn(B, H, FRAMES, D)); x.v.copy_(rn(B, H, FRAMES, D))
        cross_c.append(x)
    q, qx = rn(LAYERS, B, H, N, D), rn(LAYERS, B, H, N, D)
    kn, vn = rn(LAYERS, B, H, N, D), rn(LAYERS, B, H, N, D)
    out = torch.empty((LAYERS, B, H, N, D), dtype=torch.float32, device="cuda")
    outx = torch.empty_like(out)
    logits = torch.randn(B, N, V, generator=g, device="cuda") * 2
    draft = torch.randint(0, V, (B, N), generator=g, device="cuda", dtype=torch.int32)
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = kb.workspace(max(kb.attn_workspace_bytes(B, H, N, FRAMES), kb.verify_workspace_bytes(B, N, V)))
    before = np.random.default_rng(6).integers(32, 444, size=(steps, B))
    lens = [torch.tensor(before[i] + N, dtype=torch.int32, device="cuda") for i in range(steps)]

    def step(i):
        for l in range(LAYERS):
            kb.decode_step_self_ragged(q[l], kn[l], vn[l], self_c[l], lens[i], S_MAX, 1 / 8,
                                       out=out[l], ws=ws)
            kb.decode_attn_cross(qx[l], cross_c[l], FRAMES, 1 / 8, out=outx[l], ws=ws)
        kb.verify_accept(logits, draft, ws=ws, accept_len=acc, next_token=nxt)

    graphs = _graph_steps(torch, step, range(steps))
    sec = _time_graphs(torch, graphs, reps * 8)
    kv = sum(LAYERS * (2 * (int(L) + N) * ROW_BYTES + CROSS_BYTES + 2 * N * ROW_BYTES)
             for row in before for L in row) / steps
    self_us = _kernel_us(torch, kb, lambda i: kb.decode_step_self_ragged(
        q[i % LAYERS], kn[i % LAYERS], vn[i % LAYERS], self_c[i % LAYERS], lens[i % steps], S_MAX,
        1 / 8, out=out[0], ws=ws))
    cross_us = _kernel_us(torch, kb, lambda i: kb.decode_attn_cross(
        qx[i % LAYERS], cross_c[i % LAYERS], FRAMES, 1 / 8, out=outx[0], ws=ws))
    verify_us = _kernel_us(torch, kb, lambda i: kb.verify_accept(
        logits, draft, ws=ws, accept_len=acc, next_token=nxt))
    return {"metric": "ragged batched verify steps/s (4 sequences x N=5 drafts), large-v2 shape, 1 GPU",
            "value": round(1 / sec, 2), "unit": "verify steps/s", "ms_per_step": round(sec * 1e3, 4),
            "dtype": "f16",
            "sequence_steps_per_s": round(B / sec, 1),
            "effective_kv_gbps": round(kv / sec / 1e9, 1),
            "hbm_peak_frac": round(kv / sec / 1e9 / HBM_PEAK_GBPS, 4),
            "kernels_us_alone": {"step_self_ragged_B4_N5": round(self_us, 3),
                                 "cross_B4_N5": round(cross_us, 3),
                                 "verify_accept_B4_V51865": round(verify_us, 3)},
            "config": {"workload": "whisper-large-v2 ragged verify: 4 sequences, lengths before the "
                                   "step drawn in [32, 443] per step and sequence; 32 layers x "
                                   "[append 5 + self N=5 (one ragged launch), cross N=5 over each "
                                   "sequence's 1500 frames] + verify_accept [4, 5, 51865]"}}


def workload_specloop(torch, kb, reps):
    """End-to-end speculative decoding at the large-v2 shape with synthetic
    position-indexed models: a 2-layer assistant drafts 5 tokens (5 greedy
    single-token steps + 1 more append), the 32-layer main model verifies 6
    rows in one pass, P moves on the device; against the main model alone
    decoding greedily with the same machinery. Both loops run as captured
    graphs replayed back to back."""
    from kv_cached_decode_amd.specloop import SpecConfig, SpecLoop
    loop = SpecLoop(SpecConfig())
    loop.capture()
    loop.reset()
    loop.replay(4)
    torch.cuda.synchronize()
    spec_s, spec_tok, spec_it = 0.0, 0, 0
    for _ in range(reps):
        loop.reset()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        loop.replay(loop.max_iters)
        torch.cuda.synchronize()
        spec_s += time.perf_counter() - t0
        spec_tok += loop.tokens_emitted()
        spec_it += loop.max_iters
    log_, stream = loop.emitted()
    greedy_ref = loop.LM.argmax(-1).cpu().tolist()
    p0 = loop.cfg.prompt
    matches = stream == greedy_ref[p0:p0 + len(stream)]
    g_s, g_tok = 0.0, 0
    for _ in range(reps):
        loop.reset()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        loop.replay(loop.max_greedy, greedy=True)
        torch.cuda.synchronize()
        g_s += time.perf_counter() - t0
        g_tok += loop.max_greedy
    gstream = loop.greedy_stream()
    matches = matches and gstream[:len(stream)] == stream
    tps, gtps = spec_tok / spec_s, g_tok / g_s
    return {"metric": "speculative decoding tokens/s (2-layer assistant, 5 drafts), large-v2 shape, 1 GPU",
            "value": round(tps, 1), "unit": "tokens/s", "dtype": "f16",
            "greedy_tokens_per_s": round(gtps, 1), "speedup_vs_greedy": round(tps / gtps, 3),
            "tokens_per_iteration": round(spec_tok / spec_it, 3),
            "ms_per_iteration": round(spec_s / spec_it * 1e3, 4),
            "stream_equals_greedy": bool(matches),
            "config": {"workload": "whisper-large-v2 shape, synthetic per-position q/k/v and logits "
                                   "(assistant argmax agrees with the main model's w.p. 0.75); "
                                   f"{loop.max_iters} iterations from a {p0}-token prompt; greedy: "
                                   f"{loop.max_greedy} steps"}}


def _prefill_state(torch, kb, layers=4, seed=8):
    g = torch.Generator(device="cuda").manual_seed(seed)
    B, Hkv, S = 8, 3, 1024
    caches = []
    for _ in range(layers):
        c = kb.Cache(B, Hkv, S, torch.bfloat16)
        c.k.copy_(torch.randn(B, Hkv, S, D, generator=g, device="cuda").bfloat16())
        c.v.copy_(torch.randn(B, Hkv, S, D, generator=g, device="cuda").bfloat16())
        caches.append(c)
    q = torch.randn(layers, B, 9, 512, D, generator=g, device="cuda").bfloat16()
    return caches, q


def prefill_flops(B=8, Hq=9, P=512):
    """QK^T and PV over the causal (query, key) pairs, 2 flops per MAC."""
    return 4 * D * B * Hq * (P * (P + 1) // 2)


def workload_prefill(torch, kb, reps):
    """The GQA prefill attention alone (the prefill tile: 64 query rows per
    workgroup, keys staged through LDS): B8, 9 query / 3 KV heads x 64, bf16,
    rotary base 1e4, 512 causal queries over 512 cached keys, one layer's
    cache per launch."""
    layers, P = 4, 512
    caches, q = _prefill_state(torch, kb, layers)
    out = torch.empty((8, 9, P, D), dtype=torch.float32, device="cuda")
    ws = kb.workspace(kb.attn_workspace_bytes(8, 9, P, P))
    us = _kernel_us(torch, kb, lambda i: kb.decode_attn_self(q[i % layers], caches[i % layers], P,
                                                             0.125, rope_base=1e4, out=out, ws=ws),
                    n=32 * max(1, reps))
    flops = prefill_flops()
    tflops = flops / (us * 1e-6) / 1e12
    return {"metric": "GQA prefill attention TFLOP/s (512 causal queries), 1 GPU", "value": round(tflops, 2),
            "unit": "TFLOP/s", "dtype": "bf16", "kernel_us": round(us, 3),
            "algorithmic_gflop": round(flops / 1e9, 3),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
            "config": {"workload": "GQA prefill attention: B8, Hq9/Hkv3 x 64, bf16, RoPE 1e4, 512 causal "
                                   "queries over 512 keys (one launch per layer's cache)"}}


def workload_beam(torch, kb, reps):
    """Beam search with 5 beams at the large-v2 shape: per step, beam_select
    over [1, 5, 51865] fp32 logits (N(0, 4)) with the running scores the step
    before produced, then 32 layers of [the beam step: each beam's parent rows
    read from one of the layer's two caches and written into the other with
    the new row, plus self attention, in one launch; cross attention over a
    cross cache shared by the beams]; 224 steps. The same steps with an
    in-place kv_reorder before the fused append + attention (one cache per
    layer) are timed beside it."""
    g = torch.Generator(device="cuda").manual_seed(4)
    rn = lambda *sh: (torch.randn(*sh, generator=g, device="cuda") / 8).half()
    B, steps, V, eot = 5, 224, 51865, 50256
    pairs, cross_c = [], []
    for _ in range(LAYERS):
        pr = [kb.Cache(B, H, S_MAX, torch.float16) for _ in range(2)]
        for c in pr:
            c.k.copy_(rn(B, H, S_MAX, D)); c.v.copy_(rn(B, H, S_MAX, D))
        pairs.append(pr)
        x = kb.Cache(1, H, FRAMES, torch.float16)
        x.k.copy_(rn(1, H, FRAMES, D)); x.v.copy_(rn(1, H, FRAMES, D))
        cross_c.append(x)
    q, qx = rn(LAYERS, B, H, 1, D), rn(LAYERS, B, H, 1, D)
    kn, vn = rn(LAYERS, B, H, 1, D), rn(LAYERS, B, H, 1, D)
    logits = torch.randn(steps, 1, B, V, generator=g, device="cuda") * 2
    outs = [kb.beam_select(logits[0], torch.zeros(1, B, device="cuda"), eot) for _ in range(2)]
    for o in outs:
        o["score"].zero_()
    out = torch.empty((LAYERS, B, H, 1, D), dtype=torch.float32, device="cuda")
    outx = torch.empty_like(out)
    ws = kb.workspace(kb.attn_workspace_bytes(B, H, 1, FRAMES))
    wsb = kb.workspace(kb.beam_workspace_bytes(1, B, V))

    def step(s):
        cur, prev = outs[s % 2], outs[(s + 1) % 2]
        kb.beam_select(logits[s], prev["score"], eot, ws=wsb, out=cur)
        parent = cur["parent"][0]
        for l in range(LAYERS):
            src, dst = pairs[l][s % 2], pairs[l][(s + 1) % 2]
            kb.decode_step_self_beams(q[l], kn[l], vn[l], src, dst, parent, s + 1, 1 / 8,
                                      out=out[l], ws=ws)
            kb.decode_attn_cross(qx[l], cross_c[l], FRAMES, 1 / 8, out=outx[l], ws=ws)

    def step_inplace(s):
        cur, prev = outs[s % 2], outs[(s + 1) % 2]
        kb.beam_select(logits[s], prev["score"], eot, ws=wsb, out=cur)
        parent = cur["parent"][0]
        for l in range(LAYERS):
            if s > 0:
                kb.kv_reorder(pairs[l][0], parent, s)
            kb.decode_step_self(q[l], kn[l], vn[l], pairs[l][0], s + 1, 1 / 8, out=out[l], ws=ws)
            kb.decode_attn_cross(qx[l], cross_c[l], FRAMES, 1 / 8, out=outx[l], ws=ws)

    graphs = _graph_steps(torch, step, range(steps))
    # one untimed pass records the parents the scoring chose
    changed = 0
    for s, gr in enumerate(graphs):
        gr.replay()
        changed += int((outs[s % 2]["parent"][0].cpu() != torch.arange(B, dtype=torch.int32)).sum())
    changed /= steps
    sec = _time_graphs(torch, graphs, reps)
    del graphs
    sec_inplace = _time_graphs(torch, _graph_steps(torch, step_inplace, range(steps)), reps)
    # the beam step reads each beam's s parent rows once (for the copy and the
    # attention) and writes them and the new row; cross attention reads the
    # shared cache; scoring reads the logits
    kv = sum(LAYERS * (B * 2 * s * ROW_BYTES * 2 + B * 2 * ROW_BYTES + CROSS_BYTES) + B * V * 4
             for s in range(steps)) / steps
    parent = outs[0]["parent"][0]
    cross_period = _graph_period(torch, [lambda l=l: kb.decode_attn_cross(
        qx[l], cross_c[l], FRAMES, 1 / 8, out=outx[l], ws=ws) for l in range(LAYERS)])
    beam_us = _kernel_us(torch, kb, lambda i: kb.decode_step_self_beams(
        q[i % LAYERS], kn[i % LAYERS], vn[i % LAYERS], pairs[i % LAYERS][0], pairs[i % LAYERS][1],
        parent, 201, 1 / 8, out=out[0], ws=ws))
    reorder_us = _kernel_us(torch, kb, lambda i: kb.kv_reorder(pairs[i % LAYERS][0], parent, 200))
    select_us = _kernel_us(torch, kb, lambda i: kb.beam_select(logits[i % steps], outs[1]["score"], eot,
                                                              ws=wsb, out=outs[0]))
    return {"metric": "beam-search decode steps/s (5 beams), large-v2 shape, 1 GPU",
            "value": round(1 / sec, 2), "unit": "steps/s", "ms_per_step": round(sec * 1e3, 4),
            "dtype": "f16",
            "effective_kv_gbps": round(kv / sec / 1e9, 1),
            "hbm_peak_frac": round(kv / sec / 1e9 / HBM_PEAK_GBPS, 4),
            "roofline": roof(CROSS_BYTES, cross_period,
                             "decode_attn_cross, 5 beam rows sharing one cache (matrix-core tile), "
                             "32 back-to-back launches in a graph"),
            "beams_changed_per_step": round(changed, 2),
            "inplace_reorder_steps_per_s": round(1 / sec_inplace, 2),
            "kernels_us_alone": {"beam_step_len201": round(beam_us, 3),
                                 "kv_reorder_len200": round(reorder_us, 3),
                                 "beam_select_5x51865": round(select_us, 3)},
            "config": {"workload": "whisper-large-v2 beam 5: beam_select [1, 5, 51865] + 32 layers x "
                                   "[beam step: parent rows copied between two caches + append + "
                                   "self attention, one launch; cross shared by beams]; 224 steps",
                       "timed": f"224 step graphs x {reps} replays"}}


def workload_gqa(torch, kb, reps):
    """GQA decoder-only LM: 30 layers, B=8, 9 query / 3 KV heads of 64, bf16,
    RoPE base 10000. Prefill of 512 prompt tokens (append + causal attention of
    512 queries, matrix-core tile), then decode steps from length 513 to 1024."""
    g = torch.Generator(device="cuda").manual_seed(5)
    rn = lambda *sh: torch.randn(*sh, generator=g, device="cuda").bfloat16()
    Lyr, B, Hq, Hk, P, S = 30, 8, 9, 3, 512, 1024
    caches = [kb.Cache(B, Hk, S, torch.bfloat16) for _ in range(Lyr)]
    qp, kp, vp = rn(Lyr, B, Hq, P, D), rn(Lyr, B, Hk, P, D), rn(Lyr, B, Hk, P, D)
    qd, kd, vd = rn(Lyr, B, Hq, 1, D), rn(Lyr, B, Hk, 1, D), rn(Lyr, B, Hk, 1, D)
    outp = torch.empty((B, Hq, P, D), dtype=torch.float32, device="cuda")
    outd = torch.empty((Lyr, B, Hq, 1, D), dtype=torch.float32, device="cuda")
    ws = kb.workspace(max(kb.attn_workspace_bytes(B, Hq, P, P), kb.attn_workspace_bytes(B, Hq, 1, S)))

    def prefill(_):
        for l in range(Lyr):
            kb.decode_step_self(qp[l], kp[l], vp[l], caches[l], P, 0.125, rope_base=1e4, out=outp, ws=ws)

    def decode(s):
        for l in range(Lyr):
            kb.decode_step_self(qd[l], kd[l], vd[l], caches[l], s + 1, 0.125, rope_base=1e4, out=outd[l], ws=ws)

    pg = _graph_steps(torch, prefill, [0])
    t_prefill = _time_graphs(torch, pg, max(1, reps))
    del pg
    dg = _graph_steps(torch, decode, range(P, S))
    sec = _time_graphs(torch, dg, reps)
    del dg
    row = Hk * D * 2
    kv = sum(Lyr * B * (2 * (s + 1) * row + 2 * row) for s in range(P, S)) / (S - P)
    dec_period = _graph_period(torch, [lambda l=l: kb.decode_step_self(
        qd[l], kd[l], vd[l], caches[l], 768, 0.125, rope_base=1e4, out=outd[l], ws=ws) for l in range(Lyr)])
    prefill_us = _kernel_us(torch, kb, lambda i: kb.decode_attn_self(qp[i % Lyr], caches[i % Lyr], P, 0.125, rope_base=1e4, out=outp, ws=ws), n=30)
    flops = prefill_flops()
    ptf = flops / (prefill_us * 1e-6) / 1e12
    return {"metric": "GQA decode steps/s (B=8, 9q/3kv heads, len 513..1024), 1 GPU",
            "value": round(1 / sec, 2), "unit": "steps/s", "ms_per_step": round(sec * 1e3, 4),
            "dtype": "bf16",
            "effective_kv_gbps": round(kv / sec / 1e9, 1),
            "hbm_peak_frac": round(kv / sec / 1e9 / HBM_PEAK_GBPS, 4),
            "roofline": roof(B * Hk * 768 * 2 * row, dec_period,
                             "decode_step_self at len 768, rotary keys (matrix-core tile), "
                             "30 back-to-back launches in a graph"),
            "prefill_ms": round(t_prefill * 1e3, 4),
            "prefill_attention_kernel_us": round(prefill_us, 3),
            "prefill_roofline": {"bound": "mfma", "achieved": round(ptf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(ptf / MFMA_BF16_PEAK_TFLOPS, 4),
                                 "kernel": "decode_attn_self, 512 causal queries, rotary (matrix-core tile)"},
            "config": {"workload": "GQA LM: 30 layers, B8, Hq9/Hkv3 x 64, bf16, RoPE 1e4; prefill 512 "
                                   "then decode to 1024",
                       "timed": f"prefill graph x {max(1, reps)}; 512 decode step graphs x {reps} replays"}}


def workload_kernels(torch, kb, reps):
    """A handful of eager launches of each hot kernel (no graphs), for
    hardware-counter runs, which collect per dispatch: cross attention
    (1 and 5 rows per head), the fused self step at lengths 64 / 224 / 448,
    the GQA decode step with rotary keys at 768, the prefill tile, and the
    known-size calibration kernels (a 7,680,000-byte read probe and a
    7,680,000-byte kv_append). Prints the launch counts."""
    from kv_cached_decode_amd import inputs as I
    g = torch.Generator(device="cuda").manual_seed(9)
    rn = lambda *sh: (torch.randn(*sh, generator=g, device="cuda") / 8).half()
    n = 4
    xs = []
    for _ in range(n):
        x = kb.Cache(1, H, FRAMES, torch.float16)
        kb.kv_append(x, rn(1, H, FRAMES, D), rn(1, H, FRAMES, D), 0)   # 7,680,000 B written
        xs.append(x)
    sc = [kb.Cache(1, H, S_MAX, torch.float16) for _ in range(n)]
    for c in sc:
        c.k.copy_(rn(1, H, S_MAX, D)); c.v.copy_(rn(1, H, S_MAX, D))
    ws = kb.workspace(max(kb.attn_workspace_bytes(1, H, 5, FRAMES), kb.attn_workspace_bytes(8, 9, 512, 1024)))
    counts = {}
    q1, q5 = rn(1, H, 1, D), rn(1, H, 5, D)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for i in range(n):
        kb.decode_attn_cross(q1, xs[i], FRAMES, 0.125, ws=ws)
        kb.read_probe(xs[i].k, xs[i].v, CROSS_BYTES // 2, sink)
    counts["cross_1row"] = counts["read_probe_7680000B"] = counts["kv_append_7680000B"] = n
    for i in range(n):
        kb.decode_attn_cross(q5, xs[i], FRAMES, 0.125, ws=ws)
    counts["cross_5rows"] = n
    for L in (64, 224, 448):
        for i in range(n):
            kb.decode_step_self(q1, rn(1, H, 1, D), rn(1, H, 1, D), sc[i], L, 0.125, ws=ws)
        counts[f"step_self_len{L}"] = n
    gq = [kb.Cache(8, 3, 1024, torch.bfloat16) for _ in range(n)]
    for c in gq:
        c.k.copy_(torch.randn(8, 3, 1024, D, generator=g, device="cuda").bfloat16())
        c.v.copy_(torch.randn(8, 3, 1024, D, generator=g, device="cuda").bfloat16())
    qd = torch.randn(8, 9, 1, D, generator=g, device="cuda").bfloat16()
    kd = torch.randn(8, 3, 1, D, generator=g, device="cuda").bfloat16()
    for i in range(n):
        kb.decode_step_self(qd, kd, kd, gq[i], 768, 0.125, rope_base=1e4, ws=ws)
    counts["gqa_step_len768_rope"] = n
    qp = torch.randn(8, 9, 512, D, generator=g, device="cuda").bfloat16()
    for i in range(n):
        kb.decode_attn_self(qp, gq[i], 512, 0.125, rope_base=1e4, ws=ws)
    counts["prefill_512"] = n
    torch.cuda.synchronize()
    return {"metric": "kernel launches for counter collection", "value": sum(counts.values()),
            "unit": "launches", "launches": counts}


if __name__ == "__main__":
    main()
