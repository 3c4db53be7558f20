"""Benchmark of the load-balanced MoE token path on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload dsv3]

One step = route_topk (+ load histogram) -> plan_balance -> align_sort ->
dispatch -> combine over one batch of synthetic router logits and bf16
activations already resident in HBM (identity expert: combine reads the
dispatched rows).  Prints one JSON line: token-slots/s of the whole step,
per-kernel device times from HIP events recorded on the launch stream, the
HBM roofline of the dominant kernel (combine), and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, vendor figure
PROFILES = os.path.join(ROOT, "profiles")


def algorithmic_bytes(w, C):
    """Bytes each step must move (padding rows excluded; fp32 y).  Route:
    logits read, ids + gates written.  Align: ids read, slot and sorted_ids
    written.  Dispatch: x read once, K copies written, slot read.  Combine:
    K rows read, slot + gate read, fp32 y written."""
    N, P, E, H = w.N, w.P, w.E, w.H
    return {
        "route": N * E * 4 + P * 8,
        "align": P * 12,
        "dispatch": N * H * 2 + P * H * 2 + P * 4,
        "combine": P * H * 2 + P * 8 + N * H * 4,
    }


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "load_balanced_token_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"source_hash:\s*(\w+)", txt)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m or not b or m.group(1) != source_hash("move.hip", "rows.h", "lbt_internal.h"):
        return None
    return float(b.group(1))


def cpu_baseline(name, sample_S, **overrides):
    """The oracle, as it stands, on a bounded sample of the workload: the same
    generator and shapes with S reduced to ``sample_S`` tokens per rank."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    import oracle
    from workloads import WORKLOADS, router_logits, activations

    w = WORKLOADS[name].with_(S=sample_S, **overrides)
    logits = router_logits(w, 0)
    x = activations(w, 0)
    score = oracle.SOFTMAX if w.score == "softmax" else oracle.SIGMOID
    steps = {}
    t0 = tl = time.perf_counter()

    def lap(name):
        nonlocal tl
        now = time.perf_counter()
        steps[name] = now - tl
        tl = now

    ids, gates = oracle.route_topk(logits, w.K, score)
    lap("O1_route")
    counts = oracle.load_matrix(ids, w.R, w.S, w.E)
    lap("O2_histogram")
    plan = oracle.plan_balance(counts, w.K, w.S, w.B, w.blk)
    lap("O3_plan")
    al = oracle.align_sort(ids, plan)
    lap("O4_align")
    rows, data = oracle.dispatch_rows(x, al["slot"], w.K)
    lap("O5_dispatch")
    order = np.argsort(rows)
    srt = rows[order]
    y, _ = oracle.combine(lambda r: data[order[np.searchsorted(srt, r)]], al["slot"],
                          gates.astype(np.float32), w.K)
    lap("O6_combine")
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    return {
        "value": w.P / dt,
        "unit": "token-slots/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{name} shape with S={sample_S} tokens/rank (N={w.N}, P={w.P} token-slots, "
                  f"H={w.H}), layer 0; oracle route, histogram, plan, align, dispatch, combine "
                  f"end to end on one host thread in {dt:.2f} s",
        "step_s": steps,
        "host_cpu": host_cpu_model(),
        "host_logical_cpus": os.cpu_count(),
        "host_affinity_cpus": len(os.sched_getaffinity(0)),
    }


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


# hipDeviceAttribute_t values of the ROCm 7 HIP runtime headers
_HIP_ATTR = {"sclk_khz": 5, "memory_bus_width_bits": 59, "memory_clock_khz": 60,
             "compute_units": 63}


def device_report(torch, dev_index=0):
    """Name, ISA, compute units, engine and memory clocks and the memory bus
    width of the device the run used (hipDeviceGetAttribute)."""
    import ctypes
    p = torch.cuda.get_device_properties(dev_index)
    rep = {"name": p.name, "arch": p.gcnArchName, "total_memory_gib": p.total_memory / 2 ** 30}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        for key, attr in _HIP_ATTR.items():
            v = ctypes.c_int(0)
            if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, dev_index) == 0:
                rep[key] = v.value
    except OSError:
        pass
    return rep


def decode_latency(path, buf, w, x, n_steps, dev, planner="fixed"):
    """p50/p99 latency of one step over ``n_steps`` fresh routings, for the
    whole step (route -> plan -> align -> dispatch -> combine; the first
    four are one lbt_front_dispatch call) and for the step without the
    combine.

    Every routing is resident in HBM before timing starts.  Step i is
    captured as its own HIP graph, bound to routing i where it lies, and the
    graphs are replayed in order: each replay runs the path on new router
    logits with no gather, copy or host work inside the timed region.  The
    reported p50/p99 are device-side: the replays are queued 50 at a time
    behind a spin kernel, so a step never waits for the host to submit it
    (as inside a larger graph).  ``host_paced`` keeps the same replays
    issued one by one as the host reaches them."""
    import numpy as np
    import torch
    from workloads import router_logits

    all_logits = torch.empty((n_steps, w.N, w.E), dtype=torch.float32, device=dev)
    for i in range(n_steps):
        all_logits[i] = torch.from_numpy(router_logits(w, i)).to(dev)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    plan_fn = path.plan_balance if planner == "fixed" else path.plan_quota

    def full(i):
        path.step(all_logits[i], x, buf, planner=planner)

    def no_combine(i):
        if planner == "fixed":
            path.front_dispatch(all_logits[i], x, buf)
        else:
            path.route_topk(all_logits[i], buf["ids"], buf["gates"], buf["counts"], buf["work"])
            plan_fn(buf["counts"], buf["plan"], buf["status"])
            path.align_dispatch(buf["ids"], buf["work"], buf["plan"], x, buf["slot"],
                                buf["sorted_ids"], buf["block_wrow"], buf["block_expert"],
                                buf["recv"], buf["status"])

    def replay(body):
        with torch.cuda.stream(stream):        # warm up outside the graphs
            for i in range(min(3, n_steps)):
                body(i)
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        graphs = []
        for i in range(n_steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                body(i)
            graphs.append(g)
        # a few replays first, untimed, so the timed series starts from a
        # running GPU (the first series of a process otherwise ran ~1.5 us
        # slower at p50 than the second)
        for g in graphs[:min(32, n_steps)]:
            g.replay()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_steps)]
        t0 = time.perf_counter()
        for (a, b), g in zip(evs, graphs):
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        lat = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        # The same replays with the GPU held on a spin kernel while the host
        # queues a chunk of them, so that no step waits for the host to
        # submit it: the device-side latency of a step, as inside a larger
        # graph (above, a step starts when the host's replay call reaches
        # the GPU, and the host's submission time can show in it).
        q = np.empty(n_steps)
        evq = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_steps)]
        for c0 in range(0, n_steps, queue_chunk):
            torch.cuda._sleep(spin_cycles)
            for i in range(c0, min(c0 + queue_chunk, n_steps)):
                evq[i][0].record()
                graphs[i].replay()
                evq[i][1].record()
            torch.cuda.synchronize()
        q[:] = [a.elapsed_time(b) * 1e3 for a, b in evq]
        del graphs
        # the last replay's routing, checked for a clean status
        return lat, q, wall, int(buf["status"].item())

    # spin length for the queued series: long enough for the host to queue
    # a chunk of replays (calibrated against HIP events)
    queue_chunk = 50
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    torch.cuda._sleep(1 << 20)
    ev1.record()
    torch.cuda.synchronize()
    cycles_per_us = (1 << 20) / max(ev0.elapsed_time(ev1) * 1e3, 1e-3)
    spin_cycles = int(cycles_per_us * 4000)      # 4 ms per chunk of 50 steps

    lat_nc, q_nc, _, st_nc = replay(no_combine)
    lat, q, wall, status = replay(full)
    pct = lambda a, p: float(np.percentile(a, p))   # noqa: E731
    return {"p50_us": pct(q, 50), "p99_us": pct(q, 99), "mean_us": float(q.mean()),
            "steps": n_steps, "wall_s": wall, "status": status,
            "without_combine": {"p50_us": pct(q_nc, 50), "p99_us": pct(q_nc, 99),
                                "status": st_nc},
            "host_paced": {"p50_us": pct(lat, 50), "p99_us": pct(lat, 99),
                           "without_combine_p50_us": pct(lat_nc, 50),
                           "without_combine_p99_us": pct(lat_nc, 99),
                           "note": "the host replays the graphs one by one: a step starts "
                                   "when the host's replay call reaches the GPU"},
            "note": "one HIP graph per step, each on its own resident routing; p50/p99: the "
                    "device-side step latency, replays queued 50 at a time behind a spin "
                    "kernel so that no step waits for the host's submission"}


def planner_report(lbt, torch, w, counts, B, tau_max, dev, ids=None, work=None):
    """Both planners on the same load matrix: latency (median of 20 back-to-back
    calls; either planner is one launch), the
    threshold, replica segments, the most on one rank, remote replicas, and
    (given the step's ids and workspace) how many pairs each plan serves on
    their own token's rank -- the pairs a multi-GPU run would not send."""
    import numpy as np
    stream = torch.cuda.current_stream()
    out = {}
    for name in ("fixed", "quota"):
        shape = lbt.Shape(E=w.E, K=w.K, R=w.R, S=w.S, H=w.H, B=B, blk=w.blk,
                          score_fn=lbt.SOFTMAX if w.score == "softmax" else lbt.SIGMOID,
                          tau_max=tau_max)
        p = lbt.Path(shape)
        plan = torch.empty(p.sizes["plan_words"], dtype=torch.int32, device=dev)
        fn = p.plan_balance if name == "fixed" else p.plan_quota
        for _ in range(3):
            fn(counts, plan)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(21)]
        ev[0].record(stream)
        for i in range(20):
            fn(counts, plan)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        us = float(np.median([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(20)]))
        pf = lbt.plan_fields(plan.cpu().numpy(), p.sizes, w.R, w.E)
        hdr = pf["hdr"]
        out[name] = {"us": us, "tau": int(hdr[9]), "tau_over_SK": float(hdr[9]) / max(1, w.SK),
                     "replica_segments": int(hdr[0]), "max_replicas_per_rank": int(hdr[10]),
                     "remote_replicas": int(pf["n_remote"].sum()), "feasible": bool(hdr[11]),
                     "search_candidates": (tau_max or w.SK) - w.SK + 1 if name == "quota" else 0}
        if ids is not None and work is not None:
            z = p.sizes
            i32 = dict(dtype=torch.int32, device=dev)
            slot = torch.empty(w.P, **i32)
            sorted_ids = torch.empty(w.R * z["C"], **i32)
            bw = torch.empty(w.R * z["n_blocks"], **i32)
            be = torch.empty_like(bw)
            st = torch.zeros(1, **i32)
            p.align_sort(ids, work, plan, slot, sorted_ids, bw, be, st)
            f = torch.arange(w.P, dtype=torch.int64, device=dev)
            own = int(((slot.long() // z["C"]) == (f // w.K) // w.S).sum().item())
            out[name]["own_rank_pairs"] = own
            out[name]["own_rank_fraction"] = own / max(1, w.P)
            out[name]["align_status"] = int(st.item())
    out["B"] = B
    out["tau_max"] = tau_max or w.SK
    return out


def training_report(lbt, torch, w, path, buf, dev, Hp, reps):
    """The training-side kernels at the workload's shape: replica weight
    prefetch and reduce_grad over the plan's slotted replicas (one expert
    projection of H x H' elements: bf16 weights, fp32 gradients), and the
    backward of combine and dispatch on the step's buffers.  Median of
    ``reps`` back-to-back launches timed with HIP events on the launch
    stream; algorithmic bytes as stated per kernel."""
    import numpy as np
    stream = torch.cuda.current_stream()
    plan = buf["plan"]
    pf = lbt.plan_fields(plan.cpu().numpy(), path.sizes, w.R, w.E)
    nP = int(pf["hdr"][0])
    wrow = pf["piece_wrow"][:nP]
    pexp = pf["piece_expert"][:nP]
    slotted = int((wrow >= w.E).sum())
    runs = int(len(set(pexp[wrow >= w.E].tolist())))
    row = w.H * Hp

    def time_it(fn):
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps)]))

    def entry(us, nbytes, what):
        gbps = nbytes / (us * 1e-6) / 1e9 if us > 0 else 0.0
        return {"us": us, "algorithmic_bytes": nbytes, "gbps": gbps,
                "frac_peak": gbps / HBM_PEAK_GBPS, "bytes": what}

    out = {"H_prime": Hp, "slotted_replicas": slotted, "experts_with_slots": runs}
    if w.B > 0 and slotted > 0:
        W = torch.empty((w.E, row), dtype=torch.int16, device=dev)
        S = torch.empty((w.R, w.B, row), dtype=torch.int16, device=dev)
        us = time_it(lambda: path.prefetch_weights(plan, W, S))
        out["prefetch"] = entry(us, (runs + slotted) * row * 2,
                                "bf16 H x H' weights: each distinct home row read once, "
                                "each slotted replica's slot written")
        del W, S
        G = torch.zeros((w.E, row), dtype=torch.float32, device=dev)
        SG = torch.zeros((w.R, w.B, row), dtype=torch.float32, device=dev)
        us = time_it(lambda: path.reduce_grad(plan, SG, G))
        out["reduce_grad"] = entry(us, (2 * slotted + 2 * runs) * row * 4,
                                   "fp32: each used slot read and cleared, each home "
                                   "gradient with slots read and written once")
        del G, SG
        torch.cuda.synchronize()
    dy = torch.zeros((w.N, w.H), dtype=torch.float32, device=dev)
    d_out = torch.empty_like(buf["recv"])
    d_g = torch.empty((w.N, w.K), dtype=torch.float32, device=dev)
    us = time_it(lambda: path.combine_bwd(buf["recv"], buf["slot"], buf["gates"], dy, d_out, d_g))
    out["combine_bwd"] = entry(us, w.N * w.H * 4 + 2 * w.P * w.H * 2 + w.P * 12,
                               "fp32 dy read, K bf16 rows read, K bf16 gradient rows "
                               "written, slot + gate read, gate gradient written")
    dx = torch.empty((w.N, w.H), dtype=torch.float32, device=dev)
    us = time_it(lambda: path.dispatch_bwd(d_out, buf["slot"], dx))
    out["dispatch_bwd"] = entry(us, w.P * w.H * 2 + w.P * 4 + w.N * w.H * 4,
                                "K bf16 rows read, slot read, fp32 dx written")
    del dy, d_out, d_g, dx
    torch.cuda.synchronize()
    return out


def hbm_ceilings(torch, dev, nbytes, reps=10):
    """Reference HBM streams (bench_ceiling.so): a plain read, write and copy
    of ``nbytes`` each, and the copy with non-temporal loads, median of ``reps`` launches timed with HIP events on
    the current stream; GB/s counts the bytes read plus the bytes written."""
    import ctypes
    import numpy as np
    path = os.path.join(ROOT, "bench_ceiling.so")
    if not os.path.exists(path):
        return {"error": "bench_ceiling.so is not built"}
    L = ctypes.CDLL(path)
    L.hbm_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong,
                             ctypes.c_void_p]
    L.hbm_stream.restype = ctypes.c_int
    a = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    a.fill_(7)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    out = {"bytes_per_launch": nbytes}
    for name, kind, moved in (("read", 0, nbytes), ("write", 1, nbytes), ("copy", 2, 2 * nbytes),
                              ("copy_nt", 3, 2 * nbytes)):
        bp = b.data_ptr() if kind != 1 else None
        for _ in range(3):
            assert L.hbm_stream(kind, ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(bp), nbytes, sp) == 0
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            L.hbm_stream(kind, ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(bp), nbytes, sp)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        us = float(np.median([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps)]))
        gbps = moved / (us * 1e-6) / 1e9
        out[name] = {"us": us, "gbps": gbps, "frac_peak": gbps / HBM_PEAK_GBPS}
    del a, b
    torch.cuda.synchronize()
    return out


class StepRunner:
    """Buffers and inputs of one workload, resident in HBM, and the timed step
    (route -> plan -> align -> dispatch -> combine) over them."""

    def __init__(self, lbt, torch, w, dev, planner="fixed", tau_max=0, x_on_device=False):
        import numpy as np
        from workloads.gen import X_CHUNK, x_chunk
        self.torch, self.w, self.dev, self.planner = torch, w, dev, planner
        shape = lbt.Shape(E=w.E, K=w.K, R=w.R, S=w.S, H=w.H, B=w.B, blk=w.blk,
                          score_fn=lbt.SOFTMAX if w.score == "softmax" else lbt.SIGMOID,
                          tau_max=tau_max if planner == "quota" else 0)
        self.path = lbt.Path(shape)
        self.C = self.path.sizes["C"]
        self.buf = self.path.alloc(dev)
        print(f"[bench] {w.name}: E={w.E} K={w.K} R={w.R} S={w.S} H={w.H} B={w.B} blk={w.blk} "
              f"C={self.C}; generating inputs", file=sys.stderr, flush=True)
        if x_on_device:
            # N(0,1) rounded to bf16, drawn on the device (the values of x do
            # not change what the path does or how long it takes)
            g = torch.Generator(device=dev)
            g.manual_seed(w.seed)
            x = torch.randn((w.N, w.H), generator=g, device=dev, dtype=torch.float32)
            self.x = x.to(torch.bfloat16).view(torch.int16)
            del x
        else:
            self.x = torch.empty((w.N, w.H), dtype=torch.int16, device=dev)
            for c in range((w.N + X_CHUNK - 1) // X_CHUNK):
                blk = x_chunk(w, 0, c)
                self.x[c * X_CHUNK: c * X_CHUNK + blk.shape[0]] = \
                    torch.from_numpy(blk.view(np.int16)).to(dev)
        self.buf["status"].zero_()
        torch.cuda.synchronize()
        self.stream = torch.cuda.current_stream()
        self.plan_fn = self.path.plan_balance if planner == "fixed" else self.path.plan_quota

    names = ["route", "plan", "align", "dispatch", "combine"]

    def step(self, logits, evs=None):
        path, buf, stream = self.path, self.buf, self.stream
        rec = (lambda i: evs[i].record(stream)) if evs is not None else (lambda i: None)
        rec(0)
        path.route_topk(logits, buf["ids"], buf["gates"], buf["counts"], buf["work"])
        rec(1)
        self.plan_fn(buf["counts"], buf["plan"], buf["status"])
        rec(2)
        path.align_sort(buf["ids"], buf["work"], buf["plan"], buf["slot"], buf["sorted_ids"],
                        buf["block_wrow"], buf["block_expert"], buf["status"])
        rec(3)
        path.dispatch(self.x, buf["slot"], buf["recv"])
        rec(4)
        path.combine(buf["recv"], buf["slot"], buf["gates"], buf["y"])
        rec(5)

    def timed(self, logits, steps, warmup):
        """Warm up, then time ``steps`` steps with nothing but the steps on
        the stream (wall seconds; the device time between one event before
        and one after them is kept as ``timed_dev_us``, per step).  Then run
        as many steps again, untimed, with an event between every two
        kernels: mean per-kernel event times (us) and each of those steps'
        device time (us)."""
        import numpy as np
        torch, stream = self.torch, self.stream
        for _ in range(warmup):
            self.step(logits)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(steps):
            self.step(logits)
        b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        self.timed_dev_us = a.elapsed_time(b) * 1e3 / max(steps, 1)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(self.names) + 1)]
               for _ in range(steps)]
        for i in range(steps):
            self.step(logits, evs[i])
        torch.cuda.synchronize()
        per = {n: [] for n in self.names}
        for e in evs:
            for j, n in enumerate(self.names):
                per[n].append(e[j].elapsed_time(e[j + 1]) * 1e3)   # microseconds
        return (wall, {n: float(np.mean(v)) for n, v in per.items()},
                [e[0].elapsed_time(e[-1]) * 1e3 for e in evs])

    def plan_alone_us(self, reps=20):
        """The planner alone: median of back-to-back launches on the step's
        load matrix (checked equal to the step's plan)."""
        import numpy as np
        torch, buf = self.torch, self.buf
        plan2 = torch.empty_like(buf["plan"])
        pev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        for _ in range(3):
            self.plan_fn(buf["counts"], plan2)
        pev[0].record(self.stream)
        for i in range(reps):
            self.plan_fn(buf["counts"], plan2)
            pev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        assert torch.equal(plan2, buf["plan"]), "standalone plan differs from the step's"
        return float(np.median([pev[i].elapsed_time(pev[i + 1]) * 1e3 for i in range(reps)]))

    def summary(self, wall, avg_us, step_dev_us, steps):
        """Throughput and HBM fractions of a timed run."""
        import numpy as np
        w = self.w
        ab = algorithmic_bytes(w, self.C)
        hdr = self.buf["plan"][:16].cpu().numpy()
        gb = lambda n, us: ab[n] / (us * 1e-6) / 1e9   # noqa: E731
        dc = (ab["dispatch"] + ab["combine"]) / ((avg_us["dispatch"] + avg_us["combine"]) * 1e-6) / 1e9
        ms = wall / steps * 1e3
        return {
            "ms_per_step": ms,
            "token_slots_per_s": w.P * steps / wall,
            "step_hbm_gbps": sum(ab.values()) / (ms * 1e-3) / 1e9,
            "dispatch_combine_gbps": dc,
            "dispatch_combine_frac_peak": dc / HBM_PEAK_GBPS,
            "dispatch_frac_peak": gb("dispatch", avg_us["dispatch"]) / HBM_PEAK_GBPS,
            "combine_frac_peak": gb("combine", avg_us["combine"]) / HBM_PEAK_GBPS,
            "route_frac_peak": gb("route", avg_us["route"]) / HBM_PEAK_GBPS,
            "align_frac_peak": gb("align", avg_us["align"]) / HBM_PEAK_GBPS,
            "kernel_us": avg_us,
            "step_device_us_timed": getattr(self, "timed_dev_us", None),
            "step_device_us_median": float(np.median(step_dev_us)),
            "step_device_us_min": float(np.min(step_dev_us)),
            "max_vio": float(hdr[1]) * w.E / w.P - 1.0,
            "rank_imbalance_before": float(hdr[2]) / w.SK - 1.0,
            "replica_segments": int(hdr[0]),
            "max_replicas_per_rank": int(hdr[10]),
            "status": int(self.buf["status"].item()),
        }

    def free(self):
        del self.buf, self.x, self.path
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def workloads_block(lbt, torch, dev, steps, warmup, decode_steps):
    """Every other workload at its full shape, each in its own guard so that
    a failure records an error and keeps the line: WideEP and Kimi-K3 (step
    time, dispatch + combine fraction, route / plan / align times in the
    step, plan alone), decode S = 1, 16, 128 (eager step plus the p50/p99 of
    one HIP graph per step over fresh routings), and the MoonEP max_vio
    sweep (E=384, S=8192, max_vio 0.2, 1, 10, 20)."""
    from workloads import WORKLOADS, router_logits
    from workloads.gen import MAXVIO_SWEEP
    out = {}

    def one(name, fn):
        t0 = time.perf_counter()
        print(f"[bench] workloads block: {name}", file=sys.stderr, flush=True)
        try:
            out[name] = fn()
        except Exception as e:  # keep the line: record what failed
            out[name] = {"error": f"{type(e).__name__}: {e}"[:400]}
        out[name]["wall_s"] = time.perf_counter() - t0
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    def big(name):
        def fn():
            w = WORKLOADS[name]
            run = StepRunner(lbt, torch, w, dev, x_on_device=True)
            try:
                logits = torch.from_numpy(router_logits(w, 0)).to(dev)
                wall, us, dev_us = run.timed(logits, steps, warmup)
                res = run.summary(wall, us, dev_us, steps)
                res["plan_us"] = run.plan_alone_us()
                res["x"] = "N(0,1) bf16 drawn on the device"
                return res
            finally:
                run.free()
        return fn

    def decode(name):
        def fn():
            w = WORKLOADS[name]
            run = StepRunner(lbt, torch, w, dev)
            try:
                logits = torch.from_numpy(router_logits(w, 0)).to(dev)
                wall, us, dev_us = run.timed(logits, steps, warmup)
                res = run.summary(wall, us, dev_us, steps)
                res["plan_us"] = run.plan_alone_us()
                res["decode_latency"] = decode_latency(run.path, run.buf, w, run.x, decode_steps,
                                                       dev)
                return res
            finally:
                run.free()
        return fn

    def sweep():
        w = WORKLOADS["moonep"]
        run = StepRunner(lbt, torch, w, dev, x_on_device=True)
        try:
            pts = []
            for v in MAXVIO_SWEEP:
                lg = torch.from_numpy(router_logits(w.with_(vio=v), 0)).to(dev)
                wall, us, dev_us = run.timed(lg, steps, warmup)
                res = run.summary(wall, us, dev_us, steps)
                res["vio"] = v
                pts.append(res)
                del lg
            ms = [p["ms_per_step"] for p in pts]
            return {"points": pts, "ms_per_step_max_over_min": max(ms) / min(ms),
                    "x": "N(0,1) bf16 drawn on the device"}
        finally:
            run.free()

    one("wideep", big("wideep"))
    one("kimi", big("kimi"))
    for name in ("decode1", "decode16", "decode128"):
        one(name, decode(name))
    one("moonep_maxvio_sweep", sweep)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--cpu-sample-S", type=int, default=0,
                    help="tokens per rank of the oracle sample (default: up to 32768 tokens in all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=1000,
                    help="fresh-routing graph replays for the decode workloads (0: none)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--planner", choices=("fixed", "quota"), default="fixed",
                    help="planner inside the timed step")
    ap.add_argument("--B", type=int, default=-1, help="prefetch slots per rank (default: workload's)")
    ap.add_argument("--tau-max-x", type=float, default=2.0,
                    help="quota planner's threshold bound, in units of S*K")
    ap.add_argument("--vio", type=float, default=-1.0,
                    help="target max_vio of the moonep workload's routing (default 20)")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the training-side kernels (prefetch, reduce_grad, backward)")
    ap.add_argument("--h-prime", type=int, default=2048,
                    help="expert intermediate size H' of the prefetched weights")
    ap.add_argument("--maxvio-sweep", action="store_true",
                    help="moonep: also time the step at max_vio 0.2, 1, 10, 20 (same buffers)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the block of the other workloads (run with the default dsv3 only)")
    ap.add_argument("--ceilings", action="store_true",
                    help="also time plain HBM read, write and copy streams (bench_ceiling.so)")
    ap.add_argument("--x-device", action="store_true",
                    help="draw x on the device (N(0,1) bf16, torch's generator) instead of the host")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: every expert-parallel rank of the workload is a "
              "logical partition of that GPU's memory, so --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import load_balanced_token_amd as lbt
    from workloads import WORKLOADS, router_logits

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = WORKLOADS[args.workload]
    if args.B >= 0:
        w = w.with_(B=args.B)
    if args.vio >= 0:
        w = w.with_(vio=args.vio)
    tau_max = int(round(args.tau_max_x * w.SK))
    run = StepRunner(lbt, torch, w, dev, args.planner, tau_max, x_on_device=args.x_device)
    path, buf, x, C = run.path, run.buf, run.x, run.C

    sweep = []
    if args.maxvio_sweep:
        if w.skew != "maxvio":
            print("--maxvio-sweep needs a workload with the maxvio skew (moonep)", file=sys.stderr)
            sys.exit(2)
        from workloads.gen import MAXVIO_SWEEP
        for v in MAXVIO_SWEEP:
            print(f"[bench] max_vio sweep: vio={v}", file=sys.stderr, flush=True)
            lg = torch.from_numpy(router_logits(w.with_(vio=v), 0)).to(dev)
            wall_v, us_v, dev_v = run.timed(lg, args.steps, args.warmup)
            pt = run.summary(wall_v, us_v, dev_v, args.steps)
            pt["vio"] = v
            pt["remote_replicas"] = int(buf["plan"][path.sizes["off_n_remote"]:
                                                    path.sizes["off_n_remote"] + w.R].sum().item())
            sweep.append(pt)
            del lg
            torch.cuda.synchronize()

    logits = torch.from_numpy(router_logits(w, 0)).to(dev)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps after {args.warmup} warmup", file=sys.stderr,
          flush=True)
    wall, avg_us, step_dev_us = run.timed(logits, args.steps, args.warmup)
    plan_alone_us = run.plan_alone_us()
    summ = run.summary(wall, avg_us, step_dev_us, args.steps)

    planners = planner_report(lbt, torch, w, buf["counts"], w.B, tau_max, dev,
                              ids=buf["ids"], work=buf["work"])
    training = None
    if not args.no_train:
        print("[bench] training-side kernels", file=sys.stderr, flush=True)
        training = training_report(lbt, torch, w, path, buf, dev, args.h_prime, 10)
    if args.calib_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    ceilings = None
    if args.ceilings:
        print("[bench] reference HBM streams", file=sys.stderr, flush=True)
        ceilings = hbm_ceilings(torch, dev, w.P * w.H * 2)

    ab = algorithmic_bytes(w, C)
    comb_gbps = ab["combine"] / (avg_us["combine"] * 1e-6) / 1e9
    traffic = measured_traffic("combine", w.name)
    result = {
        "metric": "token-slots/s",
        "value": summ["token_slots_per_s"],
        "unit": "token-slots/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": summ["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "E": w.E, "K": w.K, "R": w.R, "S": w.S, "H": w.H,
                   "B": w.B, "blk": w.blk, "C": C, "token_slots_per_step": w.P,
                   "planner": args.planner,
                   **({"vio": w.vio} if w.skew == "maxvio" else {}),
                   "gate": w.score, "combine_accumulate": "fp32", "y": "fp32",
                   "expert": "identity (out = recv)"},
        "roofline": {"bound": "hbm", "kernel": "k_combine",
                     "achieved": comb_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": comb_gbps / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": ab["combine"]},
        "step_hbm_gbps": summ["step_hbm_gbps"],
        "step_pct_hbm_peak": summ["step_hbm_gbps"] / HBM_PEAK_GBPS,
        "dispatch_combine_gbps": summ["dispatch_combine_gbps"],
        "dispatch_combine_frac_peak": summ["dispatch_combine_frac_peak"],
        "dispatch_gbps": summ["dispatch_frac_peak"] * HBM_PEAK_GBPS,
        "kernel_us": avg_us,
        "kernels": {n: {"us": avg_us[n], "algorithmic_bytes": ab[n],
                        "frac_peak": ab[n] / (avg_us[n] * 1e-6) / 1e9 / HBM_PEAK_GBPS}
                    for n in ("route", "align", "dispatch", "combine")},
        "plan_us": plan_alone_us,
        "plan_in_step_us": avg_us["plan"],
        "step_device_us_timed": summ["step_device_us_timed"],
        "step_device_us_median": summ["step_device_us_median"],
        "step_device_us_min": summ["step_device_us_min"],
        "max_vio": summ["max_vio"],
        "rank_imbalance_before": summ["rank_imbalance_before"],
        "replica_segments": summ["replica_segments"],
        "planners": planners,
        **({"maxvio_sweep": sweep} if sweep else {}),
        **({"training": training} if training else {}),
        **({"hbm_ceilings": ceilings} if ceilings else {}),
        "status": summ["status"],
        "device": torch.cuda.get_device_name(0),
        "device_info": device_report(torch, 0),
    }
    if w.name.startswith("decode") and args.decode_steps > 0:
        print(f"[bench] decode latency over {args.decode_steps} fresh routings (HIP graph)",
              file=sys.stderr, flush=True)
        result["decode_latency"] = decode_latency(path, buf, w, x, args.decode_steps, dev,
                                                  args.planner)
    del path, buf, x, logits
    run.free()
    if args.workload == "dsv3" and not args.no_workloads:
        result["workloads"] = workloads_block(lbt, torch, dev, args.steps, args.warmup,
                                              args.decode_steps)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        sample_S = args.cpu_sample_S or max(1, min(w.S, 32768 // w.R))
        result["cpu_baseline"] = cpu_baseline(w.name, sample_S, B=w.B, vio=w.vio)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
