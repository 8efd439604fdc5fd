#!/usr/bin/env python3
"""Benchmark: MoE dispatch + combine on one MI355X.

One step = the whole path on one batch: moe_plan_and_dispatch_begin (the
launches that need only the IDs), moe_plan_and_dispatch_end (the one launch
that writes the payload), moe_combine (identity experts for bf16 workloads:
the combine reads the packed rows the dispatch wrote; random bf16 expert
outputs otherwise).  Depending on the problem (moe_plan_and_dispatch_mode),
_begin launches nothing, the plan's counting kernel, or the whole plan.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line on stdout.  ``value`` = algorithmic bytes of one step
(plan + dispatch + combine, see ``step_bytes``) / measured step time, in
GB/s.  Inputs are resident in HBM before timing starts; consecutive steps
rotate over several copies of all buffers so that a step does not find its
inputs in the 256 MB last-level cache from the step before.

Per-kernel durations for the roofline (means, and p10/p50/p90 of each phase
and of the step) come from HIP timing events (no system-scope fence, see
TimingEvent) recorded around every call on the stream the kernels run on,
in a second pass over the same number of steps:
"plan" is _begin, "dispatch" is _end (one kernel), "combine" the combine.
``payload_only`` repeats the rate counting only packed rows that hold a
token.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
DEFAULT_WORKLOAD = "zipf_bf16_n16384"
# further configurations measured in the same run, each reported with its own
# roofline under "configs" (the decode shape's µs are under "decode")
EXTRA_WORKLOADS = ("uniform_bf16_n4096", "fp8_b128_n8192", "gated_map_bf16_n4096")
METRIC = "dispatch+combine effective HBM GB/s (% of peak) on 1 GPU; µs at decode shape"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def row_bytes(fmt, h):
    return {"bf16": 2 * h, "fp8": h + 4 * (h // 128), "mxfp4": h // 2 + h // 32,
            "nvfp4": h // 2 + h // 16}[fmt]


def step_bytes(w, r_used, r_max, kept=None):
    """Algorithmic bytes of one step (each array read or written once).

    One buffer: r_used = R_used rows (live + pad), r_max = R_max.  Exchange:
    r_used = receive rows in use over all buffers, r_max = EP * C; the
    dispatch writes every receive row (live rows, then zero rows).  Fixed
    expert capacity: r_used = r_max = E * cap rows, all written; kept = pairs
    kept, the rows the combine reads.  Gates at dispatch: the dispatch also
    reads the gates, the combine does not.  Routing given as a dense map: the
    plan also converts it (reads the map's N*E bytes and the probabilities
    of the kept experts, writes the IDs and gates)."""
    t = w.tokens
    nk = t * w.k
    if kept is not None:
        plan = 4 * nk + 4 * nk + 4 * r_max                       # ids, slot, packed_src
        dispatch = 2 * t * w.h + r_max * row_bytes(w.fmt, w.h)   # read x once, write all rows
        combine = 4 * nk + 4 * nk + 2 * w.h * kept + 2 * t * w.h  # slot, w, kept rows, out
    elif w.exchange:
        plan = 4 * nk + 4 * nk + 4 * r_max                       # ids, recv_slot, recv_src
        dispatch = 2 * t * w.h + r_max * row_bytes(w.fmt, w.h)   # read x once, write all rows
        combine = 4 * nk + 4 * nk + 2 * w.h * r_used + 2 * t * w.h  # slot, w, kept rows, out
    else:
        plan = 4 * nk + 4 * nk + 4 * r_max                     # ids, slot, packed_src
        dispatch = 2 * t * w.h + r_used * row_bytes(w.fmt, w.h)  # read x once, write live+pad rows
        combine = 4 * nk + 4 * nk + 2 * w.h * nk + 2 * t * w.h   # slot, w, k rows of y, out
    if w.gated:
        dispatch += 4 * nk   # the gates, applied to each copy
        combine -= 4 * nk    # no weights in the combine
    if w.routing_input == "map":
        plan += t * w.e + 4 * nk + 4 * nk + 4 * nk  # map, kept probabilities, ids, gates
    return dict(plan=plan, dispatch=dispatch, combine=combine,
                total=plan + dispatch + combine)


def buffer_rows(w, expert_cap=0):
    """Rows of the packed buffer (R_max; E * cap with a fixed expert
    capacity) or of all receive buffers (EP * C)."""
    if expert_cap:
        return w.e * expert_cap
    return w.ep * w.capacity if w.exchange else w.n * w.k + w.e * (w.a - 1)


def traffic_from_profile(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, or None if there is none or the kernels changed since."""
    from combine_topk_ids_amd.rocprof_summary import kernel_source_hash
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if not k else k["hbm_bytes_per_launch"]


class Path:
    """Device buffers and the three calls of one step, for one workload."""

    def __init__(self, moe, torch, w, inp, copies, expert_cap=0):
        self.moe, self.torch, self.w = moe, torch, w
        self.p = moe.problem(w.n, w.h, w.k, w.e, w.ep, recv_capacity=w.capacity,
                             pad_multiple=w.a, fmt=w.fmt, zero_tail=False,
                             expert_capacity=expert_cap)
        self.expert_cap = expert_cap
        self.r_max = moe.moe_max_rows(self.p)
        dev = "cuda"
        x = torch.from_numpy(inp["hidden"].view(np.int16)).to(dev).view(torch.bfloat16)
        ids = torch.from_numpy(inp["ids"]).to(dev)
        wts = torch.from_numpy(inp["weights"]).to(dev)
        y = None
        if "expert_out" in inp:
            y = torch.from_numpy(inp["expert_out"].view(np.int16)).to(dev).view(torch.bfloat16)
        self.gs = torch.tensor([w.input_scale], dtype=torch.float32, device=dev)
        self.from_map = w.routing_input == "map"
        if self.from_map:
            rmap = torch.from_numpy(inp["map"]).to(dev)
            probs = torch.from_numpy(inp["probs"]).to(dev)
        self.sets = []
        for c in range(copies):
            plan = moe.alloc_plan(self.p, dev)
            payload, scales = moe.alloc_payload(self.p, dev)
            payload.view(torch.uint8).zero_()
            if scales is not None:
                scales.zero_()
            s = dict(
                x=x if c == 0 else x.clone(), ids=ids if c == 0 else ids.clone(),
                w=wts if c == 0 else wts.clone(),
                y=(y if c == 0 else y.clone()) if y is not None else payload,
                plan=plan, payload=payload, scales=scales,
                out=torch.empty((w.n, w.h), dtype=torch.bfloat16, device=dev))
            if self.from_map:
                # the IDs and gates are written by the map conversion each step;
                # its status word and workspace are buffers of their own
                s.update(map=rmap if c == 0 else rmap.clone(),
                         probs=probs if c == 0 else probs.clone(),
                         map_status=torch.empty(1, dtype=torch.int32, device=dev),
                         map_ws=torch.empty(max(moe.moe_map_workspace_bytes(self.p), 256),
                                            dtype=torch.uint8, device=dev))
            self.sets.append(s)

    def _routing(self, s):
        """A dense routing map is turned into the compact IDs and gates."""
        if self.from_map:
            self.moe.moe_routing_map_to_topk(self.p, s["map"], s["probs"], s["ids"], s["w"],
                                             s["map_status"], s["map_ws"])

    def step(self, i, ev=None):
        s = self.sets[i % len(self.sets)]
        m, p = self.moe, self.p
        gs = self.gs if self.w.fmt == "nvfp4" else None
        gates = s["w"] if self.w.gated else None
        if ev is not None:
            ev[0].record()
        self._routing(s)
        m.moe_plan_and_dispatch_begin(p, s["ids"], s["plan"])
        if ev is not None:
            ev[1].record()
        m.moe_plan_and_dispatch_end(p, s["ids"], s["plan"], s["x"], s["payload"], s["scales"],
                                    topk_weights=gates, input_scale=gs)
        if ev is not None:
            ev[2].record()
        m.moe_combine(p, s["plan"], s["y"], None if self.w.gated else s["w"], s["out"])
        if ev is not None:
            ev[3].record()

    def step_three_calls(self, i):
        """The same step as moe_dispatch_plan, moe_dispatch, moe_combine (the
        plan's kernels, then the dispatch kernel)."""
        s = self.sets[i % len(self.sets)]
        m, p = self.moe, self.p
        self._routing(s)
        m.moe_dispatch_plan(p, s["ids"], s["plan"])
        if self.w.fmt == "nvfp4":
            m.moe_dispatch_scaled(p, s["plan"], s["x"], self.gs, s["payload"], s["scales"])
        elif self.w.gated:
            m.moe_dispatch_gated(p, s["plan"], s["x"], s["w"], s["payload"], s["scales"])
        else:
            m.moe_dispatch(p, s["plan"], s["x"], s["payload"], s["scales"])
        m.moe_combine(p, s["plan"], s["y"], None if self.w.gated else s["w"], s["out"])

    def mode(self):
        return {self.moe.PD_ONE_LAUNCH: "one_launch", self.moe.PD_TILED: "tiled",
                self.moe.PD_SEPARATE: "separate"}[self.moe.moe_plan_and_dispatch_mode(self.p)]

    def dispatch_kernel(self):
        """The kernel _end launches: in one launch without padding the kernel
        that counts each pair's row (the library takes it up to 512 ballots a
        wave, which every one-launch workload here is far below)."""
        m = self.mode()
        if m == "separate":
            return "dispatch_kernel"
        if m == "one_launch" and self.w.a == 1:
            return "plan_dispatch_rank_kernel"
        return "plan_dispatch_kernel"

    def r_used(self):
        return int(self.sets[0]["plan"].expert_offsets[-1].item())

    def kept(self):
        """Pairs kept by a fixed expert capacity (rows the combine reads)."""
        return int(self.sets[0]["plan"].dest_counts.sum().item())

    def live_rows(self):
        """Packed rows that hold a token (not padding)."""
        if self.expert_cap:
            return self.kept()
        return int(self.sets[0]["plan"].expert_counts.sum().item())


class ExchangePath:
    """Device buffers and the three calls of one step of the exchange across
    EP simulated ranks (exchange plan, dispatch into the receive buffers,
    reverse combine)."""

    def __init__(self, moe, torch, w, inp, copies):
        self.moe, self.torch, self.w = moe, torch, w
        self.p = moe.problem(w.n, w.h, w.k, w.e, w.ep, recv_capacity=w.capacity, fmt=w.fmt)
        dev = "cuda"
        x = torch.from_numpy(inp["hidden"].view(np.int16)).to(dev).view(torch.bfloat16)
        ids = torch.from_numpy(inp["ids"].reshape(w.ranks, w.n, w.k)).to(dev)
        wts = torch.from_numpy(inp["weights"]).to(dev)
        y = None
        if "expert_out" in inp:
            y = torch.from_numpy(inp["expert_out"].view(np.int16)).to(dev).view(torch.bfloat16)
        self.sets = []
        for c in range(copies):
            xb = moe.alloc_exchange(self.p, dev)
            payload, scales = moe.alloc_recv_payload(self.p, dev)
            payload.view(torch.uint8).zero_()
            if scales is not None:
                scales.zero_()
            self.sets.append(dict(
                x=x if c == 0 else x.clone(), ids=ids if c == 0 else ids.clone(),
                w=wts if c == 0 else wts.clone(),
                y=(y if c == 0 else y.clone()) if y is not None else payload,
                xb=xb, payload=payload, scales=scales,
                out=torch.empty((w.tokens, w.h), dtype=torch.bfloat16, device=dev)))

    def step(self, i, ev=None):
        s = self.sets[i % len(self.sets)]
        m, p = self.moe, self.p
        if ev is not None:
            ev[0].record()
        m.moe_exchange_plan(p, s["ids"], s["xb"])
        if ev is not None:
            ev[1].record()
        m.moe_exchange_dispatch(p, s["xb"], s["x"], s["payload"], s["scales"])
        if ev is not None:
            ev[2].record()
        m.moe_exchange_combine(p, s["xb"], s["y"], s["w"], s["out"])
        if ev is not None:
            ev[3].record()

    def dispatch_kernel(self):
        """The kernel of the dispatch call."""
        return "dispatch_kernel"

    def r_used(self):
        rows = self.sets[0]["xb"].recv_rows.clamp(max=self.w.capacity)
        return int(rows.sum().item())

    def live_rows(self):
        """Receive rows that hold a token (not zero rows)."""
        return self.r_used()


class _SameSet:
    """A path whose every step uses the first buffer set."""

    def __init__(self, path):
        self.path = path

    def step(self, i, ev=None):
        self.path.step(0, ev)


class _ThreeCalls:
    """A single-buffer path stepped as moe_dispatch_plan, moe_dispatch,
    moe_combine."""

    def __init__(self, path):
        self.path = path

    def step(self, i, ev=None):
        self.path.step_three_calls(i)


def time_steps(torch, path, steps, warmup):
    for i in range(warmup):
        path.step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        path.step(warmup + i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


class TimingEvent:
    """A HIP event for timing only, recorded on torch's current stream (the
    stream the library's kernels are launched on).  Created with
    hipEventDisableSystemFence: recording it does not write back and
    invalidate the caches at system scope, which a default event does, so
    an interval between two such events adds about 1 µs to the kernel
    inside it, against about 3 µs with default events.  The HIP runtime is
    the one libmoe.so is linked against (the symbols are looked up through
    its handle)."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence
    _hip = None

    @classmethod
    def _runtime(cls, moe):
        if cls._hip is None:
            import ctypes
            hip, V = moe.lib, ctypes.c_void_p
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(V), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [V, V]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), V, V]
            hip.hipEventDestroy.argtypes = [V]
            cls._hip = hip
        return cls._hip

    def __init__(self, moe, torch):
        import ctypes
        self._ct, self.torch = ctypes, torch
        self.hip = self._runtime(moe)
        self.h = ctypes.c_void_p()
        self._check(self.hip.hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE),
                    "hipEventCreateWithFlags")

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def record(self):
        stream = self._ct.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        self._check(self.hip.hipEventRecord(self.h, stream), "hipEventRecord")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both recorded and complete)."""
        ms = self._ct.c_float()
        self._check(self.hip.hipEventElapsedTime(self._ct.byref(ms), self.h, end.h),
                    "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        if getattr(self, "h", None) and self.h.value:
            self.hip.hipEventDestroy(self.h)


def time_kernels(torch, path, steps, moe):
    evs = [[TimingEvent(moe, torch) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        path.step(i, evs[i])
    torch.cuda.synchronize()
    d = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3]),
                   e[0].elapsed_time(e[3])] for e in evs])
    out = {}
    for c, name in enumerate(("plan", "dispatch", "combine", "step")):
        out[name] = float(np.mean(d[:, c]))
        for q in (10, 50, 90):
            out[f"{name}_p{q}"] = float(np.percentile(d[:, c], q))
    return out


def stream_reference(torch, gib=1.0):
    """Achievable-bandwidth context and counter calibration: a plain
    streaming kernel of known size (negate 1 GiB of bf16: 1 GiB read,
    1 GiB written)."""
    n = int(gib * (1 << 30)) // 2
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    s.record()
    for _ in range(reps):
        torch.neg(a, out=b)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b
    return 2 * n * 2 / (ms * 1e-3) / 1e9


def decode_latency(moe, torch, w, inp, iters=200, per_graph=16):
    """µs per plan + dispatch + combine at the decode shape, three ways:
    back-to-back calls from Python (host-bound: each call costs a few µs of
    Python and ctypes), one HIP graph per step, and one HIP graph holding
    `per_graph` steps (closest to the GPU's own time per step).  For a single
    packed buffer the same is reported for the step made of the three
    separate calls (``three_calls``: the plan's kernel, then the dispatch)."""
    path = (ExchangePath if w.exchange else Path)(moe, torch, w, inp, copies=1)
    out = dict(workload=w.name)
    if isinstance(path, Path):
        out["plan_and_dispatch"] = path.mode()
    # discarded passes first: the first graph figures measured in a process
    # came out high (up to twice the later ones), whatever the graph held
    _latencies(torch, path, lambda: path.step(0), iters, per_graph)
    if isinstance(path, Path):
        _latencies(torch, path, lambda: path.step_three_calls(0), iters, per_graph)
    out.update(_latencies(torch, path, lambda: path.step(0), iters, per_graph))
    if isinstance(path, Path):
        out["three_calls"] = _latencies(torch, path, lambda: path.step_three_calls(0), iters,
                                        per_graph)
    return out


def _latencies(torch, path, step, iters, per_graph):
    for i in range(20):
        step()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def clock(fn, reps, rounds=5):
        # median of `rounds` timed runs: the host-bound figures jump between runs
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        per = max(reps // rounds, 1)
        out = []
        for _ in range(rounds):
            s.record()
            for _ in range(per):
                fn()
            e.record()
            torch.cuda.synchronize()
            out.append(s.elapsed_time(e) / per * 1e3)
        return float(np.median(out))

    plain = clock(step, iters)
    ref = path.sets[0]["out"].clone()
    graphs = {}
    for n in (1, per_graph):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                step()
        graphs[n] = (g, clock(g.replay, max(iters // n, 10)) / n)
    # every replay recomputes the same output as the eager path
    path.sets[0]["out"].zero_()
    graphs[per_graph][0].replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(ref.view(torch.int16), path.sets[0]["out"].view(torch.int16)))
    out = dict(us_per_step_python_launch=round(plain, 2), us_per_step_graph=round(graphs[1][1], 2))
    out[f"us_per_step_graph_x{per_graph}"] = round(graphs[per_graph][1], 2)
    out["graph_matches_eager"] = same
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores():
    """Host cores this process may run on."""
    return len(os.sched_getaffinity(0))


def cpu_baseline(w, inp, pass_s=5.0, runs=3):
    """The CPU oracle on the host: plan + dispatch + combine on the first M
    tokens of the workload (a smaller instance of the same routing), M chosen
    so that one single-thread pass takes about pass_s; the median of `runs`
    passes on one thread, then of `runs` passes on every host core the
    process may use (the oracle's OpenMP row loops); GB/s by wall clock with
    the same algorithmic byte formula.  Both give bit-identical outputs."""
    import oracle
    oracle.build(force=False)
    if w.exchange:
        return cpu_baseline_exchange(w, inp, pass_s, runs)

    def one_pass(m):
        ids, wts, x = inp["ids"][:m], inp["weights"][:m], inp["hidden"][:m]
        t0 = time.perf_counter()
        kept = None
        if w.capacity_factor is not None:
            cap = oracle.expert_capacity(m, w.k, w.e, w.capacity_factor)
            pl = oracle.capacity_plan(ids, w.e, w.ep, cap, m * min(w.k, w.l), w.h)
            kept = int(pl["dest_counts"].sum())
        else:
            pl = oracle.plan(ids, w.e, w.ep, w.a, m * min(w.k, w.l), w.h)
        if w.fmt == "nvfp4":
            pay, _ = oracle.dispatch_nvfp4(x, pl, w.input_scale, zero_tail=False)
        else:
            pay, _ = oracle.dispatch(w.fmt, x, pl, zero_tail=False)
        y = pay.view(np.uint16).reshape(pl["r_max"], -1) if "expert_out" not in inp \
            else inp["expert_out"]
        oracle.combine(pl["slot"], wts, y)
        dt = time.perf_counter() - t0
        sub = dataclasses.replace(w, n=m)
        return dt, step_bytes(sub, pl["r_used"], pl["r_max"], kept)["total"]

    res, m, cores = _cpu_runs(w, one_pass, min(w.n, 64), pass_s, runs)
    return cpu_record(res, m, cores, f"the first {m} of {w.n} tokens of {w.name} "
                                     f"({w.describe()})", runs)


def _cpu_runs(w, one_pass, m0, pass_s, runs):
    import oracle
    cores = host_cores()
    oracle.set_threads(1)
    dt, _ = one_pass(m0)
    m = int(min(w.n, max(1, m0 * pass_s / max(dt, 1e-6))))
    res = {}
    for threads in (1, cores):
        oracle.set_threads(threads)
        one_pass(min(m, 16))  # start the threads
        meas = [one_pass(m) for _ in range(runs)]
        gbps = sorted(nb / dt / 1e9 for dt, nb in meas)
        res[threads] = (gbps[len(gbps) // 2], float(np.median([dt for dt, _ in meas])))
    oracle.set_threads(cores)
    return res, m, cores


def cpu_record(res, m, cores, what, runs=3):
    (one, t_one), (allc, t_all) = res[1], res[cores]
    return dict(value=round(allc, 3), unit="GB/s", cores=cores, kind="oracle",
                single_thread=dict(value=round(one, 3), unit="GB/s", cores=1),
                cpu_model=cpu_model(),
                sample=f"plan+dispatch+combine over {what}; median of {runs} passes by wall "
                       f"clock: {t_one:.2f} s a pass on 1 thread, {t_all:.2f} s on {cores} "
                       f"threads (OpenMP over rows; identical outputs)")


def cpu_baseline_exchange(w, inp, pass_s, runs):
    """The CPU oracle's exchange (plan, receive buffers, reverse combine) on
    the first M tokens of every rank, with C scaled by M / N."""
    import oracle
    ids3 = inp["ids"].reshape(w.ranks, w.n, w.k)
    x3 = inp["hidden"].reshape(w.ranks, w.n, w.h)
    w3 = inp["weights"].reshape(w.ranks, w.n, w.k)

    def one_pass(m):
        cap = -(-w.capacity * m // w.n)
        ids = np.ascontiguousarray(ids3[:, :m])
        x = np.ascontiguousarray(x3[:, :m].reshape(-1, w.h))
        wts = np.ascontiguousarray(w3[:, :m].reshape(-1, w.k))
        t0 = time.perf_counter()
        xp = oracle.exchange_plan(ids, w.e, cap, w.h)
        pay, _ = oracle.exchange_dispatch(w.fmt, x, xp)
        y = pay.view(np.uint16).reshape(w.ep * cap, -1) if "expert_out" not in inp \
            else inp["expert_out"]
        oracle.combine(xp["recv_slot"].reshape(-1, w.k), wts, y)
        dt = time.perf_counter() - t0
        sub = dataclasses.replace(w, n=m, recv_capacity=cap)
        used = int(np.minimum(xp["recv_rows"], cap).sum())
        return dt, step_bytes(sub, used, w.ep * cap)["total"]

    res, m, cores = _cpu_runs(w, one_pass, min(w.n, 16), pass_s, runs)
    return cpu_record(res, m, cores,
                      f"the first {m} of {w.n} tokens of each of {w.ranks} ranks of {w.name} "
                      f"({w.describe()}; C scaled to {-(-w.capacity * m // w.n)})", runs)


def measure(moe, torch, w, args, context=True):
    """Time one workload: the step over rotating buffer sets, per-kernel
    events, the roofline of the dominant kernel; with `context`, also the
    warm step (one buffer set) and the step as three separate calls."""
    expert_cap = 0
    if w.capacity_factor is not None:
        expert_cap = moe.moe_expert_capacity(w.n, w.k, w.e, w.capacity_factor)
    r_max = buffer_rows(w, expert_cap)
    from combine_topk_ids_amd.workloads import make_inputs
    inp = make_inputs(w, seed=0, expert_rows=r_max)
    set_bytes = (w.tokens * w.h * 2 * 2 + r_max * row_bytes(w.fmt, w.h)
                 + (r_max * w.h * 2 if "expert_out" in inp else 0))
    copies = args.copies or max(2, min(8, -(-(768 << 20) // max(set_bytes, 1)) + 1))
    path = ExchangePath(moe, torch, w, inp, copies) if w.exchange else \
        Path(moe, torch, w, inp, copies, expert_cap)
    log(f"[bench] {w.name}: {w.describe()}; {copies} buffer sets of "
        f"{set_bytes / 1e6:.1f} MB rotated")

    ms, wall = time_steps(torch, path, args.steps, args.warmup)
    log(f"[bench] {w.name}: timed {args.steps} steps: {ms * 1e3:.2f} us/step (wall {wall:.3f} s)")
    warm_ms = three_ms = None
    if context:
        # the same buffer set every step, so inputs may stay in the caches
        warm_ms, _ = time_steps(torch, _SameSet(path), args.steps, args.warmup)
        log(f"[bench] {w.name}: warm (one buffer set): {warm_ms * 1e3:.2f} us/step")
        if not w.exchange:
            # the same step as the plan call, the dispatch call, the combine
            three_ms, _ = time_steps(torch, _ThreeCalls(path), args.steps, args.warmup)
            log(f"[bench] {w.name}: plan_and_dispatch {path.mode()}; as three calls: "
                f"{three_ms * 1e3:.2f} us/step")
    kt = time_kernels(torch, path, args.steps, moe)
    log(f"[bench] {w.name}: per-kernel means (us): plan {kt['plan'] * 1e3:.2f} dispatch "
        f"{kt['dispatch'] * 1e3:.2f} combine {kt['combine'] * 1e3:.2f}")
    log(f"[bench] {w.name}: p10/p50/p90 (us): " + "; ".join(
        f"{n} {kt[n + '_p10'] * 1e3:.2f}/{kt[n + '_p50'] * 1e3:.2f}/{kt[n + '_p90'] * 1e3:.2f}"
        for n in ("plan", "dispatch", "combine", "step")))
    ru = path.r_used()
    b = step_bytes(w, ru, r_max, path.kept() if expert_cap else None)
    value = b["total"] / (ms * 1e-3) / 1e9
    # the same step counting only rows that hold a token (no pad, zero or
    # tail rows written)
    live = path.live_rows()
    disp_live = 2 * w.tokens * w.h + live * row_bytes(w.fmt, w.h)
    payload_only = dict(live_rows=live, dispatch_bytes=disp_live,
                        total_bytes=b["plan"] + disp_live + b["combine"],
                        gbps=round((b["plan"] + disp_live + b["combine"]) / (ms * 1e-3) / 1e9, 1))

    dom = "dispatch" if kt["dispatch"] >= kt["combine"] else "combine"
    kname = "combine_kernel"
    dom_bytes = b[dom]
    if dom == "dispatch":
        kname = path.dispatch_kernel()
        if kname.startswith("plan_dispatch"):
            # it also reads the IDs and writes slot and packed_src
            dom_bytes = b["dispatch"] + b["plan"]
    achieved = dom_bytes / (kt[dom] * 1e-3) / 1e9
    traffic = traffic_from_profile(w.name, kname)
    roofline = dict(bound="hbm", kernel=kname, achieved=round(achieved, 1),
                    peak=PEAK_HBM_GBPS, unit="GB/s", frac=round(achieved / PEAK_HBM_GBPS, 4),
                    traffic=traffic, algorithmic_bytes=dom_bytes,
                    avg_launch_us=round(kt[dom] * 1e3, 2))

    config = {"workload": w.name, "tokens": w.n, "hidden": w.h, "experts": w.e,
              "top_k": w.k, "ep_ranks_simulated": w.ep, "pad_multiple": w.a,
              "format": w.fmt, "routing": w.routing, "r_used": ru, "r_max": r_max,
              "buffer_sets": copies}
    if not w.exchange:
        config["plan_and_dispatch"] = path.mode()
    if w.exchange:
        config.update(source_ranks=w.ranks, recv_capacity=w.capacity,
                      path="exchange: source-major receive buffers of C rows per rank")
    if w.fmt == "nvfp4":
        config["input_scale"] = w.input_scale
    if expert_cap:
        config.update(capacity_factor=w.capacity_factor, expert_capacity=expert_cap,
                      pairs_kept=path.kept(), path="fixed expert capacity, later pairs dropped")
    if w.gated:
        config["gates"] = "applied at dispatch; combine without weights"
    if w.routing_input == "map":
        config["routing_input"] = "dense multihot map + dense probabilities, converted each step"
    rec = dict(value=round(value, 1), unit="GB/s", ms_per_step=round(ms, 5),
               frac_of_peak=round(value / PEAK_HBM_GBPS, 4), dtype=w.fmt, config=config,
               bytes_per_step=b, payload_only=payload_only,
               kernel_us={k: round(v * 1e3, 2) for k, v in kt.items()}, roofline=roofline)
    if context:
        rec["warm_us_per_step"] = round(warm_ms * 1e3, 2)
        rec["three_calls_us_per_step"] = None if three_ms is None else round(three_ms * 1e3, 2)
    del path
    torch.cuda.empty_cache()
    return rec, inp


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--extra", default=",".join(EXTRA_WORKLOADS),
                    help="comma-separated workloads also measured, each under 'configs' "
                         "('' for none)")
    ap.add_argument("--copies", type=int, default=0, help="buffer sets rotated over (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-workload", default="decode_mxfp4_n128",
                    help="workload whose µs per step is reported under 'decode'")
    ap.add_argument("--no-copy-ref", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library "
              "measures one GPU's share of the work, with expert-parallel ranks simulated as "
              "segments of one buffer.", file=sys.stderr)
        sys.exit(2)

    import torch
    import combine_topk_ids_amd.moe as moe
    from combine_topk_ids_amd.workloads import WORKLOADS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = WORKLOADS[args.workload]
    log(f"[bench] headline workload {w.name}: {w.describe()}")
    head, inp = measure(moe, torch, w, args, context=True)

    extra = {}
    configs = {}
    for name in [x for x in args.extra.split(",") if x and x != w.name]:
        rec, _ = measure(moe, torch, WORKLOADS[name], args, context=False)
        configs[name] = rec
    if configs:
        extra["configs"] = configs
    if not args.no_copy_ref:
        extra["stream_ref_gbps"] = round(stream_reference(torch), 1)
        log(f"[bench] 1 GiB read + 1 GiB write streaming kernel: {extra['stream_ref_gbps']} GB/s")
    if not args.no_decode:
        dw = WORKLOADS[args.decode_workload]
        dinp = make_inputs(dw, seed=0, expert_rows=buffer_rows(dw))
        extra["decode"] = decode_latency(moe, torch, dw, dinp)
        log(f"[bench] decode: {extra['decode']}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp)
        log(f"[bench] cpu baseline: {cpu}")

    rec = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.fmt,
        "data": "synthetic",
        "config": head["config"],
        "frac_of_peak": head["frac_of_peak"],
        "bytes_per_step": head["bytes_per_step"],
        "payload_only": head["payload_only"],
        "warm_us_per_step": head["warm_us_per_step"],
        "three_calls_us_per_step": head["three_calls_us_per_step"],
        "kernel_us": head["kernel_us"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
    }
    rec.update(extra)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
