#!/usr/bin/env python3
"""Throughput of the chunkwise GLA forward pass (key-only decay, four scan
directions) on one MI355X, against the HBM roofline, with the CPU oracle timed
beside it.

A step is one pass of the workload's call list through gla_chunk_fwd: for the
16.4K-token grid (B=1, 12 heads, 128x128 tokens, d_k=d_v=64, fp16) the four scan
directions.  Inputs sit in HBM before timing starts.  Each call reads its own
device copy of the inputs and writes its own outputs, and the copies are cycled
so that the bytes touched between two reuses of a copy exceed the 256 MB
last-level (Infinity) cache: every call streams from HBM as a real layer
stack would, instead of re-reading cache-resident data.

Beside it, the same protocol times the backward pass of the same workload
(gla_chunk_bwd, under "backward"), the block's other token mixer, the
Spatial SwiGLU step (gla_spatial_swiglu) on the 16.4K grid with 2048 hidden
channels, reported under "spatial_swiglu", and the SAGA-style non-causal
gated linear attention (gla_saga_fwd) on the same token count, under "saga".

Prints ONE JSON line on stdout; details go to stderr.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GLA chunkwise fwd tokens/s at 1.6K & 16.4K tokens; % of HBM/MFMA roofline"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 MFMA, published
LLC_BYTES = 256 << 20           # Infinity Cache
KERNEL_SRC = os.path.join(ROOT, "recurrent_vision_token_amd", "csrc", "gla_kernels.hip")
SWIGLU_SRC = os.path.join(ROOT, "recurrent_vision_token_amd", "csrc", "swiglu_kernels.hip")
SAGA_SRC = os.path.join(ROOT, "recurrent_vision_token_amd", "csrc", "saga_kernels.hip")
BWD_SRC = os.path.join(ROOT, "recurrent_vision_token_amd", "csrc", "gla_bwd_kernels.hip")
KERNEL_NAMES = ("span_summary", "span_scan", "chunk_output", "spatial_swiglu", "saga_kv_partial",
                "saga_kv_reduce", "saga_out", "chunk_bwd", "bwd_state_summaries", "bwd_state_scans")


def kernel_key(name):
    """The KERNEL_NAMES entry a (demangled) kernel name belongs to, or None."""
    return next((k for k in KERNEL_NAMES if k in name), None)


DEVICE_HDR = os.path.join(ROOT, "recurrent_vision_token_amd", "csrc", "gla_device.h")


def source_of(kernel):
    if kernel == "spatial_swiglu":
        return SWIGLU_SRC
    if kernel == "chunk_bwd":
        return BWD_SRC
    return SAGA_SRC if kernel.startswith("saga") else KERNEL_SRC


TILES_HDR = os.path.join(ROOT, "recurrent_vision_token_amd", "csrc", "gla_tiles.h")


def source_hash(kernel):
    """Hash of the device code a kernel is built from (its file and the shared
    device headers)."""
    h = hashlib.sha256()
    paths = [source_of(kernel), DEVICE_HDR]
    if source_of(kernel) in (KERNEL_SRC, BWD_SRC):
        paths.append(TILES_HDR)
    for path in paths:
        h.update(open(path, "rb").read())
    from recurrent_vision_token_amd.build import flags_for
    h.update(" ".join(flags_for(os.path.basename(source_of(kernel)))).encode())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(wl):
    """Per-call algorithmic bytes and flops of the method (per token-head unit)."""
    es = 2 if wl.dtype == "fp16" else 4
    th = wl.B * wl.heads * wl.T                         # token-heads per call
    bh = wl.B * wl.heads
    io_bytes = th * es * (3 * wl.d_k + 2 * wl.d_v)      # read q, k, log_alpha, v; write out
    state_bytes = bh * wl.d_k * wl.d_v * 4              # final state
    flops = th * ((wl.chunk + 1) * (wl.d_k + wl.d_v) + 4 * wl.d_k * wl.d_v)
    return {"bytes": io_bytes + state_bytes, "io_bytes_per_token_head": es * (3 * wl.d_k + 2 * wl.d_v),
            "flops": flops, "token_heads": th}


def kernel_bytes(wl, n_spans, kernels=3):
    """Algorithmic bytes each kernel of one call moves (its own reads and writes).
    kernels = 2 is the two-pass path: no scan, and the output workgroup of span
    s reads the summaries (state and gate) of spans 0..s-1."""
    es = 2 if wl.dtype == "fp16" else 4
    th = wl.B * wl.heads * wl.T
    bh = wl.B * wl.heads
    st = wl.d_k * wl.d_v * 4
    # entry states of the three-pass path: float16 on the float16 path
    st_entry = wl.d_k * wl.d_v * es
    if kernels == 2:
        entry = bh * n_spans * (n_spans - 1) // 2 * (st + 4 * wl.d_k)
    else:
        entry = bh * n_spans * st_entry if n_spans > 1 else 0
    out = {"chunk_output": th * es * (3 * wl.d_k + 2 * wl.d_v) + bh * st + entry}
    if n_spans > 1:
        # three passes: summaries in the entry states' precision (float16 on
        # the float16 path), scanned in place; two passes: float32 summaries
        st_sum = st_entry if kernels == 3 else st
        out["span_summary"] = th * es * (2 * wl.d_k + wl.d_v) + bh * n_spans * (st_sum + 4 * wl.d_k)
        if kernels == 3:
            out["span_scan"] = bh * n_spans * (st_sum + 4 * wl.d_k + st_entry)
    return out


_HOST_INPUTS = {}


def host_inputs(wl, seed):
    """A workload's seeded host inputs, generated once per (workload, seed): the
    batched configuration's 2 GB take tens of seconds to draw, and its forward
    and backward lines share them."""
    from recurrent_vision_token_amd.workloads import workload_inputs
    key = (wl.name, seed)
    if key not in _HOST_INPUTS:
        _HOST_INPUTS[key] = tuple(workload_inputs(wl, seed))
    return _HOST_INPUTS[key]


class Runner:
    """Device copies of a workload's inputs, cycled across calls.

    ext=True drives the extended entry point instead: the gate tensor is taken
    as gate logits (fused activation, tau 16) and every call starts from a
    stored initial state."""

    def __init__(self, wl, torch, min_sets_bytes=2 * LLC_BYTES, ext=False):
        self.torch = torch
        self.wl = wl
        self.dev = torch.device("cuda:0")
        calls = wl.calls
        host = {}
        for seed, _ in calls:
            if seed not in host:
                host[seed] = host_inputs(wl, seed)
        self.host = host
        per_call = algorithmic(wl)["bytes"]
        reps = max(1, math.ceil(min_sets_bytes / (per_call * len(calls))))
        self.sets = []
        for _ in range(reps):
            for seed, d in calls:
                q, k, v, la = (torch.from_numpy(x).to(self.dev) for x in host[seed])
                out = torch.empty(v.shape, dtype=v.dtype, device=self.dev)
                fs = torch.empty((wl.B, wl.heads, wl.d_k, wl.d_v), dtype=torch.float32, device=self.dev)
                init = torch.full((wl.B, wl.heads, wl.d_k, wl.d_v), 0.01, dtype=torch.float32,
                                  device=self.dev) if ext else None
                self.sets.append((q, k, v, la, out, fs, d, init))
        self.cursor = 0
        torch.cuda.synchronize()

        # raw C-ABI arguments of every set, so the timed loop only marshals ints
        from recurrent_vision_token_amd import _lib
        lib = _lib.load()
        stream = torch.cuda.current_stream(self.dev).cuda_stream
        if ext:
            self.fn = lib.gla_chunk_fwd_ex
            self.args = [(q.data_ptr(), k.data_ptr(), v.data_ptr(), la.data_ptr(), 1, 16.0,
                          init.data_ptr(), d, wl.B, wl.heads, wl.H, wl.W, wl.d_k, wl.d_v,
                          wl.chunk, out.data_ptr(), fs.data_ptr(), stream)
                         for (q, k, v, la, out, fs, d, init) in self.sets]
        else:
            self.fn = lib.gla_chunk_fwd if wl.dtype == "fp16" else lib.gla_chunk_fwd_f32
            self.args = [(q.data_ptr(), k.data_ptr(), v.data_ptr(), la.data_ptr(), d, wl.B,
                          wl.heads, wl.H, wl.W, wl.d_k, wl.d_v, wl.chunk, out.data_ptr(),
                          fs.data_ptr(), stream)
                         for (q, k, v, la, out, fs, d, _) in self.sets]

    def step(self, events=None):
        """One pass of the call list; events: list of 6-event lists, one per call."""
        from recurrent_vision_token_amd import _lib
        for c in range(len(self.wl.calls)):
            a = self.args[self.cursor]
            self.cursor = (self.cursor + 1) % len(self.sets)
            if events is not None:
                rc = _lib.set_kernel_events([e.cuda_event for e in events[c]])
                if rc != 0:
                    raise RuntimeError("gla_set_kernel_events failed: %d" % rc)
            rc = self.fn(*a)
            if rc != 0:
                raise RuntimeError("gla_chunk_fwd failed: %d" % rc)


def time_workload(wl, torch, steps, warmup, ext=False, extras=False):
    """Timed loop (no instrumentation), then an event-instrumented pass of the
    same length for the per-kernel durations.  With extras, also the spread of
    per-step times (an event pair around every step of a further pass) and a
    warm figure (every call re-reads one resident input set)."""
    r = Runner(wl, torch, ext=ext)
    ncall = len(wl.calls)
    log("[bench] %s: %d device input sets (%.0f MB), %d calls/step" %
        (wl.name, len(r.sets), len(r.sets) * algorithmic(wl)["bytes"] / 1e6, ncall))
    for _ in range(warmup):
        r.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        r.step()
    t_issue = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    log("[bench] %s: host issue %.1f us/call, wall %.1f us/call" %
        (wl.name, (t_issue - t0) * 1e6 / (steps * ncall), (t1 - t0) * 1e6 / (steps * ncall)))

    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(ncall)]
           for _ in range(steps)]
    stream = torch.cuda.current_stream()
    for per_step in evs:                      # materialise the HIP events
        for per_call in per_step:
            for e in per_call:
                e.record(stream)
    torch.cuda.synchronize()
    for s in range(steps):
        r.step(evs[s])
    torch.cuda.synchronize()
    k_ms = {"span_summary": [], "span_scan": [], "chunk_output": [], "call": []}
    for per_step in evs:
        for e in per_step:
            k_ms["span_summary"].append(e[0].elapsed_time(e[1]))
            k_ms["span_scan"].append(e[2].elapsed_time(e[3]))
            k_ms["chunk_output"].append(e[4].elapsed_time(e[5]))
            k_ms["call"].append(e[0].elapsed_time(e[5]))
    mean = {k: sum(v) / len(v) for k, v in k_ms.items()}
    # the measurement protocol of the pages' comparison: an event pair around
    # every call (no per-kernel hook), 20 warm-up calls, the median of at
    # least 100 calls (cycling the input sets and directions)
    n_calls = max(100, steps * ncall)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(n_calls + 1)]
    for e in marks:
        e.record(stream)
    for i in range(20):
        rc = r.fn(*r.args[i % len(r.args)])
        if rc != 0:
            raise RuntimeError("gla_chunk_fwd failed: %d" % rc)
    torch.cuda.synchronize()
    marks[0].record(stream)
    for i in range(n_calls):
        rc = r.fn(*r.args[i % len(r.args)])
        if rc != 0:
            raise RuntimeError("gla_chunk_fwd failed: %d" % rc)
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    per_call = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(n_calls))
    pc = lambda f: per_call[min(n_calls - 1, int(f * (n_calls - 1) + 0.5))]
    mean["per_call_ms"] = {"median": pc(0.5), "p10": pc(0.1), "p90": pc(0.9), "calls": n_calls,
                           "warmup_calls": 20}
    if extras:
        # per-step spread: plain event records between steps (no per-kernel hook)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        for e in marks:
            e.record(stream)
        torch.cuda.synchronize()
        marks[0].record(stream)
        for s in range(steps):
            r.step()
            marks[s + 1].record(stream)
        torch.cuda.synchronize()
        per = sorted(marks[s].elapsed_time(marks[s + 1]) for s in range(steps))
        pick = lambda f: per[min(len(per) - 1, int(f * (len(per) - 1) + 0.5))]
        mean["step_ms"] = {"median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9)}
        # warm: the first set's inputs for every call of the step
        args = [r.args[0][:4] + a[4:] for a in r.args[:ncall]]
        for _ in range(warmup):
            for a in args:
                r.fn(*a)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            for a in args:
                rc = r.fn(*a)
                if rc != 0:
                    raise RuntimeError("gla_chunk_fwd failed: %d" % rc)
        torch.cuda.synchronize()
        mean["warm_ms_step"] = (time.perf_counter() - t0) * 1e3 / steps
    return r, ms_step, mean


SWIGLU_WORKLOAD = "swiglu_hires16.4k"


def swiglu_bytes(swl):
    """Algorithmic bytes of one Spatial SwiGLU call: read gate and value, write
    out (2 bytes per channel each, 6 * C per token), plus the 3x3 weights and
    the bias."""
    return swl.B * swl.T * swl.C * 2 * 3 + swl.C * 10 * 2


class SwigluRunner:
    """Device copies of the Spatial SwiGLU inputs, cycled across calls like Runner."""

    def __init__(self, swl, torch, min_sets_bytes=2 * LLC_BYTES):
        from recurrent_vision_token_amd import _lib
        from recurrent_vision_token_amd.workloads import make_swiglu_inputs
        self.swl = swl
        dev = torch.device("cuda:0")
        self.host = make_swiglu_inputs(swl.B, swl.H, swl.W, swl.C, seed=swl.seed)
        g, v, w, b = self.host
        wt, bt = torch.from_numpy(w).to(dev), torch.from_numpy(b).to(dev)
        reps = max(2, math.ceil(min_sets_bytes / swiglu_bytes(swl)))
        self.sets = []
        for _ in range(reps):
            gt, vt = torch.from_numpy(g).to(dev), torch.from_numpy(v).to(dev)
            self.sets.append((gt, vt, torch.empty_like(gt)))
        self.keep = (wt, bt)
        stream = torch.cuda.current_stream(dev).cuda_stream
        self.fn = _lib.load().gla_spatial_swiglu
        self.args = [(gt.data_ptr(), vt.data_ptr(), swl.C, wt.data_ptr(), bt.data_ptr(), swl.B,
                      swl.H, swl.W, swl.C, o.data_ptr(), stream) for (gt, vt, o) in self.sets]
        self.cursor = 0
        torch.cuda.synchronize()

    def step(self, events=None):
        from recurrent_vision_token_amd import _lib
        a = self.args[self.cursor]
        self.cursor = (self.cursor + 1) % len(self.sets)
        if events is not None:
            rc = _lib.set_kernel_events([e.cuda_event for e in events])
            if rc != 0:
                raise RuntimeError("gla_set_kernel_events failed: %d" % rc)
        rc = self.fn(*a)
        if rc != 0:
            raise RuntimeError("gla_spatial_swiglu failed: %d" % rc)


def time_swiglu(swl, torch, steps, warmup):
    """Wall-clock loop of single calls, then an event-instrumented pass for the
    kernel's own duration (recorded by its dispatch, on the call's stream)."""
    r = SwigluRunner(swl, torch)
    log("[bench] %s: %d device input sets (%.0f MB)" %
        (swl.name, len(r.sets), len(r.sets) * swiglu_bytes(swl) / 1e6))
    for _ in range(warmup):
        r.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        r.step()
    torch.cuda.synchronize()
    ms_call = (time.perf_counter() - t0) * 1e3 / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    stream = torch.cuda.current_stream()
    for per_call in evs:
        for e in per_call:
            e.record(stream)
    torch.cuda.synchronize()
    for e in evs:
        r.step(e)
    torch.cuda.synchronize()
    k_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / len(evs)
    return r, ms_call, k_ms


def swiglu_cpu_baseline(swl, host):
    """The Spatial SwiGLU oracle as it stands (numpy float64) on the full image."""
    from oracle import spatial_swiglu
    g, v, w, b = host
    t0 = time.perf_counter()
    c0 = time.process_time()
    spatial_swiglu(g, v, w, b)
    wall = time.perf_counter() - t0
    cores = max(1, int(round((time.process_time() - c0) / wall)))
    return {"value": swl.B * swl.T / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "one full call (%s, numpy float64), %.1f s wall" % (swl.name, wall)}


def swiglu_summary(swl, ms_call, k_ms, cpu):
    nb = swiglu_bytes(swl)
    ach = nb / (k_ms * 1e-3) / 1e9
    return {
        "entry": "gla_spatial_swiglu: silu(gate) * (3x3 depthwise conv of value + bias)",
        "workload": "%s: B=%d, %dx%d grid (%d tokens), C=%d channels, fp16, gate/value "
                    "~ N(0,1), weights/bias ~ U(-1/3, 1/3), seed %d" %
                    (swl.name, swl.B, swl.H, swl.W, swl.T, swl.C, swl.seed),
        "value": swl.B * swl.T / (ms_call * 1e-3),
        "unit": "tokens/s",
        "ms_per_call": round(ms_call, 4),
        "dtype": "f16",
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profiles(SWIGLU_WORKLOAD, "spatial_swiglu")
                     if swl.name == SWIGLU_WORKLOAD else None,
                     "traffic_counts": TRAFFIC_NOTE,
                     "kernel": "spatial_swiglu", "algorithmic_bytes_per_launch": nb,
                     "avg_launch_us": round(k_ms * 1e3, 2),
                     "note": "one kernel per call: its bytes are the method's"},
        "cpu_baseline": cpu,
    }


class BwdRunner:
    """Device copies of a workload's inputs plus output gradients, cycled
    across backward calls like Runner; every call passes an initial state and
    a final-state gradient and asks for all five gradients."""

    def __init__(self, wl, torch, min_sets_bytes=2 * LLC_BYTES):
        from recurrent_vision_token_amd import _lib
        from recurrent_vision_token_amd.workloads import make_bwd_inputs
        self.wl = wl
        dev = torch.device("cuda:0")
        self.host = {}
        for seed, _ in wl.calls:
            if seed not in self.host:
                self.host[seed] = list(host_inputs(wl, seed)) + list(make_bwd_inputs(
                    wl.B, wl.heads, wl.H, wl.W, wl.d_v, wl.d_k, seed=seed + 1000))
        per_call = bwd_bytes(wl)["call"]
        reps = max(1, math.ceil(min_sets_bytes / (per_call * len(wl.calls))))
        self.sets = []
        for _ in range(reps):
            for seed, d in wl.calls:
                x = [torch.from_numpy(a).to(dev) for a in self.host[seed]]
                outs = [torch.empty_like(x[i]) for i in (0, 1, 2, 3)] + [torch.empty_like(x[6])]
                self.sets.append((x, outs, d))
        stream = torch.cuda.current_stream(dev).cuda_stream
        self.fn = _lib.load().gla_chunk_bwd
        self.args = [tuple(t.data_ptr() for t in x[:5]) + (x[5].data_ptr(), x[6].data_ptr(), d,
                                                           wl.B, wl.heads, wl.H, wl.W, wl.d_k,
                                                           wl.d_v, wl.chunk) +
                     tuple(o.data_ptr() for o in outs) + (stream,)
                     for (x, outs, d) in self.sets]
        self.cursor = 0
        torch.cuda.synchronize()

    def step(self, events=None):
        from recurrent_vision_token_amd import _lib
        for c in range(len(self.wl.calls)):
            a = self.args[self.cursor]
            self.cursor = (self.cursor + 1) % len(self.sets)
            if events is not None:
                rc = _lib.set_kernel_events([e.cuda_event for e in events[c]])
                if rc != 0:
                    raise RuntimeError("gla_set_kernel_events failed: %d" % rc)
            rc = self.fn(*a)
            if rc != 0:
                raise RuntimeError("gla_chunk_bwd failed: %d" % rc)


def bwd_bytes(wl):
    """Algorithmic bytes of one backward call: read q, k, v, log_alpha, d_out,
    write dq, dk, dv, dlog_alpha (fp16), the states in and out (fp32); and the
    chunk kernel's own traffic, which adds the forward and adjoint state of
    every chunk (fp16) to the tensors."""
    th = wl.B * wl.heads * wl.T
    bh = wl.B * wl.heads
    st = wl.d_k * wl.d_v * 4
    n = -(-wl.T // wl.chunk)
    tensors = th * 2 * (3 * wl.d_k + 2 * wl.d_v) + th * 2 * (3 * wl.d_k + wl.d_v)
    # every chunk reads its forward and adjoint entry states (float16)
    return {"call": tensors + 3 * bh * st, "chunk_bwd": tensors + 2 * bh * n * (st // 2)}


def time_bwd(wl, torch, steps, warmup):
    r = BwdRunner(wl, torch)
    ncall = len(wl.calls)
    log("[bench] %s backward: %d device sets (%.0f MB), %d calls/step" %
        (wl.name, len(r.sets), len(r.sets) * bwd_bytes(wl)["call"] / 1e6, ncall))
    for _ in range(warmup):
        r.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        r.step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(ncall)]
           for _ in range(steps)]
    stream = torch.cuda.current_stream()
    for per_step in evs:
        for per_call in per_step:
            for e in per_call:
                e.record(stream)
    torch.cuda.synchronize()
    for s_ in range(steps):
        r.step(evs[s_])
    torch.cuda.synchronize()
    flat = [e for per_step in evs for e in per_step]
    k_ms = {"state_summaries": sum(e[0].elapsed_time(e[1]) for e in flat) / len(flat),
            "state_scans": sum(e[2].elapsed_time(e[3]) for e in flat) / len(flat),
            "chunk_bwd": sum(e[4].elapsed_time(e[5]) for e in flat) / len(flat),
            "call": sum(e[0].elapsed_time(e[5]) for e in flat) / len(flat)}
    return r, ms_step, k_ms


def bwd_cpu_baseline(wl, host):
    """The backward oracle as it stands on one full call of the workload."""
    from oracle import gla_backward
    seed, d = wl.calls[0]
    q, k, v, la, do, dfin, init = host[seed]
    t0 = time.perf_counter()
    c0 = time.process_time()
    gla_backward(q, k, v, la, do, d, d_final_state=dfin, initial_state=init)
    wall = time.perf_counter() - t0
    cores = max(1, int(round((time.process_time() - c0) / wall)))
    return {"value": wl.B * wl.T / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "one full backward call (%s, direction %d, numpy float64 reverse token "
                      "loop), %.1f s wall" % (wl.name, d, wall)}


def bwd_summary(wl, ms_step, k_ms, cpu):
    nb = bwd_bytes(wl)
    # A wider head runs as a grid of 64 x 64 blocks, each with the three
    # kernels, in order on the stream; the kernel events then bracket the
    # last block's kernels, and the call's chunk kernels take `blocks` times
    # that (the last block also adds its partial gradients to the earlier
    # ones', so this slightly overstates them).
    blocks = (wl.d_k // 64) * (wl.d_v // 64)
    # the call's method bytes over the dominant kernel's launches; its own
    # bytes (state reads included; one block only) separately
    ach = nb["call"] / (blocks * k_ms["chunk_bwd"] * 1e-3) / 1e9
    own = nb["chunk_bwd"] / (k_ms["chunk_bwd"] * 1e-3) / 1e9 if blocks == 1 else None
    wall_call_ms = ms_step / len(wl.calls)
    path = nb["call"] / (wall_call_ms * 1e-3) / 1e9
    tokens = len(wl.calls) * wl.B * wl.T
    return {
        "entry": "gla_chunk_bwd: dq, dk, dv, dlog_alpha, d_initial_state (fp16, fp32 states)",
        "workload": describe(wl) + "; d_out ~ N(0,1), d_final_state and initial_state ~ N(0,1)/8",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "ms_per_step": round(ms_step, 4),
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profiles(wl.name, "chunk_bwd"),
                     "traffic_counts": TRAFFIC_NOTE,
                     "kernel": "chunk_bwd" if blocks == 1 else
                               "chunk_bwd (%d launches per call, one per 64 x 64 block)" % blocks,
                     "algorithmic_bytes_per_launch": nb["call"] // blocks,
                     "avg_launch_us": round(k_ms["chunk_bwd"] * 1e3, 2),
                     "kernel_bytes_per_launch": nb["chunk_bwd"] if blocks == 1 else None,
                     "dominant_kernel_frac": round(own / HBM_PEAK_GBPS, 4) if own else None},
        "path": {"wall_us_per_call": round(wall_call_ms * 1e3, 2),
                 "event_us_per_call": round(k_ms["call"] * 1e3, 2),
                 "algorithmic_bytes_per_call": nb["call"],
                 "achieved_GBps": round(path, 1), "hbm_frac": round(path / HBM_PEAK_GBPS, 4),
                 "kernel_us": {k: round(v * 1e3, 2) for k, v in k_ms.items() if k != "call"},
                 "kernel_us_of": "the call" if blocks == 1 else "its last 64 x 64 block"},
        "cpu_baseline": cpu,
    }


SAGA_WORKLOAD = "saga_hires16.4k"


def saga_bytes(swl):
    """Algorithmic bytes of one SAGA call: read q, k, v and the two gates,
    write out (fp16); and of its dominant kernel, the map accumulation, which
    reads k, v and the gates."""
    th = swl.B * swl.heads * swl.N
    return th * 2 * (3 * swl.d_k + 3 * swl.d_v), th * 2 * (2 * swl.d_k + 2 * swl.d_v)


class SagaRunner:
    """Device copies of the SAGA inputs, cycled across calls like Runner."""

    def __init__(self, swl, torch, min_sets_bytes=2 * LLC_BYTES):
        from recurrent_vision_token_amd import _lib
        from recurrent_vision_token_amd.workloads import make_saga_inputs
        self.swl = swl
        dev = torch.device("cuda:0")
        self.host = make_saga_inputs(swl.B, swl.heads, swl.N, swl.d_k, swl.d_v, seed=swl.seed)
        reps = max(2, math.ceil(min_sets_bytes / saga_bytes(swl)[0]))
        self.sets = []
        for _ in range(reps):
            t = [torch.from_numpy(x).to(dev) for x in self.host]
            self.sets.append((t, torch.empty_like(t[2])))
        stream = torch.cuda.current_stream(dev).cuda_stream
        self.fn = _lib.load().gla_saga_fwd
        self.args = [tuple(x.data_ptr() for x in t) + (swl.B, swl.heads, swl.N, swl.d_k, swl.d_v,
                                                       o.data_ptr(), None, stream)
                     for (t, o) in self.sets]
        self.cursor = 0
        torch.cuda.synchronize()

    def step(self, events=None):
        from recurrent_vision_token_amd import _lib
        a = self.args[self.cursor]
        self.cursor = (self.cursor + 1) % len(self.sets)
        if events is not None:
            rc = _lib.set_kernel_events([e.cuda_event for e in events])
            if rc != 0:
                raise RuntimeError("gla_set_kernel_events failed: %d" % rc)
        rc = self.fn(*a)
        if rc != 0:
            raise RuntimeError("gla_saga_fwd failed: %d" % rc)


def time_saga(swl, torch, steps, warmup):
    """Wall-clock loop of single calls, then an event-instrumented pass for the
    three kernels' own durations."""
    r = SagaRunner(swl, torch)
    log("[bench] %s: %d device input sets (%.0f MB)" %
        (swl.name, len(r.sets), len(r.sets) * saga_bytes(swl)[0] / 1e6))
    for _ in range(warmup):
        r.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        r.step()
    torch.cuda.synchronize()
    ms_call = (time.perf_counter() - t0) * 1e3 / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    stream = torch.cuda.current_stream()
    for per_call in evs:
        for e in per_call:
            e.record(stream)
    torch.cuda.synchronize()
    for e in evs:
        r.step(e)
    torch.cuda.synchronize()
    names = ("saga_kv_partial", "saga_kv_reduce", "saga_out")
    k_ms = {n: sum(e[2 * i].elapsed_time(e[2 * i + 1]) for e in evs) / len(evs)
            for i, n in enumerate(names)}
    k_ms["call"] = sum(e[0].elapsed_time(e[5]) for e in evs) / len(evs)
    return r, ms_call, k_ms


def saga_cpu_baseline(swl, host):
    """The SAGA oracle as it stands (numpy float64 matrix products) on the full workload."""
    from oracle import saga_forward
    t0 = time.perf_counter()
    c0 = time.process_time()
    saga_forward(*host)
    wall = time.perf_counter() - t0
    cores = max(1, int(round((time.process_time() - c0) / wall)))
    return {"value": swl.B * swl.N / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "one full call (%s, numpy float64), %.2f s wall" % (swl.name, wall)}


def saga_summary(swl, ms_call, k_ms, cpu):
    # the dominant kernel (map accumulation) moves only k, v and the two gates,
    # all of them method bytes; q and out belong to the output kernel, so the
    # roofline takes the kernel's own bytes and the whole call goes to `path`
    total, acc = saga_bytes(swl)
    ach = acc / (k_ms["saga_kv_partial"] * 1e-3) / 1e9
    path = total / (ms_call * 1e-3) / 1e9
    return {
        "entry": "gla_saga_fwd: O = Q [(K*A)^T (V*B)], non-causal",
        "workload": "%s: B=%d, heads=%d, N=%d tokens, d_k=%d, d_v=%d, fp16, q/k/v ~ N(0,1)/8, "
                    "gates sigmoid(N(0,1)), seed %d" %
                    (swl.name, swl.B, swl.heads, swl.N, swl.d_k, swl.d_v, swl.seed),
        "value": swl.B * swl.N / (ms_call * 1e-3),
        "unit": "tokens/s",
        "ms_per_call": round(ms_call, 4),
        "dtype": "f16",
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profiles(SAGA_WORKLOAD, "saga_kv_partial")
                     if swl.name == SAGA_WORKLOAD else None,
                     "traffic_counts": TRAFFIC_NOTE,
                     "kernel": "saga_kv_partial", "algorithmic_bytes_per_launch": acc,
                     "avg_launch_us": round(k_ms["saga_kv_partial"] * 1e3, 2),
                     "note": "the kernel's reads are all method bytes (k, v, gates)"},
        "path": {"wall_us_per_call": round(ms_call * 1e3, 2),
                 "event_us_per_call": round(k_ms["call"] * 1e3, 2), "algorithmic_bytes_per_call": total,
                 "achieved_GBps": round(path, 1), "hbm_frac": round(path / HBM_PEAK_GBPS, 4),
                 "kernel_us": {k: round(v * 1e3, 2) for k, v in k_ms.items() if k != "call"}},
        "cpu_baseline": cpu,
    }


def plan_of(wl):
    """(n_spans, kernels) of the forward call on the current device."""
    from recurrent_vision_token_amd import _lib
    _, ns, kernels = _lib.plan_forward(wl.dtype, wl.B, wl.heads, wl.H, wl.W, wl.d_k, wl.d_v, wl.chunk)
    return ns, kernels


TRAFFIC_NOTE = ("L2-miss bytes per launch: FETCH_SIZE + WRITE_SIZE, scaled against a copy "
                "kernel of known size; misses served by the Infinity Cache count too")


def traffic_from_profiles(wl_name, kernel):
    """L2-miss bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-scaled) from
    committed counter runs, if they match this source."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % wl_name)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        k = rec["kernels"][kernel]
        if k.get("kernel_source_sha256") != source_hash(kernel):
            return None
        return k["hbm_bytes_per_launch"]
    except Exception:
        return None


def cpu_baseline(wl, host, budget_s=12.0):
    """The oracle as it stands, on a bounded sample of the same workload.
    Also returns its outputs, [(call index, out, final_state)]."""
    from oracle import gla_forward
    t0 = time.perf_counter()
    c0 = time.process_time()
    tokens = 0
    done = 0
    refs = []
    for i, (seed, d) in enumerate(wl.calls):
        q, k, v, la = host[seed]
        o, f = gla_forward(q, k, v, la, d)
        refs.append((i, o, f))
        tokens += wl.B * wl.T
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    wall = time.perf_counter() - t0
    cpu = time.process_time() - c0
    cores = max(1, int(round(cpu / wall)))
    return ({"value": tokens / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
             "sample": "%d of the %d calls of one step (%s, full size, numpy float64 token loop), "
                       "%.1f s wall" % (done, len(wl.calls), wl.name, wall),
             "host_cpus": {"os_cpu_count": os.cpu_count(),
                           "sched_affinity": len(os.sched_getaffinity(0))}}, refs)


def _pool_ready(_):
    time.sleep(0.3)  # hold the worker, so that every worker of the pool starts now
    return os.getpid()


def _oracle_slice(args):
    from oracle import gla_forward
    q, k, v, la, d = args
    return gla_forward(q, k, v, la, d)


def start_oracle_pool(max_workers=16):
    """Worker processes for the all-cores oracle figure, started (fresh
    interpreters, spawn) before this process touches the GPU; at most 16, the
    CPU share of one GPU."""
    import concurrent.futures
    import multiprocessing
    n = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    pool = concurrent.futures.ProcessPoolExecutor(
        max_workers=n, mp_context=multiprocessing.get_context("spawn"))
    pids = set(pool.map(_pool_ready, range(n)))
    return pool, len(pids)


def cpu_baseline_pool(wl, host, pool, workers):
    """The same oracle over independent (batch, head) sequences in a process
    pool: the fair all-cores CPU figure (one step of the workload)."""
    t0 = time.perf_counter()
    tasks = []
    for seed, d in wl.calls:
        q, k, v, la = host[seed]
        for b in range(wl.B):
            for h in range(wl.heads):
                sl = (slice(b, b + 1), slice(h, h + 1))
                tasks.append((q[sl], k[sl], v[sl], la[sl], d))
    for _ in pool.map(_oracle_slice, tasks):
        pass
    wall = time.perf_counter() - t0
    return {"value": len(wl.calls) * wl.B * wl.T / wall, "unit": "tokens/s", "cores": workers,
            "kind": "oracle",
            "sample": "one step (%d calls) of %s, %d (batch, head) sequences per call spread over "
                      "%d worker processes, %.1f s wall" % (len(wl.calls), wl.name, wl.B * wl.heads,
                                                            workers, wall)}


def gpu_parity(runner, refs, torch):
    """Errors of the GPU outputs against the oracle's, for the calls the CPU
    baseline computed: each call re-run once on its own input set."""
    import numpy as np
    worst = {"out": {"rel_fro": 0.0, "max_rel": 0.0, "cosine_min": 1.0},
             "final_state": {"rel_fro": 0.0, "max_rel": 0.0, "cosine_min": 1.0}}
    for i, ro, rf in refs:
        rc = runner.fn(*runner.args[i])
        if rc != 0:
            raise RuntimeError("gla_chunk_fwd failed: %d" % rc)
        torch.cuda.synchronize()
        q, k, v, la, out, fs = runner.sets[i][:6]
        for name, got, ref in (("out", out, ro), ("final_state", fs, rf)):
            g = got.float().cpu().numpy().astype(np.float64).ravel()
            r = ref.ravel()
            w = worst[name]
            w["rel_fro"] = max(w["rel_fro"], float(np.linalg.norm(g - r) / np.linalg.norm(r)))
            w["max_rel"] = max(w["max_rel"], float(np.abs(g - r).max() / np.abs(r).max()))
            w["cosine_min"] = min(w["cosine_min"],
                                  float(g @ r / (np.linalg.norm(g) * np.linalg.norm(r))))
    for w in worst.values():
        for k in w:
            w[k] = float("%.4g" % w[k])
    return dict(worst, calls_checked=len(refs),
                bar="rel_fro <= 5e-3 and max_rel <= 2e-2 (fp16); the pages report cosine >= 0.9989")


def copy_bandwidth(torch, mb=1024, reps=20):
    """Device-to-device copy rate (read + write bytes per second): the
    practical streaming ceiling of this machine."""
    n = (mb << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def describe(wl):
    dirs = sorted(set(d for _, d in wl.calls))
    return ("%s: B=%d, heads=%d, %dx%d grid (%d tokens), d_k=%d, d_v=%d, chunk=%d, %s, "
            "gate_std=%g, seeds %s, scan dirs %s, %d calls per step" %
            (wl.name, wl.B, wl.heads, wl.H, wl.W, wl.T, wl.d_k, wl.d_v, wl.chunk, wl.dtype,
             wl.gate_std, sorted(set(s for s, _ in wl.calls)), dirs, len(wl.calls)))


def summarize(wl, ms_step, mean, ext=False):
    alg = algorithmic(wl)
    if ext:  # the initial state is read once more per (b, h)
        alg["bytes"] += wl.B * wl.heads * wl.d_k * wl.d_v * 4
    ncall = len(wl.calls)
    tokens_step = ncall * wl.B * wl.T
    spans, kernels = plan_of(wl)
    kb = kernel_bytes(wl, spans, kernels)
    if ext:
        kb["span_scan" if kernels == 3 else "chunk_output"] += wl.B * wl.heads * wl.d_k * wl.d_v * 4
    present = [k for k in kb if mean[k] > 0]
    dom = max(present, key=lambda k: mean[k])
    # the call's method bytes over the dominant kernel's launch (one launch
    # covers every token and head of the call), and that kernel's own bytes
    ach = alg["bytes"] / (mean[dom] * 1e-3) / 1e9
    own = kb[dom] / (mean[dom] * 1e-3) / 1e9
    wall_call_ms = ms_step / ncall
    path_gbps = alg["bytes"] / (wall_call_ms * 1e-3) / 1e9
    out = {
        "tokens_per_step": tokens_step,
        "value": tokens_step / (ms_step * 1e-3),
        "dominant": dom,
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": traffic_from_profiles(wl.name, dom),
                     "traffic_counts": TRAFFIC_NOTE,
                     "kernel": dom, "algorithmic_bytes_per_launch": alg["bytes"],
                     "avg_launch_us": round(mean[dom] * 1e3, 2),
                     "kernel_bytes_per_launch": kb[dom],
                     "dominant_kernel_frac": round(own / HBM_PEAK_GBPS, 4)},
        # whole call at the timed loop's wall-clock rate (the instrumented pass
        # spaces its launches out: event_us_per_call is first summary start to
        # last output stop there)
        "path": {"wall_us_per_call": round(wall_call_ms * 1e3, 2),
                 "event_us_per_call": round(mean["call"] * 1e3, 2),
                 "algorithmic_bytes_per_call": alg["bytes"],
                 "achieved_GBps": round(path_gbps, 1),
                 "hbm_frac": round(path_gbps / HBM_PEAK_GBPS, 4),
                 "mfma_frac": round(alg["flops"] / (wall_call_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                 "kernel_us": {k: round(mean[k] * 1e3, 2) for k in ("span_summary", "span_scan", "chunk_output")},
                 "n_spans": spans, "kernels": kernels},
    }
    if "per_call_ms" in mean:
        m = mean["per_call_ms"]
        out["per_call_us"] = {"median": round(m["median"] * 1e3, 2), "p10": round(m["p10"] * 1e3, 2),
                              "p90": round(m["p90"] * 1e3, 2), "calls": m["calls"],
                              "warmup_calls": m["warmup_calls"],
                              "protocol": "event pair around every call, median"}
    if "step_ms" in mean:
        out["step_ms"] = {k: round(v, 4) for k, v in mean["step_ms"].items()}
    if "warm_ms_step" in mean:
        w = mean["warm_ms_step"]
        out["warm"] = {"ms_per_step": round(w, 4), "value": tokens_step / (w * 1e-3),
                       "note": "every call re-reads one resident input set (Infinity Cache hits)"}
    return out


def counters_to_traffic(fetch_dir, write_dir, copy_mb, workload, only=()):
    """Per-launch HBM bytes from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for
    the device copy of known size that the runs include.  Writes
    profiles/traffic_<workload>.json and prints a markdown summary."""
    import csv
    import statistics

    def per_kernel(d, counter):
        vals = {}
        for row in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            key = kernel_key(name)
            if key is None and "copy" in name.lower():
                key = "copy"
            if key is not None:
                vals.setdefault(key, []).append(float(row["Counter_Value"]))
        # the calibration copy is the largest copy dispatch of the run (input
        # uploads may show up as smaller copy kernels)
        return {k: (max(v) if k == "copy" else statistics.mean(v)) for k, v in vals.items()}

    f = per_kernel(fetch_dir, "FETCH_SIZE")
    w = per_kernel(write_dir, "WRITE_SIZE")
    copy_bytes = copy_mb << 20
    f_scale = copy_bytes / (f["copy"] * 1024.0)
    w_scale = copy_bytes / (w["copy"] * 1024.0)
    lines = ["| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | L2-miss read (MB) | L2-miss write (MB) | "
             "total (MB) |",
             "|---|---|---|---|---|---|"]
    recs = {}
    for k in KERNEL_NAMES:
        if k not in f or (only and k not in only):
            continue
        rd = f[k] * 1024.0 * f_scale
        wr = w[k] * 1024.0 * w_scale
        wl_name = (SWIGLU_WORKLOAD if k == "spatial_swiglu" else
                   SAGA_WORKLOAD if k.startswith("saga") else workload)
        rec = recs.setdefault(wl_name, {"workload": wl_name, "copy_bytes": copy_bytes,
                                        "fetch_scale": f_scale, "write_scale": w_scale,
                                        "kernels": {}})
        rec["kernels"][k] = {"fetch_kib": f[k], "write_kib": w[k], "hbm_read_bytes": rd,
                             "hbm_write_bytes": wr, "hbm_bytes_per_launch": rd + wr,
                             "kernel_source_sha256": source_hash(k)}
        lines.append("| %s | %.0f | %.0f | %.1f | %.1f | %.1f |" % (k, f[k], w[k], rd / 1e6, wr / 1e6,
                                                                  (rd + wr) / 1e6))
    for wl_name, rec in recs.items():
        out = os.path.join(ROOT, "profiles", "traffic_%s.json" % wl_name)
        if only and os.path.exists(out):
            old = json.load(open(out))
            old["kernels"].update(rec["kernels"])
            rec = old
        json.dump(rec, open(out, "w"), indent=1)
        print("wrote", out)
    print("copy kernel of %d bytes: FETCH_SIZE %.0f KiB (scale %.3f), WRITE_SIZE %.0f KiB (scale %.3f)"
          % (copy_bytes, f["copy"], f_scale, w["copy"], w_scale))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="hires16.4k")
    ap.add_argument("--secondary", default="gtr1.6k", help="'' to skip")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ext", action="store_true",
                    help="skip the extended entry point (fused gate + initial state) line")
    ap.add_argument("--swiglu", default=SWIGLU_WORKLOAD,
                    help="Spatial SwiGLU workload to time beside the attention path ('' to skip)")
    ap.add_argument("--no-img768", dest="img768", action="store_false",
                    help="skip the 768x768-image line (12 calls, one per block)")
    ap.add_argument("--no-sweep", dest="sweep", action="store_false",
                    help="skip the time-vs-token-count sweep")
    ap.add_argument("--no-batched", dest="batched", action="store_false",
                    help="skip the batched line (B=32, 16 heads, 64x64, d_k=128, d_v=64)")
    ap.add_argument("--no-extras", dest="extras", action="store_false",
                    help="skip the per-step spread and warm passes of the main workload")
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the backward pass line (gla_chunk_bwd on the main workload)")
    ap.add_argument("--saga", default=SAGA_WORKLOAD,
                    help="SAGA non-causal gated attention workload to time ('' to skip)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run one device-to-device copy of this many MB (a kernel of "
                         "known traffic, to scale hardware byte counters against)")
    ap.add_argument("--counters-to-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output folders into profiles/traffic_*.json")
    ap.add_argument("--traffic-kernels", default="",
                    help="comma-separated kernels to record with --counters-to-traffic "
                         "(default: all found; records of other kernels are kept)")
    args = ap.parse_args()

    if args.counters_to_traffic:
        counters_to_traffic(args.counters_to_traffic[0], args.counters_to_traffic[1],
                            args.copy_calibration_mb or 256, args.workload,
                            [k for k in args.traffic_kernels.split(",") if k])
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(sequences shard across GPUs with no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("RANK", "0")) != 0:
        return

    pool = None
    if not args.no_cpu_baseline:
        pool, pool_workers = start_oracle_pool()   # before any GPU call

    import torch
    from recurrent_vision_token_amd import load
    from recurrent_vision_token_amd.workloads import WORKLOADS, Workload

    load()  # fails loudly if the HIP library is not built
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a HIP device")

    if args.copy_calibration_mb > 0:
        n = args.copy_calibration_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: %d bytes read, %d bytes written" % (n, n))
        del src, dst

    wl = WORKLOADS[args.workload]
    runner, ms_step, mean = time_workload(wl, torch, args.steps, args.warmup, extras=args.extras)
    main_sum = summarize(wl, ms_step, mean)
    log("[bench] %s: %.3f ms/step, %.3e tokens/s, %.2f us/call, kernels %s" %
        (wl.name, ms_step, main_sum["value"], main_sum["path"]["wall_us_per_call"],
         main_sum["path"]["kernel_us"]))

    secondary = None
    if args.secondary:
        wl2 = WORKLOADS[args.secondary]
        _, ms2, mean2 = time_workload(wl2, torch, max(20, args.steps), max(5, args.warmup))
        s2 = summarize(wl2, ms2, mean2)
        secondary = {"workload": describe(wl2), "value": s2["value"], "unit": "tokens/s",
                     "ms_per_step": round(ms2, 4), "roofline": s2["roofline"], "path": s2["path"],
                     "per_call_us": s2.get("per_call_us")}
        log("[bench] %s: %.3f ms/step, %.3e tokens/s, %.2f us/call" %
            (wl2.name, ms2, s2["value"], s2["path"]["wall_us_per_call"]))

    img = None
    if args.img768:
        wl4 = WORKLOADS["img768"]
        _, ms4, mean4 = time_workload(wl4, torch, max(20, args.steps // 2), max(5, args.warmup))
        s4 = summarize(wl4, ms4, mean4)
        img = {"workload": describe(wl4), "gla_us_per_image": round(ms4 * 1e3, 2),
               "value": s4["value"], "unit": "tokens/s", "roofline": s4["roofline"],
               "path": s4["path"]}
        log("[bench] %s: %.1f us of attention per image (12 calls), %.3e tokens/s" %
            (wl4.name, ms4 * 1e3, s4["value"]))

    batched = None
    if args.batched:
        wl5 = WORKLOADS["batched"]
        _, ms5, mean5 = time_workload(wl5, torch, 40, 40)
        s5 = summarize(wl5, ms5, mean5)
        batched = {"workload": describe(wl5), "value": s5["value"], "unit": "tokens/s",
                   "ms_per_call": round(ms5, 4), "roofline": s5["roofline"], "path": s5["path"]}
        log("[bench] %s: %.1f us per call, %.3e tokens/s, output kernel %.0f GB/s" %
            (wl5.name, ms5 * 1e3, s5["value"], s5["roofline"]["achieved"]))

    sweep = None
    if args.sweep:
        sweep = []
        for side in (40, 48, 64, 80, 96, 128):
            wls = Workload("grid%d" % side, 1, 12, side, side, 64, 64, 64, "fp16", 1.0,
                           [1, 1, 1, 1], [0, 1, 2, 3])
            _, msw, meanw = time_workload(wls, torch, 50, 10)
            sw = summarize(wls, msw, meanw)
            sweep.append({"grid": "%dx%d" % (side, side), "tokens": side * side,
                          "us_per_call": round(msw * 1e3 / 4, 2), "tokens_per_s": sw["value"],
                          "path_hbm_frac": sw["path"]["hbm_frac"]})
        log("[bench] time vs tokens (B=1, 12 heads, 4 directions): %s" %
            ", ".join("%s %.1f us" % (x["grid"], x["us_per_call"]) for x in sweep))

    # (not in counter runs: their calibration copy must be the run's largest)
    copy_gbps = None if args.copy_calibration_mb > 0 else copy_bandwidth(torch)
    if copy_gbps:
        log("[bench] device copy: %.0f GB/s (read + write)" % copy_gbps)

    ext = None
    if not args.no_ext and wl.dtype == "fp16":
        _, ms3, mean3 = time_workload(wl, torch, args.steps, args.warmup, ext=True)
        s3 = summarize(wl, ms3, mean3, ext=True)
        ext = {"entry": "gla_chunk_fwd_ex: gate logits with fused logsigmoid(z)/16 activation, "
                        "initial state", "workload": describe(wl), "value": s3["value"],
               "unit": "tokens/s", "ms_per_step": round(ms3, 4), "roofline": s3["roofline"],
               "path": s3["path"]}
        log("[bench] %s extended entry: %.3f ms/step, %.3e tokens/s, kernels %s" %
            (wl.name, ms3, s3["value"], s3["path"]["kernel_us"]))

    bwd = None
    if not args.no_bwd and wl.dtype == "fp16" and wl.d_k == 64 and wl.d_v == 64:
        brun, ms_b, k_b = time_bwd(wl, torch, max(10, args.steps // 4), max(3, args.warmup // 4))
        b_cpu = None if args.no_cpu_baseline else bwd_cpu_baseline(wl, brun.host)
        bwd = bwd_summary(wl, ms_b, k_b, b_cpu)
        log("[bench] %s backward: %.3f ms/step, %.3e tokens/s, kernels %s" %
            (wl.name, ms_b, bwd["value"], bwd["path"]["kernel_us"]))
        del brun

    # the backward pass on the batched configuration (d_k = 128: two key blocks)
    bwd_batched = None
    if args.batched and not args.no_bwd:
        wl5 = WORKLOADS["batched"]
        brun, ms_b, k_b = time_bwd(wl5, torch, 10, 3)
        bwd_batched = bwd_summary(wl5, ms_b, k_b, None)
        log("[bench] %s backward: %.3f ms/call, %.3e tokens/s, kernels of its last block %s" %
            (wl5.name, ms_b, bwd_batched["value"], bwd_batched["path"]["kernel_us"]))
        del brun

    swiglu = None
    if args.swiglu:
        from recurrent_vision_token_amd.workloads import SWIGLU_WORKLOADS
        swl = SWIGLU_WORKLOADS[args.swiglu]
        srun, ms_sw, k_sw = time_swiglu(swl, torch, max(20, args.steps), max(5, args.warmup))
        sw_cpu = None if args.no_cpu_baseline else swiglu_cpu_baseline(swl, srun.host)
        swiglu = swiglu_summary(swl, ms_sw, k_sw, sw_cpu)
        log("[bench] %s: %.2f us/call wall, kernel %.2f us, %.3e tokens/s, %.0f GB/s" %
            (swl.name, ms_sw * 1e3, k_sw * 1e3, swiglu["value"], swiglu["roofline"]["achieved"]))
        del srun

    saga = None
    if args.saga:
        from recurrent_vision_token_amd.workloads import SAGA_WORKLOADS
        gwl = SAGA_WORKLOADS[args.saga]
        grun, ms_g, k_g = time_saga(gwl, torch, max(20, args.steps), max(5, args.warmup))
        g_cpu = None if args.no_cpu_baseline else saga_cpu_baseline(gwl, grun.host)
        saga = saga_summary(gwl, ms_g, k_g, g_cpu)
        log("[bench] %s: %.2f us/call wall, kernels %s, %.3e tokens/s" %
            (gwl.name, ms_g * 1e3, saga["path"]["kernel_us"], saga["value"]))
        del grun

    cpu = cpu_all = parity = None
    if not args.no_cpu_baseline:
        cpu, refs = cpu_baseline(wl, runner.host)
        log("[bench] cpu oracle: %.3e tokens/s on %d core(s)" % (cpu["value"], cpu["cores"]))
        parity = gpu_parity(runner, refs, torch)
        log("[bench] parity vs the oracle: %s" % parity)
        cpu_all = cpu_baseline_pool(wl, runner.host, pool, pool_workers)
        log("[bench] cpu oracle, all cores: %.3e tokens/s on %d processes" %
            (cpu_all["value"], cpu_all["cores"]))
        pool.shutdown()
    if copy_gbps:
        main_sum["roofline"]["frac_of_device_copy"] = round(
            main_sum["roofline"]["achieved"] / copy_gbps, 4)

    line = {
        "metric": METRIC,
        "value": main_sum["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if wl.dtype == "fp16" else "f32",
        "data": "synthetic",
        "config": {"workload": describe(wl), "tokens_per_step": main_sum["tokens_per_step"],
                   "input_copies_cycled": len(runner.sets)},
        "roofline": main_sum["roofline"],
        "path": main_sum["path"],
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "parity_vs_oracle": parity,
        "device_copy_GBps": round(copy_gbps, 1) if copy_gbps else None,
        "per_call_us": main_sum.get("per_call_us"),
        "step_ms": main_sum.get("step_ms"),
        "warm": main_sum.get("warm"),
        "secondary": secondary,
        "img768": img,
        "batched": batched,
        "time_vs_tokens": sweep,
        "fused_gate_initial_state": ext,
        "backward": bwd,
        "backward_batched": bwd_batched,
        "spatial_swiglu": swiglu,
        "saga": saga,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
