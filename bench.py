#!/usr/bin/env python3
"""Benchmark of one GPU's share of MoE EP layout -> dispatch -> combine.

One step = ep_get_dispatch_layout_notify (the layout and the dispatch's
notify phase of the same routing) + ep_dispatch_scatter + ep_combine (bf16
out) over one batch of the DeepSeek-V3-shaped prefill workload (T=4096
tokens, H=7168 bf16, E=256 experts in G=8 groups, top-8, uniform routing).
Inputs and the stand-in expert outputs are resident in HBM before the timed
region.

Cache policy of the headline: cold.  Before every step, warm-up and timed
alike, the GPU reads a 512 MiB buffer (twice the 256 MB MALL), so nothing of
the step's inputs is left in the MALL or the L2s; the read lies outside the
step's events.  (A read, not a write: written flush data would sit dirty in
the MALL and be written back during the step.)  Back to back, the source
rows x (58.7 MB) stay in the MALL from one step to the next: those warm
figures are reported beside the cold ones, under "warm".

Timing.  Timing-only HIP events (created without the system-scope cache
fence, which a default event adds between the kernels it separates) on the
launch stream at four points of every step: before the layout + notify call,
before the scatter, before the combine and after it.  Every figure is the
median over the K timed steps, with the min and the mean beside it.
value = T / median step time; ms_per_step = that median.  The timed region
is exactly K steps, each with its flush read, between two device
synchronisations; its wall time is timed_region_ms (about 1 s at the
default K = 3000, so that the GPU's busy time is long enough to be seen by a
sampler outside the process).

dispatch_combine = the scatter and the combine (the dispatch's notify phase
runs inside the layout call), between the events before the scatter and
after the combine; its bytes are the two calls' algorithmic bytes (one copy
per routed slot in each direction).

roofline: the step's dominant kernel (the scatter's or the combine's, the
longer one), its algorithmic bytes over its mean duration from the events
around it, against the 8 TB/s peak; traffic = the HBM bytes rocprofv3's
FETCH_SIZE and WRITE_SIZE counters measured for it (profiles/hbm_traffic.json)
while they were taken on the current kernel sources.  Ceilings: the read,
copy and 4 KiB-chunk write probes of include/moedisp_tools.h, timed in the
same run; each bulk kernel is also reported against the time its read and
write bytes take at the read probe's and the address-ordered write probe's
rates.

Further legs, each of which can be skipped: the other workloads (skewed
routing, fp8 decode, Mixtral shape; cold and warm), quantise-on-dispatch (FP32
and UE8M0 block scales), the group-deduplicated path, decode-step latency
(four calls, the small-batch path, and that path from a HIP graph).  The CPU
oracle, per phase on the host, is the reported baseline.

Prints one JSON line.  `--gpus` above 1 is refused: the library runs one
GPU's share of the path on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import socket
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine tokens/s and HBM GB/s (% of peak) at T=4096 H=7168 E=256 k=8"
COLD_FLUSH_BYTES = 512 << 20  # read before each step: twice the MALL
TARGET_FRAC = 0.70            # dispatch + combine against the 8 TB/s peak
PROFILE = "profiles/dsv3_prefill_bench_trace.md"  # rocprofv3 summary of `bench.py --profile-run`


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def make_inputs(wl, dev):
    import torch
    x = torch.from_numpy(np.ascontiguousarray(wl.x).view(np.uint8).reshape(wl.T, wl.row_bytes)).to(dev)
    xs = torch.from_numpy(wl.x_scales).to(dev) if wl.x_scales is not None else None
    idx = torch.from_numpy(wl.topk_idx).to(dev)
    w = torch.from_numpy(wl.topk_weights).to(dev)
    return x, xs, idx, w


class TimingEvent:
    """A HIP event for timing only, recorded on a given stream: created with
    hipEventDisableSystemFence, so recording it neither writes back nor
    invalidates the caches (a default event does both, which costs a few
    microseconds between the kernels it separates and slows the next one).
    Same runtime as torch's (the library loaded under the same soname)."""

    _hip = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes as C
        if TimingEvent._hip is None:
            hip = C.CDLL("libamdhip64.so.7")
            hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
            hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
            hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
            hip.hipEventDestroy.argtypes = [C.c_void_p]
            TimingEvent._hip = hip
        self._C = C
        self.e = C.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(C.byref(self.e), TimingEvent.FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = TimingEvent._hip.hipEventRecord(self.e, self._C.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        ms = self._C.c_float()
        rc = TimingEvent._hip.hipEventElapsedTime(self._C.byref(ms), self.e, end.e)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        e, self.e = getattr(self, "e", None), None
        if e and TimingEvent._hip is not None:
            TimingEvent._hip.hipEventDestroy(e)

    def __del__(self):
        # at interpreter exit the runtime or the class may already be gone
        try:
            self.close()
        except Exception:
            pass


class EventGrid:
    """rows x cols timing events, destroyed together."""

    def __init__(self, rows, cols):
        self.ev = [[TimingEvent() for _ in range(cols)] for _ in range(rows)]

    def __getitem__(self, i):
        return self.ev[i]

    def us(self, a, b) -> np.ndarray:
        """Microseconds from column a to column b, per row."""
        return np.array([r[a].elapsed_time(r[b]) for r in self.ev]) * 1e3

    def close(self):
        for r in self.ev:
            for e in r:
                e.close()
        self.ev = []


def stats(a) -> dict:
    a = np.asarray(a, dtype=np.float64)
    return {"median": float(np.median(a)), "min": float(a.min()), "mean": float(a.mean()), "n": int(a.size)}


def shape_of(M, W, wl):
    dt = M.FP8_E4M3 if wl.x_dtype == W.X_FP8 else M.BF16
    return M.moedisp_shape.make(wl.T, wl.H, wl.E, wl.G, wl.k, dt, wl.scale_block)


def box_info():
    import torch
    p = torch.cuda.get_device_properties(0)
    uuid = getattr(p, "uuid", None)
    return {"host": socket.gethostname(), "gpu": torch.cuda.get_device_name(0),
            "arch": getattr(p, "gcnArchName", "?"), "uuid": str(uuid) if uuid is not None else None,
            "cus": p.multi_processor_count}


def scatter_kernel_name(M, shape) -> str:
    return "moedisp_scatter_pull" if M.ep_plan_query(shape)["pull"] else "moedisp_scatter"


def run_gpu(cid, steps, warmup, dev, warm=True, split=True):
    """Cold steps of config `cid` (the timed region), then untimed passes:
    warm steps back to back, and cold steps of the separate calls (layout,
    notify, scatter, combine) for the per-call figures."""
    import torch
    import combine_ep_get_dispatch_amd as M
    from combine_ep_get_dispatch_amd import workloads as W
    from combine_ep_get_dispatch_amd.traffic import algorithmic_bytes

    wl = W.config(cid)
    shape = shape_of(M, W, wl)
    bufs = M.EpBuffers(shape, dev)
    x, xs, idx, w = make_inputs(wl, dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)

    # one dispatch to size the stand-in expert outputs (outside timing)
    bufs.layout(idx)
    bufs.dispatch(x, xs, idx, w)
    st = bufs.status()
    if st:
        raise RuntimeError(f"device status {st} on config {cid}")
    R = int(bufs.expert_offsets[-1].item())
    offs = bufs.expert_offsets.cpu().numpy()
    eo = torch.zeros((wl.T * wl.k, wl.H), dtype=torch.bfloat16, device=dev)
    rs = bufs.recv_scales[:R] if bufs.recv_scales is not None else None
    eo[:R] = W.expert_outputs(wl, bufs.recv_x[:R], rs, W.row_experts(offs), device=dev)
    del rs

    stream = torch.cuda.current_stream()
    flush = torch.ones(COLD_FLUSH_BYTES, dtype=torch.uint8, device=dev).view(torch.int32)
    sink = torch.empty((), dtype=torch.int32, device=dev)

    def flush_caches():
        torch.amax(flush, dim=0, out=sink)

    # the step; `ev` (optional) gets events before layout_notify, before the
    # scatter, before the combine and after it
    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        bufs.layout_notify(idx, stream)
        if ev is not None:
            ev[1].record(stream)
        bufs.dispatch_scatter(x, xs, idx, w, stream)
        if ev is not None:
            ev[2].record(stream)
        bufs.combine(eo, out, M.BF16, True, stream)
        if ev is not None:
            ev[3].record(stream)

    def phases(g: EventGrid) -> dict:
        d = {"layout_notify_us": g.us(0, 1), "scatter_us": g.us(1, 2), "combine_us": g.us(2, 3),
             "dc_us": g.us(1, 3), "step_us": g.us(0, 3)}
        return {k: stats(v) for k, v in d.items()}

    # --- timed region: cold steps ---------------------------------------
    for _ in range(warmup):
        flush_caches()
        step()
    torch.cuda.synchronize()
    g = EventGrid(steps, 4)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        flush_caches()
        step(g[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    st = bufs.status()
    if st:
        raise RuntimeError(f"device status {st} after the timed steps on config {cid}")
    cold = phases(g)
    g.close()
    res_warm = None
    if warm:  # untimed: back to back
        for _ in range(max(2, warmup // 2)):
            step()
        g = EventGrid(steps, 4)
        torch.cuda.synchronize()
        for i in range(steps):
            step(g[i])
        torch.cuda.synchronize()
        res_warm = phases(g)
        g.close()
    calls = None
    if split:  # untimed, cold: the separate calls, events between every call
        n = min(steps, 50)
        g = EventGrid(n, 5)
        torch.cuda.synchronize()
        for i in range(n):
            flush_caches()
            g[i][0].record(stream)
            bufs.layout(idx, stream)
            g[i][1].record(stream)
            bufs.dispatch_notify(idx, stream)
            g[i][2].record(stream)
            bufs.dispatch_scatter(x, xs, idx, w, stream)
            g[i][3].record(stream)
            bufs.combine(eo, out, M.BF16, True, stream)
            g[i][4].record(stream)
        torch.cuda.synchronize()
        calls = {"layout_us": stats(g.us(0, 1)), "dispatch_notify_us": stats(g.us(1, 2)),
                 "dispatch_scatter_us": stats(g.us(2, 3)), "combine_us": stats(g.us(3, 4)),
                 "dispatch_us": stats(g.us(1, 3))}
        g.close()
    st = bufs.status()
    if st:
        raise RuntimeError(f"device status {st} after the untimed passes on config {cid}")
    x_elt = 1 if wl.x_dtype == W.X_FP8 else 2
    B = algorithmic_bytes(wl.T, wl.H, wl.E, wl.G, wl.k, R, x_elt, wl.scale_block)
    res = dict(config=cid, workload=wl.name, T=wl.T, H=wl.H, E=wl.E, G=wl.G, k=wl.k, x_dtype=wl.x_dtype, R=R,
               routing=wl.meta["routing"], mask_frac=wl.meta["mask_frac"], bytes=B,
               kernels={"scatter": scatter_kernel_name(M, shape), "combine": "moedisp_combine"},
               cold=cold, warm=res_warm, calls_cold=calls, timed_region_ms=(t1 - t0) * 1e3)
    del bufs, eo, out, x, xs, idx, w, flush, sink
    torch.cuda.empty_cache()
    return res


def dc_summary(res, which="cold"):
    """dispatch_combine figures of one pass of run_gpu."""
    from combine_ep_get_dispatch_amd.traffic import HBM_PEAK_GBPS
    B = res["bytes"]
    ph = res[which]
    dc_bytes = B["dispatch"] - B["notify"] + B["combine"]
    us = ph["dc_us"]["median"]
    gbps = dc_bytes / (us * 1e-6) / 1e9
    return {"us": us, "us_min": ph["dc_us"]["min"], "us_mean": ph["dc_us"]["mean"],
            "tokens_per_s": res["T"] / (us * 1e-6), "gbps": gbps, "frac": gbps / HBM_PEAK_GBPS,
            "frac_at_min": dc_bytes / (ph["dc_us"]["min"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, "bytes": dc_bytes,
            "scatter_us": ph["scatter_us"]["median"], "combine_us": ph["combine_us"]["median"],
            "calls": "ep_dispatch_scatter + ep_combine (the notify phase runs in ep_get_dispatch_layout_notify)"}


def page_conventions(res, which="cold"):
    """The bandwidth figures of the source page's own benchmark conventions,
    for context (not this line's metric): per phase, token bytes T*H*elt
    over the phase's time (the high-throughput bench counts the tokens sent,
    not the expanded receive layout), and per routed copy R*H*elt (the
    low-latency combine counts one copy per dispatched token, as dispatch
    does).  Phases: the scatter (the dispatch's copy) and the combine, cold
    medians."""
    ph = res[which]
    t_d = ph["scatter_us"]["median"] * 1e-6
    t_c = ph["combine_us"]["median"] * 1e-6
    elt = 1 if res["x_dtype"] == "fp8_e4m3" else 2
    tok = res["T"] * res["H"] * elt
    copies = res["R"] * res["H"] * elt
    out = res["R"] * res["H"] * 2
    return {"dispatch_us": t_d * 1e6, "combine_us": t_c * 1e6, "token_bytes": tok,
            "dispatch_token_gbps": tok / t_d / 1e9, "combine_token_gbps": res["T"] * res["H"] * 2 / t_c / 1e9,
            "copy_bytes": copies, "dispatch_copy_gbps": copies / t_d / 1e9, "combine_copy_gbps": out / t_c / 1e9}


def run_gpu_quant(cid, block, fmt, steps, warmup, dev):
    """Quantise-on-dispatch (notify + quantising scatter) on config `cid`,
    back to back; medians over `steps`."""
    import torch
    import combine_ep_get_dispatch_amd as M
    from combine_ep_get_dispatch_amd import workloads as W
    from combine_ep_get_dispatch_amd.traffic import HBM_PEAK_GBPS, algorithmic_bytes_quant

    wl = W.config(cid)
    bufs = M.EpBuffers(shape_of(M, W, wl), dev).enable_quant(block, fmt)
    x, _, idx, w = make_inputs(wl, dev)
    bufs.layout(idx)
    bufs.dispatch_quant(x, idx, w)
    if bufs.status():
        raise RuntimeError(f"device status on quantised config {cid}")
    R = int(bufs.expert_offsets[-1].item())
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        bufs.dispatch_notify(idx, stream)
        bufs.dispatch_scatter_quant(x, idx, w, stream)
    g = EventGrid(steps, 3)
    torch.cuda.synchronize()
    for i in range(steps):
        g[i][0].record(stream)
        bufs.dispatch_notify(idx, stream)
        g[i][1].record(stream)
        bufs.dispatch_scatter_quant(x, idx, w, stream)
        g[i][2].record(stream)
    torch.cuda.synchronize()
    if bufs.status():
        raise RuntimeError(f"device status after quantised steps on config {cid}")
    ntf, sct, dis = np.median(g.us(0, 1)), np.median(g.us(1, 2)), np.median(g.us(0, 2))
    g.close()
    B = algorithmic_bytes_quant(wl.T, wl.H, wl.E, wl.k, R, block, 4 if fmt == M.SCALE_FP32 else 1)
    res = dict(workload=wl.name, block=block, scale_fmt="fp32" if fmt == M.SCALE_FP32 else "ue8m0", R=R,
               cache="warm", notify_us=float(ntf), scatter_us=float(sct), dispatch_us=float(dis),
               dispatch_tokens_per_s=wl.T / (dis * 1e-6), dispatch_gbps=B["dispatch"] / (dis * 1e-6) / 1e9,
               scatter_gbps=B["scatter"] / (sct * 1e-6) / 1e9, bytes=B)
    res["scatter_frac"] = res["scatter_gbps"] / HBM_PEAK_GBPS
    del bufs, x, idx, w
    torch.cuda.empty_cache()
    return res


def run_gpu_groups(cid, steps, warmup, dev):
    """The group-deduplicated path on config `cid`: layout, group dispatch,
    local expert permutation, local reduce, group combine; back to back,
    medians over `steps`."""
    import torch
    import combine_ep_get_dispatch_amd as M
    from combine_ep_get_dispatch_amd import workloads as W
    from combine_ep_get_dispatch_amd.traffic import HBM_PEAK_GBPS, algorithmic_bytes_groups

    wl = W.config(cid)
    bufs = M.EpBuffers(shape_of(M, W, wl), dev)
    gb = M.EpGroupBuffers(bufs)
    x, xs, idx, w = make_inputs(wl, dev)
    bufs.layout(idx)
    gb.dispatch_groups(x, xs, idx, w)
    gb.permute()
    if bufs.status():
        raise RuntimeError(f"device status on the group path, config {cid}")
    R = int(bufs.expert_offsets[-1].item())
    Rg = int(gb.group_offsets[-1].item())
    eo = torch.zeros((wl.T * wl.k, wl.H), dtype=torch.bfloat16, device=dev)
    eo[:R] = bufs.recv_x[:R].view(torch.bfloat16) if wl.x_dtype == W.X_BF16 else 0
    part = torch.empty((gb.capacity, wl.H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    calls = [lambda: bufs.layout(idx, stream), lambda: gb.dispatch_groups(x, xs, idx, w, stream),
             lambda: gb.permute(stream), lambda: gb.reduce(eo, part, M.BF16, True, stream),
             lambda: gb.combine_groups(part, out, M.BF16, True, stream)]
    for _ in range(warmup):
        for c in calls:
            c()
    g = EventGrid(steps, len(calls) + 1)
    torch.cuda.synchronize()
    for i in range(steps):
        for j, c in enumerate(calls):
            g[i][j].record(stream)
            c()
        g[i][-1].record(stream)
    torch.cuda.synchronize()
    if bufs.status():
        raise RuntimeError(f"device status after the group path steps, config {cid}")
    us = np.array([np.median(g.us(j, j + 1)) for j in range(len(calls))])
    total = float(np.median(g.us(1, len(calls))))
    g.close()
    x_elt = 1 if wl.x_dtype == W.X_FP8 else 2
    B = algorithmic_bytes_groups(wl.T, wl.H, wl.E, wl.G, wl.k, R, Rg, x_elt, wl.scale_block)
    names = ["layout", "dispatch_groups", "permute", "reduce", "combine_groups"]
    res = dict(workload=wl.name, R=R, R_g=Rg, cache="warm", us={n: float(u) for n, u in zip(names, us)})
    res["gbps"] = {n: B[n] / (res["us"][n] * 1e-6) / 1e9 for n in names[1:]}
    res["frac"] = {n: v / HBM_PEAK_GBPS for n, v in res["gbps"].items()}
    res["dispatch_combine_us"] = total
    res["tokens_per_s"] = wl.T / (total * 1e-6)
    del bufs, gb, x, xs, idx, w, eo, part, out
    torch.cuda.empty_cache()
    return res


def run_gpu_decode(cid, steps, warmup, dev):
    """Decode-step latency on config `cid` (T=128): the four calls (layout,
    notify, scatter, combine), the small-batch path (layout + dispatch in one
    launch, then combine), and that path replayed from a captured HIP graph
    of 10 steps, also with the padded (low-latency) receive layout of T rows
    per expert; beside them, the same graph with two minimal kernels per step
    (the floor of two dependent launches on this part).  Each figure is the
    mean GPU time per step over back-to-back steps between two events."""
    import torch
    import combine_ep_get_dispatch_amd as M
    from combine_ep_get_dispatch_amd import workloads as W
    from combine_ep_get_dispatch_amd.traffic import algorithmic_bytes

    wl = W.config(cid)
    bufs = M.EpBuffers(shape_of(M, W, wl), dev)
    x, xs, idx, w = make_inputs(wl, dev)
    eo = torch.zeros((wl.T * wl.k, wl.H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
    bufs.layout_dispatch_small(x, xs, idx, w)
    R = int(bufs.expert_offsets[-1].item())
    if bufs.status():
        raise RuntimeError(f"device status on the decode path, config {cid}")

    def four(stream):
        bufs.layout(idx, stream)
        bufs.dispatch_notify(idx, stream)
        bufs.dispatch_scatter(x, xs, idx, w, stream)
        bufs.combine(eo, out, M.BF16, True, stream)

    def small(stream):
        bufs.layout_dispatch_small(x, xs, idx, w, stream)
        bufs.combine(eo, out, M.BF16, True, stream)

    def per_step(fn):
        stream = torch.cuda.current_stream()
        for _ in range(warmup):
            fn(stream)
        e0, e1 = TimingEvent(), TimingEvent()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        e0.close()
        e1.close()
        return us

    res = dict(workload=wl.name, T=wl.T, R=R, cache="warm")
    res["four_calls_us"] = per_step(four)
    res["small_us"] = per_step(small)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        small(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # a decode graph holds many steps; capture 10 so that the host's replay
    # call is not what is timed
    graph = torch.cuda.CUDAGraph()
    per_graph = 10
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            small(torch.cuda.current_stream())
    res["small_graph_us"] = per_step(lambda stream: graph.replay()) / per_graph
    # the same step with the padded layout: expert e's rows at [e*T, e*T + T)
    pb = M.EpPaddedBuffers(bufs, wl.T, wl.T, 0)
    eo_pad = torch.zeros((wl.E * wl.T, wl.H), dtype=torch.bfloat16, device=dev)

    def small_padded(stream):
        pb.dispatch(x, xs, idx, w, stream)
        pb.combine(eo_pad, out, M.BF16, True, stream)

    with torch.cuda.stream(side):
        small_padded(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph_pad = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_pad):
        for _ in range(per_graph):
            small_padded(torch.cuda.current_stream())
    res["small_padded_graph_us"] = per_step(lambda stream: graph_pad.replay()) / per_graph
    # the floor of a step of two dependent launches on this part: the same
    # graph of 10 steps with two minimal kernels per step (one workgroup
    # reading 16 KiB each)
    probe_src = torch.zeros(16384, dtype=torch.uint8, device=dev)
    probe_sink = torch.zeros(16, dtype=torch.uint8, device=dev)

    def two_minimal(stream):
        M.ep_probe_read(probe_src, 16384, probe_sink, stream)
        M.ep_probe_read(probe_src, 16384, probe_sink, stream)

    with torch.cuda.stream(side):
        two_minimal(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph_floor = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_floor):
        for _ in range(per_graph):
            two_minimal(torch.cuda.current_stream())
    res["graph_floor_us"] = per_step(lambda stream: graph_floor.replay()) / per_graph
    # the small-batch dispatch alone, events around each call
    stream = torch.cuda.current_stream()
    g = EventGrid(steps, 2)
    for i in range(steps):
        g[i][0].record(stream)
        bufs.layout_dispatch_small(x, xs, idx, w, stream)
        g[i][1].record(stream)
    torch.cuda.synchronize()
    res["small_dispatch_us"] = float(np.median(g.us(0, 1)))
    g.close()
    if bufs.status():
        raise RuntimeError(f"device status after the decode steps, config {cid}")
    x_elt = 1 if wl.x_dtype == W.X_FP8 else 2
    B = algorithmic_bytes(wl.T, wl.H, wl.E, wl.G, wl.k, R, x_elt, wl.scale_block)
    res["step_bytes"] = B["step"]
    res["tokens_per_s_graph"] = wl.T / (res["small_graph_us"] * 1e-6)
    # the step's bytes over its time above the two-launch floor
    above = res["small_graph_us"] - res["graph_floor_us"]
    res["above_floor_us"] = above
    res["above_floor_gbps"] = B["step"] / (above * 1e-6) / 1e9 if above > 0 else None
    del graph, graph_pad, graph_floor, pb, eo_pad, bufs, x, xs, idx, w, eo, out, probe_src, probe_sink
    torch.cuda.empty_cache()
    return res


def probe_ceilings(dev, reps=20):
    """Achievable HBM bandwidth in this run: the read-only stream and the
    copy of 1 GiB, and 4 KiB-chunk writes in address order and permuted over
    the size of the T=4096 H=7168 k=8 receive rows (GB/s, read + write bytes
    for the copy).  Medians of `reps` launches, events around each."""
    import torch
    import combine_ep_get_dispatch_amd as M
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    fill_n = 32768 * 14336
    stream = torch.cuda.current_stream()

    def rate(fn, nbytes):
        for _ in range(3):
            fn()
        g = EventGrid(reps, 2)
        torch.cuda.synchronize()
        for i in range(reps):
            g[i][0].record(stream)
            fn()
            g[i][1].record(stream)
        torch.cuda.synchronize()
        us = float(np.median(g.us(0, 1)))
        g.close()
        return nbytes / (us * 1e-6) / 1e9

    res = {"read_gbps": rate(lambda: M.ep_probe_read(src, n, sink), n),
           "copy_gbps": rate(lambda: M.ep_probe_copy(dst, src, n), 2 * n),
           "write_seq_4k_gbps": rate(lambda: M.ep_probe_fill(dst, fill_n, False), fill_n),
           "write_perm_4k_gbps": rate(lambda: M.ep_probe_fill(dst, fill_n, True), fill_n),
           "bytes": {"read": n, "copy": 2 * n, "write": fill_n}}
    del src, dst, sink
    torch.cuda.empty_cache()
    return res


def kernel_rw_bytes(B, T, H, k, R, x_elt, scale_block):
    """Read and write bytes of the scatter and the combine (the algorithmic
    accounting of traffic.algorithmic_bytes, split by direction)."""
    row = H * x_elt + ((H // scale_block) * 4 if scale_block else 0)
    scat_w = R * row + 2 * R * 4 + T * k * 4
    comb_w = T * H * 2
    scat = B["dispatch"] - B["notify"]
    return {"scatter": (scat - scat_w, scat_w), "combine": (B["combine"] - comb_w, comb_w)}


def cpu_baseline(reps: int = 3):
    """The CPU oracle (single-threaded C) on the DeepSeek-V3-shaped workload,
    each phase (layout, dispatch, combine) once untimed and then `reps`
    times; medians per phase, tokens/s of their sum."""
    import oracle
    from combine_ep_get_dispatch_amd import workloads as W
    import torch

    oracle.build(force=False)
    orc = oracle.get()
    wl = W.config(2)
    # stand-in expert outputs from one untimed oracle dispatch
    d = orc.dispatch(wl.x, wl.x_scales, wl.topk_idx, wl.topk_weights, wl.E)
    R = int(d["expert_offsets"][-1])
    eo = W.expert_outputs(wl, d["recv_x"][:R], None, W.row_experts(d["expert_offsets"]))
    eo_bits = eo.view(torch.int16).numpy().view(np.uint16)
    weights, s2r = d["recv_weights"][:R].copy(), d["slot_to_row"].copy()
    del d

    def timed(fn):
        fn()
        t = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            t.append(time.perf_counter() - t0)
        return {"median": float(np.median(t)), "min": float(np.min(t))}

    ph = {"layout": timed(lambda: orc.layout(wl.topk_idx, wl.E, wl.G)),
          "dispatch": timed(lambda: orc.dispatch(wl.x, wl.x_scales, wl.topk_idx, wl.topk_weights, wl.E)),
          "combine": timed(lambda: orc.combine(eo_bits, weights, s2r, want_f32=False, want_bf16=True))}
    per_step = sum(p["median"] for p in ph.values())
    try:
        cpu = subprocess.run(["lscpu"], capture_output=True, text=True).stdout
        model = next((l.split(":", 1)[1].strip() for l in cpu.splitlines() if l.startswith("Model name")), "?")
    except Exception:
        model = "?"
    return dict(value=wl.T / per_step, unit="tokens/s", cores=1, kind="oracle",
                sample=(f"the T=4096 H=7168 E=256 k=8 workload, each phase 1 untimed + {reps} timed runs, "
                        f"median per phase ({per_step:.2f} s per step); 1 thread of {os.cpu_count()} host cores "
                        f"({model})"),
                phases_s=ph, host_cores=os.cpu_count(), cpu_model=model)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload for the headline line (default 2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the bandwidth ceiling probes")
    ap.add_argument("--no-quant", action="store_true", help="skip the quantise-on-dispatch timings")
    ap.add_argument("--no-groups", action="store_true", help="skip the group-deduplicated path timings")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-latency timings")
    ap.add_argument("--no-warm", action="store_true", help="skip the warm (back-to-back) pass")
    ap.add_argument("--profile-run", action="store_true",
                    help="the headline config's cold steps only (every leg and pass above off): the command "
                         "whose rocprofv3 kernel trace the roofline entry is checked against")
    ap.add_argument("--profile-groups", action="store_true",
                    help="the group-deduplicated path's timed calls only, then the bandwidth probes (whose copy "
                         "calibrates the traffic counters); prints that leg's JSON, not the benchmark line: the "
                         "command whose rocprofv3 trace and counters the group path's profile holds")
    args = ap.parse_args()
    if args.profile_run:
        args.no_cpu_baseline = args.no_other_workloads = args.no_probe = True
        args.no_quant = args.no_groups = args.no_decode = args.no_warm = True

    if args.gpus != 1:
        print(f"bench.py runs one GPU's share of the path on one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    from combine_ep_get_dispatch_amd.traffic import HBM_PEAK_GBPS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.profile_groups:
        log("[bench] group-deduplicated path only")
        groups = run_gpu_groups(args.config, max(20, args.steps // 4), max(5, args.warmup // 4), dev)
        print(json.dumps({"group_path": groups, "ceilings_gbps": probe_ceilings(dev)}), flush=True)
        return
    log(f"[bench] config {args.config}: {args.warmup} warmup + {args.steps} timed cold steps")
    main_res = run_gpu(args.config, args.steps, args.warmup, dev, warm=not args.no_warm,
                       split=not args.profile_run)
    cold = main_res["cold"]
    step_us = cold["step_us"]["median"]
    log(f"[bench] config {args.config}: cold step {step_us:.1f} us (median), scatter "
        f"{cold['scatter_us']['median']:.1f} us, combine {cold['combine_us']['median']:.1f} us")

    others = {}
    if not args.no_other_workloads:
        for cid in (3, 4, 5):
            if cid == args.config:
                continue
            log(f"[bench] config {cid}")
            r = run_gpu(cid, max(20, args.steps // 4), max(5, args.warmup // 4), dev, warm=not args.no_warm,
                        split=False)
            others[r["workload"]] = {
                **{k: r[k] for k in ("T", "H", "E", "G", "k", "x_dtype", "routing", "R", "kernels")},
                "tokens_per_s": r["T"] / (r["cold"]["step_us"]["median"] * 1e-6),
                "step_us": r["cold"]["step_us"]["median"],
                "dispatch_combine": dc_summary(r), "phases_us": {k: v["median"] for k, v in r["cold"].items()},
                "warm": None if r["warm"] is None else {"dispatch_combine": dc_summary(r, "warm"),
                                                        "step_us": r["warm"]["step_us"]["median"]}}
    quant = {}
    if not args.no_quant:
        import combine_ep_get_dispatch_amd as M
        for block, fmt, tag in ((128, M.SCALE_FP32, "fp32_b128"), (32, M.SCALE_UE8M0, "ue8m0_b32")):
            log(f"[bench] quantised dispatch {tag}")
            quant[tag] = run_gpu_quant(args.config, block, fmt, max(20, args.steps // 4),
                                       max(5, args.warmup // 4), dev)
    groups = None
    if not args.no_groups:
        log("[bench] group-deduplicated path")
        groups = run_gpu_groups(args.config, max(20, args.steps // 4), max(5, args.warmup // 4), dev)
    decode = None
    if not args.no_decode:
        log("[bench] decode latency (config 4)")
        decode = run_gpu_decode(4, max(50, args.steps), max(10, args.warmup), dev)
    ceil = None
    if not args.no_probe:
        ceil = probe_ceilings(dev)
        log(f"[bench] ceilings: read {ceil['read_gbps']:.0f}, copy {ceil['copy_gbps']:.0f}, 4 KiB writes "
            f"{ceil['write_seq_4k_gbps']:.0f} in order / {ceil['write_perm_4k_gbps']:.0f} permuted GB/s")

    # dominant kernel: the longer of the scatter (all of the dispatch's row
    # bytes) and the combine; its mean duration from the events around it
    B = main_res["bytes"]
    x_elt = 1 if main_res["x_dtype"] == "fp8_e4m3" else 2
    from combine_ep_get_dispatch_amd import workloads as W
    wl_sb = W.config(args.config).scale_block
    rw = kernel_rw_bytes(B, main_res["T"], main_res["H"], main_res["k"], main_res["R"], x_elt, wl_sb)
    kern = {"scatter": (main_res["kernels"]["scatter"], cold["scatter_us"], sum(rw["scatter"])),
            "combine": ("moedisp_combine", cold["combine_us"], sum(rw["combine"]))}
    dom = max(kern, key=lambda n: kern[n][1]["mean"])
    dom_name, dom_us, dom_bytes = kern[dom]
    achieved = dom_bytes / (dom_us["mean"] * 1e-6) / 1e9
    from combine_ep_get_dispatch_amd.profiling import kernel_traffic, load_traffic
    measured = load_traffic(os.path.join(ROOT, "profiles", "hbm_traffic.json"))
    traffic = None
    kt = kernel_traffic(measured, dom_name) if measured and measured.get("workload") == main_res["workload"] else None
    if kt:
        traffic = kt["fetch_bytes"] + kt["write_bytes"]
    vs_ceiling = None
    if ceil:
        vs_ceiling = {}
        for n, (name, us, nbytes) in kern.items():
            rd, wr = rw[n]
            c_us = (rd / (ceil["read_gbps"] * 1e9) + wr / (ceil["write_seq_4k_gbps"] * 1e9)) * 1e6
            vs_ceiling[n] = {"kernel": name, "ceiling_us": c_us, "us": us["median"], "frac": c_us / us["median"],
                             "read_bytes": rd, "write_bytes": wr}

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle, per phase)")
        cpu = cpu_baseline()

    dc = dc_summary(main_res)
    line = {
        "metric": METRIC,
        "value": main_res["T"] / (step_us * 1e-6),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_us * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_res["x_dtype"],
        "data": "synthetic (seeded N(0,1) activations, uniform top-k routing, softmax weights)",
        "config": {"workload": main_res["workload"], "T": main_res["T"], "H": main_res["H"], "E": main_res["E"],
                   "G": main_res["G"], "k": main_res["k"], "x_dtype": main_res["x_dtype"],
                   "routing": main_res["routing"], "step": "layout_notify+dispatch_scatter+combine",
                   "parallelism": "none"},
        "timing": {"statistic": "median over the timed steps (min, mean beside)",
                   "cache": f"cold: {COLD_FLUSH_BYTES >> 20} MiB read before every step, outside its events",
                   "events": "timing-only HIP events on the launch stream at the step's call boundaries",
                   "timed_region_ms": main_res["timed_region_ms"], "box": box_info()},
        "hbm_gbps_step": B["step"] / (step_us * 1e-6) / 1e9,
        "hbm_frac_step": B["step"] / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        "dispatch_combine": {**dc, "target_frac": TARGET_FRAC, "meets_target": dc["frac"] >= TARGET_FRAC},
        "cold": {"step_us": step_us, "layout_notify_us": cold["layout_notify_us"]["median"],
                 "scatter_us": cold["scatter_us"]["median"], "combine_us": cold["combine_us"]["median"],
                 "dc_us": cold["dc_us"]["median"], "all": cold},
        "warm": None if main_res["warm"] is None else {
            "step_us": main_res["warm"]["step_us"]["median"],
            "tokens_per_s": main_res["T"] / (main_res["warm"]["step_us"]["median"] * 1e-6),
            "dispatch_combine": dc_summary(main_res, "warm"), "all": main_res["warm"]},
        "page_conventions": page_conventions(main_res),
        "calls_cold_us": main_res["calls_cold"],
        "kernels": main_res["kernels"],
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes": dom_bytes, "kernel_us": dom_us["mean"],
                     "kernel_us_median": dom_us["median"], "kernel_us_min": dom_us["min"],
                     "kernel_us_source": ("mean of the HIP-event intervals around the kernel's call on its "
                                          "launch stream over the timed cold steps"),
                     "profile": PROFILE},
        "ceilings_gbps": ceil,
        "vs_ceiling": vs_ceiling,
        "other_workloads": others,
        "quant_dispatch": quant,
        "group_path": groups,
        "decode": decode,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
