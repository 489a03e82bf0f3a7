#!/usr/bin/env python3
"""Benchmark of one GPU's share of MoE EP layout -> dispatch -> combine.

One step = ep_get_dispatch_layout_notify (the layout and the dispatch's
notify phase of the same routing) + ep_dispatch_scatter + ep_combine (bf16
out) over one batch of the DeepSeek-V3-shaped prefill workload (T=4096
tokens, H=7168 bf16, E=256 experts in G=8 groups, top-8, uniform routing).
Inputs and the stand-in expert outputs are resident in HBM before the timed
region; the timed region is exactly K steps between two device
synchronisations.  HIP events on the launch stream bracket the scatter kernel
of every timed step (timing-only events without the system-scope cache fence,
which a default event adds between the kernels it separates); the dominant
kernel's algorithmic bytes over its mean duration give the roofline entry,
with the HBM bytes measured by rocprofv3 counters (profiles/hbm_traffic.json)
when they were taken on the current kernel sources.  Untimed passes of K
steps give the other phases: the separate calls (ep_get_dispatch_layout,
ep_dispatch_notify, ep_dispatch_scatter, ep_combine) with events between every
call, the same calls with events only around dispatch + combine (the
dispatch_combine figure: the events between the calls add their own time to
each phase), full steps timing the fused layout + notify call, and a cold
pass that reads
512 MiB before each step (back to back, the source rows stay in the 256 MB
MALL from one step to the next; the cold pass reports the step with nothing
of its inputs cached).  The CPU oracle, timed on a bounded sample of the same
workload on the host, is the reported baseline.

Further legs, reported beside the headline (each can be skipped): the other
workloads (skewed routing, fp8 decode, Mixtral shape), quantise-on-dispatch
(FP32 and UE8M0 block scales), the group-deduplicated path, decode-step
latency (four calls, the small-batch path, and that path from a HIP graph),
a plain-copy bandwidth probe, and a write probe (4 KiB chunks in address
order and permuted) that brackets the scatter's achievable write rate.

Prints one JSON line.  `--gpus` above 1 is refused: the library runs one
GPU's share of the path on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine tokens/s and HBM GB/s (% of peak) at T=4096 H=7168 E=256 k=8"
COLD_FLUSH_BYTES = 512 << 20  # read before each step of the cold pass: twice the MALL


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

    def __del__(self):
        if TimingEvent._hip is not None and self.e:
            TimingEvent._hip.hipEventDestroy(self.e)


def shape_of(M, W, wl):
    dt = M.FP8_E4M3 if wl.x_dtype == W.X_FP8 else M.BF16
    return M.moedisp_shape.make(wl.T, wl.H, wl.E, wl.G, wl.k, dt, wl.scale_block)


def run_gpu(cid, steps, warmup, dev, cold=True):
    """Time `steps` layout+dispatch+combine steps of config `cid` (and, with
    `cold`, the cold pass)."""
    import torch
    import combine_ep_get_dispatch_amd as M
    from combine_ep_get_dispatch_amd import workloads as W
    from combine_ep_get_dispatch_amd.traffic import HBM_PEAK_GBPS, algorithmic_bytes

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
    row_expert = W.row_experts(offs)
    eo = torch.zeros((wl.T * wl.k, wl.H), dtype=torch.bfloat16, device=dev)
    rs = bufs.recv_scales[:R] if bufs.recv_scales is not None else None
    eo[:R] = W.expert_outputs(wl, bufs.recv_x[:R], rs, row_expert, device=dev)
    del rs

    stream = torch.cuda.current_stream()

    # The timed step: ep_get_dispatch_layout_notify (the layout and the
    # dispatch's notify phase of the same routing, in two launches where the
    # shape allows), ep_dispatch_scatter, ep_combine.  `ev` (optional) gets
    # events before and after the scatter, the dominant kernel.
    def step_fused(ev=None):
        bufs.layout_notify(idx, stream)
        if ev is not None:
            ev[0].record(stream)
        bufs.dispatch_scatter(x, xs, idx, w, stream)
        if ev is not None:
            ev[1].record(stream)
        bufs.combine(eo, out, M.BF16, True, stream)

    # The same step with the layout and the notify phase as separate calls,
    # for the per-phase times (untimed passes).  `ev` holds events recorded at
    # the positions named in `at` (0 before the layout, 1 before notify, 2
    # before the scatter, 3 before the combine, 4 after it).
    def step(ev=None, at=()):
        if 0 in at:
            ev[0].record(stream)
        bufs.layout(idx, stream)
        if 1 in at:
            ev[1].record(stream)
        bufs.dispatch_notify(idx, stream)
        if 2 in at:
            ev[2].record(stream)
        bufs.dispatch_scatter(x, xs, idx, w, stream)
        if 3 in at:
            ev[3].record(stream)
        bufs.combine(eo, out, M.BF16, True, stream)
        if 4 in at:
            ev[4].record(stream)

    for _ in range(warmup):
        step_fused()
    torch.cuda.synchronize()
    # timed region: events bracket the scatter of every step
    evs = [[TimingEvent() for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step_fused(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    st = bufs.status()
    if st:
        raise RuntimeError(f"device status {st} after timed steps on config {cid}")
    elapsed = t1 - t0
    sct = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e3  # us
    # untimed pass: the separate calls with events between every call, for the
    # layout, notify and combine phases
    evs = [[TimingEvent() for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(evs[i], (0, 1, 2, 3, 4))
    torch.cuda.synchronize()
    st = bufs.status()
    if st:
        raise RuntimeError(f"device status {st} after the phase pass on config {cid}")
    lay = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e3
    ntf = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e3
    com = np.array([e[3].elapsed_time(e[4]) for e in evs]) * 1e3
    # untimed pass: dispatch + combine as one block, events only before the
    # notify phase and after the combine (events between the calls add their
    # own time to each phase)
    evs = [[TimingEvent() for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(evs[i], (1, 4))
    torch.cuda.synchronize()
    st = bufs.status()
    if st:
        raise RuntimeError(f"device status {st} after the dispatch + combine pass on config {cid}")
    dcb = np.array([e[1].elapsed_time(e[4]) for e in evs]) * 1e3
    # untimed pass: full steps, with events around the fused layout + notify
    # call only
    evs = [[TimingEvent() for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        evs[i][0].record(stream)
        bufs.layout_notify(idx, stream)
        evs[i][1].record(stream)
        bufs.dispatch_scatter(x, xs, idx, w, stream)
        bufs.combine(eo, out, M.BF16, True, stream)
    torch.cuda.synchronize()
    lnt = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e3
    # untimed pass, cold: 512 MiB read before each step, so nothing of the
    # step's inputs is left in the 256 MB MALL or the L2s (back to back, the
    # source rows x stay in the MALL from one step to the next).  A read, not
    # a write: written flush data would sit dirty in the MALL and be written
    # back during the step, which measured 12 us (config 2) to 20 us
    # (config 5) on the scatter that a clean cache does not cost.
    flush = torch.ones(COLD_FLUSH_BYTES if cold else 0, dtype=torch.uint8, device=dev).view(torch.int32)
    sink = torch.empty((), dtype=torch.int32, device=dev)
    n_cold = min(steps, 50) if cold else 0
    evs = [[TimingEvent() for _ in range(4)] for _ in range(n_cold)]
    torch.cuda.synchronize()
    for i in range(n_cold):
        torch.amax(flush, dim=0, out=sink)
        evs[i][0].record(stream)
        bufs.layout_notify(idx, stream)
        evs[i][1].record(stream)
        bufs.dispatch_scatter(x, xs, idx, w, stream)
        evs[i][2].record(stream)
        bufs.combine(eo, out, M.BF16, True, stream)
        evs[i][3].record(stream)
    torch.cuda.synchronize()
    st = bufs.status()
    if st:
        raise RuntimeError(f"device status {st} after the cold pass on config {cid}")
    cold_lnt = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e3
    cold_sct = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e3
    cold_com = np.array([e[2].elapsed_time(e[3]) for e in evs]) * 1e3
    del flush
    dis = ntf + sct
    x_elt = 1 if wl.x_dtype == W.X_FP8 else 2
    B = algorithmic_bytes(wl.T, wl.H, wl.E, wl.G, wl.k, R, x_elt, wl.scale_block)
    ms_step = elapsed / steps * 1e3
    res = dict(
        config=cid, workload=wl.name, T=wl.T, H=wl.H, E=wl.E, G=wl.G, k=wl.k, x_dtype=wl.x_dtype, R=R,
        routing=wl.meta["routing"], mask_frac=wl.meta["mask_frac"],
        ms_per_step=ms_step, tokens_per_s=wl.T / (ms_step * 1e-3),
        step_gbps=B["step"] / (ms_step * 1e-3) / 1e9,
        layout_us=float(lay.mean()), dispatch_us=float(dis.mean()), combine_us=float(com.mean()),
        notify_us=float(ntf.mean()), scatter_us=float(sct.mean()), layout_notify_us=float(lnt.mean()),
        dispatch_us_min=float(dis.min()), combine_us_min=float(com.min()),
        dispatch_gbps=B["dispatch"] / (dis.mean() * 1e-6) / 1e9,
        combine_gbps=B["combine"] / (com.mean() * 1e-6) / 1e9,
        dc_us=float(dcb.mean()), dc_us_min=float(dcb.min()),
        dc_phase_sum_us=float(dis.mean() + com.mean()),
        dc_tokens_per_s=wl.T / (dcb.mean() * 1e-6),
        bytes=B,
    )
    # the pages' own byte conventions, for context: tokens x hidden per phase
    # (their bench's per-rank count) and one row per routed copy
    tok_row = wl.T * wl.H * x_elt
    res["pages_convention_gbps"] = dict(
        tokens_x_hidden=dict(dispatch=tok_row / (dis.mean() * 1e-6) / 1e9,
                             combine=wl.T * wl.H * 2 / (com.mean() * 1e-6) / 1e9),
        routed_rows_x_hidden=dict(dispatch=R * wl.H * x_elt / (dis.mean() * 1e-6) / 1e9,
                                  combine=R * wl.H * 2 / (com.mean() * 1e-6) / 1e9))
    res["dc_gbps"] = B["dispatch_combine"] / (dcb.mean() * 1e-6) / 1e9
    res["dc_frac"] = res["dc_gbps"] / HBM_PEAK_GBPS
    sc_bytes = B["dispatch"] - B["notify"] + B["combine"]
    res["cold"] = None if not n_cold else dict(
        flush_bytes=COLD_FLUSH_BYTES, steps=n_cold,
        layout_notify_us=float(cold_lnt.mean()), scatter_us=float(cold_sct.mean()),
        combine_us=float(cold_com.mean()),
        step_us=float((cold_lnt + cold_sct + cold_com).mean()),
        tokens_per_s=wl.T / ((cold_lnt + cold_sct + cold_com).mean() * 1e-6),
        scatter_combine_frac=sc_bytes / ((cold_sct.mean() + cold_com.mean()) * 1e-6) / 1e9 / HBM_PEAK_GBPS,
    )
    del bufs, eo, out, x, xs, idx, w
    torch.cuda.empty_cache()
    return res


def run_gpu_quant(cid, block, fmt, steps, warmup, dev):
    """Time quantise-on-dispatch (notify + quantising scatter) on config `cid`."""
    import torch
    import combine_ep_get_dispatch_amd as M
    from combine_ep_get_dispatch_amd import workloads as W
    from combine_ep_get_dispatch_amd.traffic import HBM_PEAK_GBPS, algorithmic_bytes_quant

    wl = W.config(cid)
    bufs = M.EpBuffers(shape_of(M, W, wl), dev).enable_quant(block, fmt)
    x, _, idx, w = make_inputs(wl, dev)
    bufs.layout(idx)
    bufs.dispatch_quant(x, idx, w)
    st = bufs.status()
    if st:
        raise RuntimeError(f"device status {st} on quantised config {cid}")
    R = int(bufs.expert_offsets[-1].item())
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        bufs.dispatch_notify(idx, stream)
        bufs.dispatch_scatter_quant(x, idx, w, stream)
    evs = [[TimingEvent() for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        evs[i][0].record(stream)
        bufs.dispatch_notify(idx, stream)
        evs[i][1].record(stream)
        bufs.dispatch_scatter_quant(x, idx, w, stream)
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    if bufs.status():
        raise RuntimeError(f"device status after quantised steps on config {cid}")
    ntf = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e3
    sct = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e3
    B = algorithmic_bytes_quant(wl.T, wl.H, wl.E, wl.k, R, block, 4 if fmt == M.SCALE_FP32 else 1)
    dis = ntf + sct
    res = dict(workload=wl.name, block=block, scale_fmt="fp32" if fmt == M.SCALE_FP32 else "ue8m0", R=R,
               notify_us=float(ntf.mean()), scatter_us=float(sct.mean()), dispatch_us=float(dis.mean()),
               dispatch_tokens_per_s=wl.T / (dis.mean() * 1e-6),
               dispatch_gbps=B["dispatch"] / (dis.mean() * 1e-6) / 1e9,
               scatter_gbps=B["scatter"] / (sct.mean() * 1e-6) / 1e9, bytes=B)
    res["scatter_frac"] = res["scatter_gbps"] / HBM_PEAK_GBPS
    del bufs, x, idx, w
    torch.cuda.empty_cache()
    return res


def run_gpu_groups(cid, steps, warmup, dev):
    """Time the group-deduplicated path on config `cid`: layout, group
    dispatch, local expert permutation, local reduce, group combine."""
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
    evs = [[TimingEvent() for _ in range(len(calls) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        for j, c in enumerate(calls):
            evs[i][j].record(stream)
            c()
        evs[i][-1].record(stream)
    torch.cuda.synchronize()
    if bufs.status():
        raise RuntimeError(f"device status after the group path steps, config {cid}")
    us = np.array([[e[j].elapsed_time(e[j + 1]) * 1e3 for j in range(len(calls))] for e in evs]).mean(axis=0)
    x_elt = 1 if wl.x_dtype == W.X_FP8 else 2
    B = algorithmic_bytes_groups(wl.T, wl.H, wl.E, wl.G, wl.k, R, Rg, x_elt, wl.scale_block)
    names = ["layout", "dispatch_groups", "permute", "reduce", "combine_groups"]
    res = dict(workload=wl.name, R=R, R_g=Rg, us={n: float(u) for n, u in zip(names, us)})
    res["gbps"] = {n: B[n] / (res["us"][n] * 1e-6) / 1e9 for n in names[1:]}
    res["frac"] = {n: g / HBM_PEAK_GBPS for n, g in res["gbps"].items()}
    res["dispatch_combine_us"] = float(us[1:].sum())
    res["tokens_per_s"] = wl.T / (us[1:].sum() * 1e-6)
    del bufs, gb, x, xs, idx, w, eo, part, out
    torch.cuda.empty_cache()
    return res


def run_gpu_decode(cid, steps, warmup, dev):
    """Decode-step latency on config `cid` (T=128): the four calls (layout,
    notify, scatter, combine), the small-batch path (layout + dispatch in one
    launch, then combine), and that path replayed from a captured HIP graph
    of 10 steps.  Each figure is the mean GPU time per step over back-to-back
    steps between two events."""
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
        return e0.elapsed_time(e1) * 1e3 / steps

    res = dict(workload=wl.name, T=wl.T, R=R)
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
    # the small-batch dispatch alone, events around each call
    stream = torch.cuda.current_stream()
    ev = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        bufs.layout_dispatch_small(x, xs, idx, w, stream)
        b.record(stream)
    torch.cuda.synchronize()
    res["small_dispatch_us"] = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))
    if bufs.status():
        raise RuntimeError(f"device status after the decode steps, config {cid}")
    x_elt = 1 if wl.x_dtype == W.X_FP8 else 2
    B = algorithmic_bytes(wl.T, wl.H, wl.E, wl.G, wl.k, R, x_elt, wl.scale_block)
    res["step_bytes"] = B["step"]
    res["tokens_per_s_graph"] = wl.T / (res["small_graph_us"] * 1e-6)
    del graph, bufs, x, xs, idx, w, eo, out
    torch.cuda.empty_cache()
    return res


def probe_fill_gbps(dev, nbytes=32768 * 14336, reps=20):
    """HBM write bandwidth of 4 KiB chunks written in address order and in a
    permuted order (ep_probe_fill), over a buffer the size of the
    T=4096 H=7168 k=8 receive rows: the two ends between which the scatter's
    row writes (one moving write front per expert segment) fall."""
    import torch
    import combine_ep_get_dispatch_amd as M
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    res = {"bytes": nbytes}
    for shuffled, tag in ((False, "sequential_4k"), (True, "shuffled_4k")):
        for _ in range(3):
            M.ep_probe_fill(dst, nbytes, shuffled)
        s, e = TimingEvent(), TimingEvent()
        torch.cuda.synchronize()
        s.record(stream)
        for _ in range(reps):
            M.ep_probe_fill(dst, nbytes, shuffled)
        e.record(stream)
        torch.cuda.synchronize()
        us = s.elapsed_time(e) * 1e3 / reps
        res[tag] = nbytes / (us * 1e-6) / 1e9
    del dst
    torch.cuda.empty_cache()
    return res


def probe_copy_gbps(dev, nbytes=1 << 30, reps=20):
    """Achievable HBM copy bandwidth (read + write bytes) with the library's
    plain 16-byte copy kernel."""
    import torch
    import combine_ep_get_dispatch_amd as M
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        M.ep_probe_copy(dst, src, nbytes)
    s, e = TimingEvent(), TimingEvent()
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    s.record(stream)
    for _ in range(reps):
        M.ep_probe_copy(dst, src, nbytes)
    e.record(stream)
    torch.cuda.synchronize()
    us = s.elapsed_time(e) * 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (us * 1e-6) / 1e9


def cpu_baseline(budget_s: float = 12.0):
    """The CPU oracle (single-threaded C) on the same DeepSeek-V3-shaped
    workload, full steps of layout + dispatch + combine until about
    `budget_s` seconds of oracle time have run (at least one step)."""
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
    del d
    times = []
    t_start = time.perf_counter()
    while not times or (time.perf_counter() - t_start < budget_s and len(times) < 20):
        t0 = time.perf_counter()
        orc.layout(wl.topk_idx, wl.E, wl.G)
        dd = orc.dispatch(wl.x, wl.x_scales, wl.topk_idx, wl.topk_weights, wl.E)
        orc.combine(eo_bits, dd["recv_weights"][:R], dd["slot_to_row"], want_f32=False, want_bf16=True)
        times.append(time.perf_counter() - t0)
        del dd
    per_step = float(np.median(times))
    try:
        cpu = subprocess.run(["lscpu"], capture_output=True, text=True).stdout
        model = next((l.split(":", 1)[1].strip() for l in cpu.splitlines() if l.startswith("Model name")), "?")
    except Exception:
        model = "?"
    return dict(value=wl.T / per_step, unit="tokens/s", cores=1, kind="oracle",
                sample=(f"{len(times)} full steps (layout+dispatch+combine) of the T=4096 H=7168 E=256 k=8 "
                        f"workload, median {per_step:.2f} s/step; 1 thread of {os.cpu_count()} host cores ({model})"))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload for the headline line (default 2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-quant", action="store_true", help="skip the quantise-on-dispatch timings")
    ap.add_argument("--no-groups", action="store_true", help="skip the group-deduplicated path timings")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-latency timings")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold passes (512 MiB read before each step)")
    args = ap.parse_args()

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
    log(f"[bench] config {args.config}: {args.warmup} warmup + {args.steps} timed steps")
    main_res = run_gpu(args.config, args.steps, args.warmup, dev, cold=not args.no_cold)
    log(f"[bench] config {args.config}: {main_res['ms_per_step']*1e3:.1f} us/step, "
        f"dispatch {main_res['dispatch_us']:.1f} us, combine {main_res['combine_us']:.1f} us")

    others = {}
    if not args.no_other_workloads:
        for cid in (3, 4, 5):
            if cid == args.config:
                continue
            log(f"[bench] config {cid}")
            r = run_gpu(cid, max(20, args.steps // 4), max(5, args.warmup // 4), dev, cold=not args.no_cold)
            others[r["workload"]] = {k: r[k] for k in ("T", "H", "E", "G", "k", "x_dtype", "routing", "R",
                                                       "tokens_per_s", "dc_us", "dc_tokens_per_s", "dc_gbps", "dc_frac",
                                                       "layout_us", "dispatch_us", "combine_us",
                                                       "dispatch_gbps", "combine_gbps", "cold")}
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
    probe = None if args.no_probe else probe_copy_gbps(dev)
    if probe:
        log(f"[bench] probe copy {probe:.0f} GB/s")
    probe_w = None if args.no_probe else probe_fill_gbps(dev)
    if probe_w:
        log(f"[bench] probe write {probe_w['sequential_4k']:.0f} GB/s in address order, "
            f"{probe_w['shuffled_4k']:.0f} GB/s permuted")

    # dominant kernel: the longer of the scatter kernel (which moves all of the
    # dispatch's row bytes) and the combine kernel
    B = main_res["bytes"]
    if main_res["scatter_us"] >= main_res["combine_us"]:
        dom, dom_us = "moedisp_scatter", main_res["scatter_us"]
        dom_bytes = B["dispatch"] - B["notify"]
    else:
        dom, dom_us, dom_bytes = "moedisp_combine", main_res["combine_us"], B["combine"]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    from combine_ep_get_dispatch_amd.profiling import kernel_traffic, load_traffic
    measured = load_traffic(os.path.join(ROOT, "profiles", "hbm_traffic.json"))
    traffic = None
    kt = kernel_traffic(measured, dom) if measured and measured.get("workload") == main_res["workload"] else None
    if kt:
        traffic = kt["fetch_bytes"] + kt["write_bytes"]

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline()

    line = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_res["x_dtype"],
        "data": "synthetic (seeded N(0,1) activations, uniform top-k routing, softmax weights)",
        "config": {"workload": main_res["workload"], "T": main_res["T"], "H": main_res["H"], "E": main_res["E"],
                   "G": main_res["G"], "k": main_res["k"], "x_dtype": main_res["x_dtype"],
                   "routing": main_res["routing"], "step": "layout_notify+dispatch_scatter+combine",
                   "parallelism": "none"},
        "hbm_gbps_step": main_res["step_gbps"],
        "hbm_frac_step": main_res["step_gbps"] / HBM_PEAK_GBPS,
        "dispatch_combine": {"us": main_res["dc_us"], "us_min": main_res["dc_us_min"],
                             "tokens_per_s": main_res["dc_tokens_per_s"], "gbps": main_res["dc_gbps"],
                             "frac": main_res["dc_frac"], "phase_sum_us": main_res["dc_phase_sum_us"]},
        "phases_us": {"layout_notify": main_res["layout_notify_us"], "layout": main_res["layout_us"],
                      "dispatch": main_res["dispatch_us"],
                      "dispatch_notify": main_res["notify_us"], "dispatch_scatter": main_res["scatter_us"],
                      "combine": main_res["combine_us"], "dispatch_min": main_res["dispatch_us_min"],
                      "combine_min": main_res["combine_us_min"]},
        "phases_gbps": {"dispatch": main_res["dispatch_gbps"], "combine": main_res["combine_gbps"]},
        "cold": main_res["cold"],
        "pages_convention_gbps": main_res["pages_convention_gbps"],
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic, "algorithmic_bytes": dom_bytes,
                     "kernel_us": dom_us},
        "probe_copy_gbps": probe,
        "probe_write_gbps": probe_w,
        "other_workloads": others,
        "quant_dispatch": quant,
        "group_path": groups,
        "decode": decode,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
