"""GPU parity of the small-batch path ep_layout_dispatch_small (layout and
dispatch in one launch) against the CPU oracle, and of the decode step
(small-batch dispatch + combine) captured in a HIP graph (needs an MI355X).

Bit-exact: every layout and dispatch output.  Combine: the usual bar.  The
graph test replays a captured decode step several times, with eager work and
new routing and activations copied into the captured inputs between
replays, and checks every replay against the oracle.
"""
import numpy as np
import pytest
import torch

import combine_ep_get_dispatch_amd as M
from combine_ep_get_dispatch_amd import workloads as W
import gpu_harness as GH

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.load()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def run_small(orc, wl, dev, bufs=None, inputs=None):
    o = GH.oracle_run(orc, wl)
    bufs = bufs or M.EpBuffers(GH.shape_of(wl), dev)
    inputs = inputs or GH.GpuInputs(wl, dev)
    bufs.layout_dispatch_small(inputs.x, inputs.x_scales, inputs.topk_idx, inputs.topk_weights)
    st = bufs.status()
    assert st == (o["status"] | o["layout_status"]), f"device status {st} != oracle {o['status']}"
    g, R = GH.fetch_dispatch(bufs, wl)
    GH.assert_dispatch_equal(g, o, wl)
    return o, bufs, inputs


CASES = {
    "decode_fp8": lambda: W.config(4),
    "tiny": lambda: W.config(1),
    "one_token": lambda: W.make_workload("t1", 1, 7168, 256, 8, 8, seed=80),
    "ragged_zipf": lambda: W.make_workload("zipf77", 77, 7168, 256, 8, 8, seed=81, routing="zipf", mask_frac=0.1),
    "k1": lambda: W.make_workload("k1", 200, 2048, 64, 8, 1, seed=82),
    "e1024": lambda: W.make_workload("e1024", 128, 1024, 1024, 32, 8, seed=83),
    "mixtral": lambda: W.make_workload("mixtral", 512, 4096, 8, 8, 2, seed=84),
    "max_slots": lambda: W.make_workload("max_slots", 1024, 512, 256, 8, 8, seed=85),
    "all_masked": lambda: W.make_workload("all_masked", 33, 256, 16, 4, 4, seed=86, mask_frac=1.0),
    "empty": lambda: W.make_workload("empty", 0, 256, 16, 4, 4, seed=87),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layout_dispatch_small_parity(orc, dev, name):
    wl = CASES[name]()
    _say(f"[small] {name} T={wl.T} H={wl.H} E={wl.E} G={wl.G} k={wl.k} {wl.x_dtype}")
    o, bufs, _ = run_small(orc, wl, dev)
    if wl.T:
        eo_bits = GH.oracle_expert_out(wl, o)
        eo = GH.upload_expert_out(eo_bits, wl.T * wl.k, wl.H, dev)
        g32, g16, st = GH.gpu_combine(bufs, eo, wl, dev)
        assert st == 0
        o32, o16 = orc.combine(eo_bits, o["recv_weights"][:int(o["expert_offsets"][-1])], o["slot_to_row"])
        GH.assert_combine_close(g32, g16, o32, o16)
    _say(f"[small] {name} ok")


def test_layout_dispatch_small_bad_and_repeated_ids(orc, dev):
    wl = W.make_workload("bad_ids", 64, 256, 32, 4, 4, seed=88)
    wl.topk_idx[3, 1] = 40          # out of range
    wl.topk_idx[5, 2] = -3          # negative, not -1
    wl.topk_idx[7, 3] = wl.topk_idx[7, 0]   # repeated expert
    o, bufs, _ = run_small(orc, wl, dev)
    assert o["status"] & 1 and o["layout_status"] & 2


def test_small_matches_two_call_path(orc, dev):
    """Same outputs as ep_get_dispatch_layout + ep_dispatch on the same buffers."""
    wl = W.config(4)
    inp = GH.GpuInputs(wl, dev)
    a = M.EpBuffers(GH.shape_of(wl), dev)
    b = M.EpBuffers(GH.shape_of(wl), dev)
    a.layout(inp.topk_idx)
    a.dispatch(inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights)
    b.layout_dispatch_small(inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights)
    assert a.status() == 0 and b.status() == 0
    R = int(a.expert_offsets[-1].item())
    for name in ("tokens_per_expert", "tokens_per_group", "is_token_in_group", "expert_offsets", "slot_to_row"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    for name in ("recv_x", "recv_scales", "recv_src_idx", "recv_weights"):
        assert torch.equal(getattr(a, name)[:R], getattr(b, name)[:R]), name


def test_decode_step_in_hip_graph(orc, dev):
    """Capture small-batch dispatch + combine; replay with new inputs."""
    base = W.config(4)
    bufs = M.EpBuffers(GH.shape_of(base), dev)
    inp = GH.GpuInputs(base, dev)
    eo = torch.zeros((base.T * base.k, base.H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((base.T, base.H), dtype=torch.bfloat16, device=dev)
    # warm up on a side stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        bufs.layout_dispatch_small(inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights)
        bufs.combine(eo, out, M.BF16, True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bufs.layout_dispatch_small(inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights)
        bufs.combine(eo, out, M.BF16, True)
    for rep, seed in enumerate((90, 91, 92)):
        wl = W.make_workload(f"graph{rep}", base.T, base.H, base.E, base.G, base.k, seed=seed, x_dtype=W.X_FP8,
                             scale_block=128, routing="zipf" if rep == 1 else "uniform",
                             mask_frac=0.05 if rep == 2 else 0.0, expert_kind="dequant_identity")
        o = GH.oracle_run(orc, wl)
        eo_bits = GH.oracle_expert_out(wl, o)
        # new inputs into the captured tensors; eager work between replays
        new = GH.GpuInputs(wl, dev)
        inp.x.copy_(new.x)
        inp.x_scales.copy_(new.x_scales)
        inp.topk_idx.copy_(new.topk_idx)
        inp.topk_weights.copy_(new.topk_weights)
        eo.zero_()
        R = eo_bits.shape[0]
        # expert outputs are placed at the oracle's rows, which the graph's
        # dispatch must reproduce for the combine to match
        eo[:R] = GH.bits16_to_bf16_tensor(eo_bits).to(dev)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert bufs.status() == 0
        g, _ = GH.fetch_dispatch(bufs, wl)
        GH.assert_dispatch_equal(g, o, wl)
        o32, o16 = orc.combine(eo_bits, o["recv_weights"][:R], o["slot_to_row"])
        g16 = out.view(torch.int16).cpu().numpy().view(np.uint16)
        d = GH.bf16_ulp_distance(g16, o16)
        assert d.size == 0 or d.max() <= GH.COMBINE_ULP_TOL, f"replay {rep}: combine off by {int(d.max())} ulp"
        _say(f"[graph] replay {rep} ok R={R}")


def test_prefill_step_in_hip_graph(orc, dev):
    """Capture layout + dispatch (two phases) + combine at a ragged mid size;
    replay with new routing and activations, every replay against the oracle."""
    base = W.make_workload("graph_prefill", 601, 2048, 64, 8, 8, seed=95)
    bufs = M.EpBuffers(GH.shape_of(base), dev)
    inp = GH.GpuInputs(base, dev)
    eo = torch.zeros((base.T * base.k, base.H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((base.T, base.H), dtype=torch.float32, device=dev)

    def step():
        bufs.layout(inp.topk_idx)
        bufs.dispatch_notify(inp.topk_idx)
        bufs.dispatch_scatter(inp.x, None, inp.topk_idx, inp.topk_weights)
        bufs.combine(eo, out, M.FP32, True)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep, seed in enumerate((96, 97)):
        wl = W.make_workload(f"graph_prefill{rep}", base.T, base.H, base.E, base.G, base.k, seed=seed,
                             routing="zipf" if rep else "uniform", mask_frac=0.05 * rep, expert_kind="scale_by_id")
        o = GH.oracle_run(orc, wl)
        eo_bits = GH.oracle_expert_out(wl, o)
        new = GH.GpuInputs(wl, dev)
        inp.x.copy_(new.x)
        inp.topk_idx.copy_(new.topk_idx)
        inp.topk_weights.copy_(new.topk_weights)
        eo.zero_()
        R = eo_bits.shape[0]
        eo[:R] = GH.bits16_to_bf16_tensor(eo_bits).to(dev)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert bufs.status() == 0
        g, _ = GH.fetch_dispatch(bufs, wl)
        GH.assert_dispatch_equal(g, o, wl)
        o32, _ = orc.combine(eo_bits, o["recv_weights"][:R], o["slot_to_row"], want_bf16=False)
        g32 = out.cpu().numpy()
        nz = o32 != 0
        rel = np.abs(g32[nz].astype(np.float64) - o32[nz]) / np.abs(o32[nz])
        assert rel.size == 0 or rel.max() <= GH.COMBINE_REL_TOL
        assert np.all(g32[~nz] == 0.0)
        _say(f"[graph-prefill] replay {rep} ok R={R}")


# --- padded (low-latency) layout ---------------------------------------------

def run_padded(orc, wl, dev, C, S, B):
    """ep_layout_dispatch_small_padded against the oracle: layout outputs,
    handle, every taken row (bytes, scales, source, weight bits) exact, and
    every row no slot takes still holding its sentinel."""
    o = orc.dispatch_padded(wl.x, wl.x_scales, wl.topk_idx, wl.topk_weights, wl.E, C, S, B)
    tpe, tpg, bm, st_l = orc.layout(wl.topk_idx, wl.E, wl.G)
    bufs = M.EpBuffers(GH.shape_of(wl), dev)
    pb = M.EpPaddedBuffers(bufs, C, S, B)
    pb.recv_x.fill_(0xA5)
    pb.recv_src_idx.fill_(-9)
    pb.recv_weights.fill_(-1.0)
    if pb.recv_scales is not None:
        pb.recv_scales.fill_(-2.0)
    inp = GH.GpuInputs(wl, dev)
    pb.dispatch(inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights)
    st = bufs.status()
    assert st == (o["status"] | st_l), f"device status {st} != oracle {o['status'] | st_l}"
    assert np.array_equal(bufs.tokens_per_expert.cpu().numpy(), tpe)
    assert np.array_equal(bufs.tokens_per_group.cpu().numpy(), tpg)
    assert np.array_equal(bufs.is_token_in_group.cpu().numpy().view(np.uint32), bm)
    s2r = pb.slot_to_row[:wl.T].cpu().numpy()
    assert np.array_equal(s2r, o["slot_to_row"])
    rows = wl.E * S
    taken = np.zeros(rows, bool)
    taken[o["slot_to_row"][o["slot_to_row"] >= 0]] = True
    gx = pb.recv_x.cpu().numpy()
    ox = np.ascontiguousarray(o["recv_x"]).view(np.uint8).reshape(rows, -1)
    assert np.array_equal(gx[taken], ox[taken]), "taken rows"
    assert np.all(gx[~taken] == 0xA5), "a row no slot takes was written"
    assert np.array_equal(pb.recv_src_idx.cpu().numpy()[taken], o["recv_src_idx"][taken])
    assert np.all(pb.recv_src_idx.cpu().numpy()[~taken] == -9)
    assert np.array_equal(pb.recv_weights.cpu().numpy()[taken].view(np.uint32),
                          o["recv_weights"][taken].view(np.uint32))
    if pb.recv_scales is not None:
        gs = pb.recv_scales.cpu().numpy()
        assert np.array_equal(gs[taken].view(np.uint32), o["recv_scales"][taken].view(np.uint32))
        assert np.all(gs[~taken] == -2.0)
    return o, bufs, pb, inp


def padded_expert_out(orc, wl, o_pad, S):
    """Stand-in expert outputs at the padded rows: the flat path's output of
    the same slot, moved to the slot's padded row."""
    of = GH.oracle_run(orc, wl)
    eo_flat = GH.oracle_expert_out(wl, of)
    eo = np.zeros((wl.E * S, wl.H), np.uint16)
    fr = of["slot_to_row"]
    pr = o_pad["slot_to_row"]
    m = pr >= 0
    eo[pr[m]] = eo_flat[fr[m]]
    return eo


PADDED = {
    # (workload, C, S, B): C = T is the low-latency buffer's usual size
    "decode_fp8": (lambda: W.config(4), 128, 128, 0),
    "decode_fp8_overflow": (lambda: W.config(4), 3, 3, 0),
    "ragged_base_stride": (lambda: W.make_workload("pad_ragged", 77, 7168, 256, 8, 8, seed=101, routing="zipf",
                                                   mask_frac=0.1), 20, 27, 5),
    "k16": (lambda: W.make_workload("pad_k16", 96, 512, 64, 8, 16, seed=102), 96, 100, 4),
    "e1024": (lambda: W.make_workload("pad_e1024", 128, 1024, 1024, 32, 8, seed=103), 8, 8, 0),
    "mixtral_overflow": (lambda: W.make_workload("pad_mixtral", 512, 4096, 8, 8, 2, seed=104), 120, 130, 10),
    "empty": (lambda: W.make_workload("pad_empty", 0, 256, 16, 4, 4, seed=105), 4, 4, 0),
}


@pytest.mark.parametrize("name", list(PADDED))
def test_layout_dispatch_small_padded_parity(orc, dev, name):
    mk, C, S, B = PADDED[name]
    wl = mk()
    _say(f"[padded] {name} T={wl.T} H={wl.H} E={wl.E} k={wl.k} C={C} S={S} B={B}")
    o, bufs, pb, _ = run_padded(orc, wl, dev, C, S, B)
    if "overflow" in name:
        assert o["status"] & M.binding.DEV_EXPERT_OVERFLOW
    if wl.T:
        eo_bits = padded_expert_out(orc, wl, o, S)
        eo = GH.upload_expert_out(eo_bits, wl.E * S, wl.H, dev)
        of = torch.empty((wl.T, wl.H), dtype=torch.float32, device=dev)
        ob = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
        pb.combine(eo, of, M.FP32)
        pb.combine(eo, ob, M.BF16)
        assert bufs.status() == 0
        o32, o16 = orc.combine(eo_bits, o["recv_weights"], o["slot_to_row"])
        GH.assert_combine_close(of.cpu().numpy(), ob.view(torch.int16).cpu().numpy().view(np.uint16), o32, o16)
    _say(f"[padded] {name} ok")


def test_padded_decode_step_in_hip_graph(orc, dev):
    """Capture padded dispatch + combine; replay with new routing and
    activations, every replay against the oracle."""
    base = W.config(4)
    C = S = base.T
    bufs = M.EpBuffers(GH.shape_of(base), dev)
    pb = M.EpPaddedBuffers(bufs, C, S, 0)
    inp = GH.GpuInputs(base, dev)
    eo = torch.zeros((base.E * S, base.H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((base.T, base.H), dtype=torch.bfloat16, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pb.dispatch(inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights)
        pb.combine(eo, out, M.BF16, True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pb.dispatch(inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights)
        pb.combine(eo, out, M.BF16, True)
    for rep, seed in enumerate((106, 107, 108)):
        wl = W.make_workload(f"pgraph{rep}", base.T, base.H, base.E, base.G, base.k, seed=seed, x_dtype=W.X_FP8,
                             scale_block=128, routing="zipf" if rep == 1 else "uniform",
                             mask_frac=0.05 if rep == 2 else 0.0, expert_kind="dequant_identity")
        o = orc.dispatch_padded(wl.x, wl.x_scales, wl.topk_idx, wl.topk_weights, wl.E, C, S, 0)
        eo_bits = padded_expert_out(orc, wl, o, S)
        new = GH.GpuInputs(wl, dev)
        inp.x.copy_(new.x)
        inp.x_scales.copy_(new.x_scales)
        inp.topk_idx.copy_(new.topk_idx)
        inp.topk_weights.copy_(new.topk_weights)
        eo.copy_(GH.bits16_to_bf16_tensor(eo_bits).to(dev))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert bufs.status() == 0
        assert np.array_equal(pb.slot_to_row[:wl.T].cpu().numpy(), o["slot_to_row"])
        o32, o16 = orc.combine(eo_bits, o["recv_weights"], o["slot_to_row"])
        g16 = out.view(torch.int16).cpu().numpy().view(np.uint16)
        d = GH.bf16_ulp_distance(g16, o16)
        assert d.size == 0 or d.max() <= GH.COMBINE_ULP_TOL, f"replay {rep}: combine off by {int(d.max())} ulp"
        _say(f"[pgraph] replay {rep} ok")
