"""GPU parity of ep_get_dispatch_layout_notify (the layout with the dispatch's
notify phase folded into its two launches) followed by ep_dispatch_scatter,
against the CPU oracle (needs an MI355X).

Bit-exact: every layout and dispatch output, and the device status.  The
shapes cover the folded path (the dispatch's tiles inside the layout's
workgroups: k = 1, 2, 8 and tiles of 16 to 128 tokens) and the shapes where
the call makes the two calls in order (k = 6, whose 170-token layout
workgroups hold no whole tile; E = 4096, whose tile counts exceed the LDS
budget; tiles of 256 tokens; T = 0).  The per-tile counts the scatter reads
are checked through the scatter's rows.
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


def run_layout_notify(orc, wl, dev):
    o = GH.oracle_run(orc, wl)
    bufs = M.EpBuffers(GH.shape_of(wl), dev)
    inp = GH.GpuInputs(wl, dev)
    # stale values in every output, so that a missed write shows
    for t in (bufs.tokens_per_expert, bufs.tokens_per_group, bufs.expert_offsets, bufs.slot_to_row):
        t.fill_(-7)
    bufs.layout_notify(inp.topk_idx)
    bufs.dispatch_scatter(inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights)
    st = bufs.status()
    assert st == (o["status"] | o["layout_status"]), f"device status {st} != oracle {o['status']}|{o['layout_status']}"
    g, _ = GH.fetch_dispatch(bufs, wl)
    GH.assert_dispatch_equal(g, o, wl)
    return bufs, inp, o


CASES = {
    # folded: k = 8 (128-token workgroups, tiles of 16), ragged T
    "dsv3_ragged": lambda: W.make_workload("dsv3_ragged", 601, 7168, 256, 8, 8, seed=91),
    "zipf_masked": lambda: W.make_workload("zipf_masked", 777, 1024, 256, 8, 8, seed=92, routing="zipf",
                                           mask_frac=0.1),
    # folded: k = 2 (512-token workgroups, 32 tiles each), k = 1 (1024 tokens)
    "k2": lambda: W.make_workload("k2", 3001, 512, 8, 8, 2, seed=93),
    "k1": lambda: W.make_workload("k1", 2500, 256, 64, 8, 1, seed=94),
    # folded: tiles of 128 tokens (one per k = 8 workgroup)
    "tiles128": lambda: W.make_workload("tiles128", 20000, 64, 64, 8, 8, seed=95),
    # two calls: tiles of 256 tokens, k = 6, E = 4096, T = 0
    "tiles256": lambda: W.make_workload("tiles256", 40000, 64, 32, 8, 8, seed=96),
    "k6": lambda: W.make_workload("k6", 500, 256, 48, 8, 6, seed=97),
    "e4096": lambda: W.make_workload("e4096", 300, 64, 4096, 32, 8, seed=98, routing="zipf"),
    "empty": lambda: W.make_workload("empty", 0, 256, 16, 4, 4, seed=99),
    "fp8": lambda: W.make_workload("fp8", 333, 2048, 64, 8, 4, seed=100, x_dtype=W.X_FP8, scale_block=128),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layout_notify_parity(orc, dev, name):
    wl = CASES[name]()
    _say(f"[layout_notify] {name} T={wl.T} H={wl.H} E={wl.E} G={wl.G} k={wl.k}")
    run_layout_notify(orc, wl, dev)
    _say(f"[layout_notify] {name} ok")


@pytest.mark.parametrize("cid", [2, 3, 5])
def test_layout_notify_full_size(orc, dev, cid):
    """The benchmark's call sequence at full size: layout_notify, scatter and
    combine; dispatch bit-exact, combine to the bar on every token."""
    wl = W.config(cid)
    _say(f"[layout_notify-full] config {cid} {wl.name} T={wl.T} H={wl.H} E={wl.E} k={wl.k}")
    bufs, _, o = run_layout_notify(orc, wl, dev)
    R = int(o["expert_offsets"][-1])
    eo_bits = GH.oracle_expert_out(wl, o)
    eo = GH.upload_expert_out(eo_bits, wl.T * wl.k, wl.H, dev)
    g32, g16, st = GH.gpu_combine(bufs, eo, wl, dev)
    assert st == 0
    o32, o16 = orc.combine(eo_bits, o["recv_weights"][:R], o["slot_to_row"])
    r = GH.assert_combine_close(g32, g16, o32, o16)
    _say(f"[layout_notify-full] config {cid} ok R={R} max_ulp={r['max_ulp']}")


def test_layout_notify_bad_and_repeated_ids(orc, dev):
    wl = W.make_workload("bad_ids", 300, 256, 32, 4, 4, seed=101)
    wl.topk_idx[3, 1] = 40                   # out of range
    wl.topk_idx[5, 2] = -3                   # negative, not -1
    wl.topk_idx[7, 3] = wl.topk_idx[7, 0]    # repeated expert
    _say("[layout_notify] bad ids")
    run_layout_notify(orc, wl, dev)


def test_layout_notify_then_combine_repeats(orc, dev):
    """Ten steps of layout_notify + scatter + combine on one workspace, new
    routing every other step: every step matches the oracle."""
    base = W.make_workload("rep", 1500, 512, 64, 8, 8, seed=102)
    bufs = M.EpBuffers(GH.shape_of(base), dev)
    for i in range(10):
        wl = base if i % 2 == 0 else W.make_workload("rep2", 1500, 512, 64, 8, 8, seed=103 + i, routing="zipf")
        o = GH.oracle_run(orc, wl)
        inp = GH.GpuInputs(wl, dev)
        bufs.layout_notify(inp.topk_idx)
        bufs.dispatch_scatter(inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights)
        assert bufs.status() == 0
        g, _ = GH.fetch_dispatch(bufs, wl)
        GH.assert_dispatch_equal(g, o, wl)
        eo_bits = GH.oracle_expert_out(wl, o)
        eo = GH.upload_expert_out(eo_bits, wl.T * wl.k, wl.H, dev)
        g32, g16, st = GH.gpu_combine(bufs, eo, wl, dev)
        assert st == 0
        o32, o16 = orc.combine(eo_bits, o["recv_weights"][:int(o["expert_offsets"][-1])], o["slot_to_row"])
        GH.assert_combine_close(g32, g16, o32, o16)
    _say("[layout_notify] 10 steps ok")
