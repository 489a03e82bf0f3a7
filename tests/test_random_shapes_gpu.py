"""Seeded random shapes through every dispatch path of libmoedisp against the
CPU oracle (needs an MI355X).

The shapes are drawn once from a fixed seed (T up to 3000 tokens, E up to
512 experts in 1 to 32 groups, k up to 16, bf16 rows of 16 B to 16 KB, fp8
rows with 32- or 128-channel scales, uniform or Zipf routing, some slots
masked), so that the planners' branches (push or block-pull scatter, folded
or separate notify tiles, column splits, compact lists, small path) meet
shapes no hand-picked case names.  Per shape, bit-exact unless said:
  - layout + notify (the benchmark's calls) + scatter: every output;
  - the group dispatch and its local permutation: every output;
  - the small path (where its size limit allows), flat and padded;
  - combine after the dispatch: the combine bar on every token.
"""
import numpy as np
import pytest
import torch

import combine_ep_get_dispatch_amd as M
from combine_ep_get_dispatch_amd import workloads as W
import gpu_harness as GH
import oracle_checks as K

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.load()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def draw_shapes(n=48, seed=0x5EED1234):
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        G = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
        per = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
        E = G * per
        if E > 512:
            continue
        k = int(rng.integers(1, min(16, E) + 1))
        T = int(rng.choice([0, 1, 7, 64, 129, 300, 511, 777, 1024, 1500, 2047, 3000]))
        fp8 = bool(rng.random() < 0.3)
        if fp8:
            sb = int(rng.choice([32, 128]))
            H = sb * int(rng.integers(1, 40))
        else:
            sb = 0
            H = 8 * int(rng.integers(1, 1024))   # 16-byte units of bf16
        if T * H * (1 if fp8 else 2) * k > (1 << 28):   # keep the oracle quick
            continue
        routing = "zipf" if rng.random() < 0.4 else "uniform"
        mask = float(rng.choice([0.0, 0.0, 0.05, 0.3]))
        shapes.append(dict(T=T, H=H, E=E, G=G, k=k, fp8=fp8, sb=sb, routing=routing, mask=mask,
                           seed=int(rng.integers(1, 1 << 30))))
    return shapes


SHAPES = draw_shapes()


def workload(s):
    return W.make_workload(f"rand_{s['seed']}", s["T"], s["H"], s["E"], s["G"], s["k"], seed=s["seed"],
                           x_dtype=W.X_FP8 if s["fp8"] else W.X_BF16, scale_block=s["sb"],
                           routing=s["routing"], mask_frac=s["mask"],
                           expert_kind="dequant_identity" if s["fp8"] else "scale_by_id")


def label(s):
    return (f"T{s['T']}_H{s['H']}_E{s['E']}_G{s['G']}_k{s['k']}_{'fp8b' + str(s['sb']) if s['fp8'] else 'bf16'}"
            f"_{s['routing']}_m{s['mask']}")


@pytest.mark.parametrize("s", SHAPES, ids=[label(s) for s in SHAPES])
def test_random_shape_every_path(orc, dev, s):
    wl = workload(s)
    shape = GH.shape_of(wl)
    q = M.ep_plan_query(shape)
    _say(f"[rand] {label(s)} pull={q['pull']} permute_pull={q['permute_pull']} small={q['small']}")
    o = GH.oracle_run(orc, wl)
    inputs = GH.GpuInputs(wl, dev)

    # the benchmark's calls
    b = M.EpBuffers(shape, dev)
    b.layout_notify(inputs.topk_idx)
    b.dispatch_scatter(inputs.x, inputs.x_scales, inputs.topk_idx, inputs.topk_weights)
    assert b.status() == (o["status"] | o["layout_status"])
    g, R = GH.fetch_dispatch(b, wl)
    GH.assert_dispatch_equal(g, o, wl)
    if wl.T and R:
        eo_bits = GH.oracle_expert_out(wl, o)
        eo = GH.upload_expert_out(eo_bits, wl.T * wl.k, wl.H, dev)
        g32, g16, st = GH.gpu_combine(b, eo, wl, dev)
        assert st == 0
        o32, o16 = orc.combine(eo_bits, o["recv_weights"][:R], o["slot_to_row"])
        GH.assert_combine_close(g32, g16, o32, o16)

    # the group dispatch and the local permutation
    h = K.ht_path(orc, wl)
    gd, pm, Rg, Rp = h["gd"], h["pm"], h["Rg"], h["R"]
    gb = M.EpGroupBuffers(b)
    gb.group_topk_idx.fill_(5)
    b.layout(inputs.topk_idx)
    gb.dispatch_groups(inputs.x, inputs.x_scales, inputs.topk_idx, inputs.topk_weights)
    assert b.status() == gd["status"]
    assert np.array_equal(gb.group_offsets.cpu().numpy(), gd["group_offsets"])
    assert np.array_equal(gb.token_group_row.cpu().numpy(), gd["token_group_row"])
    assert np.array_equal(gb.group_topk_idx[:Rg].cpu().numpy(), gd["recv_topk_idx"][:Rg])
    assert np.all(gb.group_topk_idx[Rg:].cpu().numpy() == -1)
    gx = np.ascontiguousarray(gd["recv_x"][:Rg]).view(np.uint8).reshape(Rg, wl.row_bytes)
    assert np.array_equal(gb.group_x[:Rg].cpu().numpy(), gx)
    gb.permute()
    assert b.status() == 0
    assert np.array_equal(b.expert_offsets.cpu().numpy(), pm["expert_offsets"])
    px = np.ascontiguousarray(pm["recv_x"][:Rp]).view(np.uint8).reshape(Rp, wl.row_bytes)
    assert np.array_equal(b.recv_x[:Rp].cpu().numpy(), px)
    assert np.array_equal(gb.perm_slot_to_row[:Rg].cpu().numpy(), pm["slot_to_row"])
    assert np.array_equal(b.recv_weights[:Rp].cpu().numpy().view(np.uint32),
                          pm["recv_weights"][:Rp].view(np.uint32))

    # the small path, flat and padded (capacity: half the fullest expert, so
    # that some shapes overflow)
    if q["small"]:
        bs = M.EpBuffers(shape, dev)
        bs.layout_dispatch_small(inputs.x, inputs.x_scales, inputs.topk_idx, inputs.topk_weights)
        assert bs.status() == (o["status"] | o["layout_status"])
        gs, _ = GH.fetch_dispatch(bs, wl)
        GH.assert_dispatch_equal(gs, o, wl)
        C = max(1, int(o["tokens_per_expert"].max(initial=0)) // 2)
        S, B = C + 3, 2
        op = orc.dispatch_padded(wl.x, wl.x_scales, wl.topk_idx, wl.topk_weights, wl.E, C, S, B)
        pb = M.EpPaddedBuffers(bs, C, S, B)
        pb.dispatch(inputs.x, inputs.x_scales, inputs.topk_idx, inputs.topk_weights)
        assert bs.status() == (op["status"] | o["layout_status"])
        assert np.array_equal(pb.slot_to_row[:wl.T].cpu().numpy(), op["slot_to_row"])
        taken = op["slot_to_row"][op["slot_to_row"] >= 0]
        ox = np.ascontiguousarray(op["recv_x"]).view(np.uint8).reshape(wl.E * S, -1)
        assert np.array_equal(pb.recv_x.cpu().numpy()[taken], ox[taken])
        assert np.array_equal(pb.recv_src_idx.cpu().numpy()[taken], op["recv_src_idx"][taken])
    _say(f"[rand] {label(s)} ok")
