"""GPU parity of the group-deduplicated (high-throughput) path against the
CPU oracle (needs an MI355X): ep_dispatch_groups, ep_group_permute,
ep_group_reduce and ep_combine_groups.

Bit-exact: group offsets, the token -> group-row handle, group rows and
scales, source tokens, restricted routing (ids and weight bits), the rows
past the last group row marked unrouted, and everything the local expert
permutation writes (its rows, offsets, weights and handle).  The local reduce
and the group combine are held to the combine bar (bit for bit in fp32 and
in the bf16 rounding); each runs on the oracle's own inputs.
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


def eq(g, o, what):
    g = np.ascontiguousarray(g)
    o = np.ascontiguousarray(o)
    if g.dtype == np.float32:
        g, o = g.view(np.uint32), o.view(np.uint32)
    if not np.array_equal(g, o):
        bad = np.argwhere(g != o) if g.shape == o.shape else None
        raise AssertionError(f"{what} differs (shape {g.shape} vs {o.shape}), first at {None if bad is None else bad[:4]}")


def run_groups(orc, wl, dev):
    _say(f"[groups] {wl.name} T={wl.T} H={wl.H} E={wl.E} G={wl.G} k={wl.k} {wl.x_dtype}")
    h = K.ht_path(orc, wl)
    gd, pm, Rg, R = h["gd"], h["pm"], h["Rg"], h["R"]
    bufs = M.EpBuffers(GH.shape_of(wl), dev)
    gb = M.EpGroupBuffers(bufs)
    inp = GH.GpuInputs(wl, dev)
    # stale values in the padding rows must not survive the call
    gb.group_topk_idx.fill_(3)
    bufs.layout(inp.topk_idx)
    gb.dispatch_groups(inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights)
    st = bufs.status()
    assert st == gd["status"], f"device status {st} != oracle {gd['status']}"
    eq(gb.group_offsets.cpu().numpy(), gd["group_offsets"], "group_offsets")
    eq(gb.token_group_row.cpu().numpy(), gd["token_group_row"], "token_group_row")
    eq(gb.group_src_idx[:Rg].cpu().numpy(), gd["recv_src_idx"][:Rg], "group recv_src_idx")
    eq(gb.group_topk_idx[:Rg].cpu().numpy(), gd["recv_topk_idx"][:Rg], "group recv_topk_idx")
    eq(gb.group_topk_weights[:Rg].cpu().numpy(), gd["recv_topk_weights"][:Rg], "group recv_topk_weights")
    assert np.all(gb.group_topk_idx[Rg:].cpu().numpy() == -1), "rows past R_g must be unrouted"
    orx = np.ascontiguousarray(gd["recv_x"][:Rg]).view(np.uint8).reshape(Rg, wl.row_bytes)
    eq(gb.group_x[:Rg].cpu().numpy(), orx, "group rows")
    if gb.group_scales is not None:
        eq(gb.group_scales[:Rg].cpu().numpy(), gd["recv_scales"][:Rg], "group scales")

    gb.permute()
    st = bufs.status()
    assert st == 0, f"permute status {st}"
    eq(bufs.expert_offsets.cpu().numpy(), pm["expert_offsets"], "permute expert_offsets")
    prx = np.ascontiguousarray(pm["recv_x"][:R]).view(np.uint8).reshape(R, wl.row_bytes)
    eq(bufs.recv_x[:R].cpu().numpy(), prx, "permuted rows")
    eq(gb.perm_src_idx[:R].cpu().numpy(), pm["recv_src_idx"][:R], "permute recv_src_idx (group rows)")
    eq(bufs.recv_weights[:R].cpu().numpy(), pm["recv_weights"][:R], "permute recv_weights")
    eq(gb.perm_slot_to_row[:Rg].cpu().numpy(), pm["slot_to_row"], "permute slot_to_row")
    assert np.all(gb.perm_slot_to_row[Rg:].cpu().numpy() == -1)
    if bufs.recv_scales is not None:
        eq(bufs.recv_scales[:R].cpu().numpy(), pm["recv_scales"][:R], "permuted scales")

    # local reduce on the oracle's expert outputs
    eo = GH.upload_expert_out(h["eo_bits"], wl.T * wl.k, wl.H, dev)
    cap = gb.capacity
    red32 = torch.empty((max(cap, 1), wl.H), dtype=torch.float32, device=dev)
    red16 = torch.empty((max(cap, 1), wl.H), dtype=torch.bfloat16, device=dev)
    gb.reduce(eo, red32, M.FP32)
    gb.reduce(eo, red16, M.BF16)
    assert bufs.status() == 0
    o32, o16 = orc.combine(h["eo_bits"], pm["recv_weights"][:R], pm["slot_to_row"])
    GH.assert_combine_close(red32[:Rg].cpu().numpy(), red16[:Rg].view(torch.int16).cpu().numpy().view(np.uint16),
                            o32, o16)
    # group combine on the oracle's group partials
    grows = GH.upload_expert_out(h["part"], max(cap, 1), wl.H, dev)
    of = torch.empty((max(wl.T, 1), wl.H), dtype=torch.float32, device=dev)
    ob = torch.empty((max(wl.T, 1), wl.H), dtype=torch.bfloat16, device=dev)
    gb.combine_groups(grows, of, M.FP32)
    gb.combine_groups(grows, ob, M.BF16)
    assert bufs.status() == 0
    g32 = of[:wl.T].cpu().numpy()
    g16 = ob[:wl.T].view(torch.int16).cpu().numpy().view(np.uint16)
    res = GH.assert_combine_close(g32, g16, h["out_f32"], h["out_bf16"])
    _say(f"[groups] {wl.name} ok R_g={Rg} R={R} max_ulp={res['max_ulp']} exact_f32={res['exact_f32']:.4f}")


CASES = {
    "tiny": lambda: W.config(1),
    "decode_fp8": lambda: W.config(4),
    "dsv3_ragged": lambda: W.make_workload("dsv3_ragged", 601, 7168, 256, 8, 8, seed=31, expert_kind="scale_by_id"),
    "zipf_ragged": lambda: W.make_workload("zipf_ragged", 777, 7168, 256, 8, 8, seed=32, routing="zipf",
                                           mask_frac=0.05, expert_kind="scale_by_id"),
    "mixtral_ragged": lambda: W.make_workload("mixtral_ragged", 3001, 4096, 8, 8, 2, seed=33,
                                              expert_kind="double_odd"),
    "groups_lt_k": lambda: W.make_workload("g_lt_k", 450, 512, 16, 2, 6, seed=70, mask_frac=0.2),
    "one_group": lambda: W.make_workload("g1", 333, 256, 16, 1, 4, seed=71),
    "groups_of_3": lambda: W.make_workload("g3", 300, 256, 24, 8, 4, seed=72, routing="zipf"),
    "g32_k8": lambda: W.make_workload("g32", 129, 256, 64, 32, 8, seed=73),
    "empty": lambda: W.make_workload("empty", 0, 256, 8, 2, 2, seed=74),
    "all_masked": lambda: W.make_workload("all_masked", 40, 256, 8, 2, 2, seed=75, mask_frac=1.0),
    # 875 units per row: the reduce's two column ranges are 438 and 437 units
    "ragged_columns": lambda: W.make_workload("ragged_cols", 300, 7000, 64, 8, 8, seed=76, mask_frac=0.1),
    # the push scatter permutes these: blocks of group rows would be under
    # 32 rows, or the experts too many for the block sort
    "push_permute_small": lambda: W.make_workload("push_small", 100, 256, 8, 2, 2, seed=79),
    "push_permute_e1024": lambda: W.make_workload("push_e1024", 300, 256, 1024, 8, 8, seed=80, mask_frac=0.05),
}


def test_permute_paths_covered():
    """The cases above reach both permutations: block-pull over compact
    lists, and the push scatter."""
    pull = {n: M.ep_plan_query(GH.shape_of(f()))["permute_pull"] for n, f in CASES.items()}
    assert pull["push_permute_small"] == 0 and pull["push_permute_e1024"] == 0
    assert pull["dsv3_ragged"] == 1 and pull["mixtral_ragged"] == 1


@pytest.mark.parametrize("name", list(CASES))
def test_group_path_parity(orc, dev, name):
    run_groups(orc, CASES[name](), dev)


def test_group_path_parity_full_size(orc, dev):
    """DeepSeek-V3 prefill shape: every group row, permuted row, partial and
    combined token."""
    run_groups(orc, W.config(2), dev)


def test_permute_entries_on_one_xcd(orc, dev):
    """Every routed slot of the group rows lies in the first block of group
    rows, which one XCD copies: that XCD's copy workgroups make several
    passes over its compact list while the other XCDs have none.  The
    permutation is ep_dispatch over the group rows, so the oracle's dispatch
    of the same rows is the expected result, bit for bit."""
    T, H, E, G, k = 512, 256, 64, 8, 8
    shape = M.moedisp_shape.make(T, H, E, G, k, M.BF16, 0)
    q = M.ep_plan_query(shape)
    assert q["permute_pull"] == 1
    cap = T * min(G, k)
    rows = min(q["permute_pull_tb"], T)  # rows of block 0, k slots each: at most T * k entries
    assert rows * k > 2 * q["permute_pull_wgs_per_xcd"]
    rng = np.random.default_rng(78)
    idx = np.full((cap, k), -1, np.int32)
    for r in range(rows):
        idx[r] = rng.choice(E, size=k, replace=False)
    w = rng.random((cap, k), dtype=np.float32)
    gx = rng.integers(0, 1 << 16, size=(cap, H), dtype=np.uint16)
    tpe, _, _, st = orc.layout(idx, E, G)
    assert st == 0
    o = orc.dispatch(gx, None, idx, w, E)
    R = int(o["expert_offsets"][-1])
    assert R == rows * k

    bufs = M.EpBuffers(shape, dev)
    gb = M.EpGroupBuffers(bufs)
    gb.group_x.copy_(torch.from_numpy(gx.view(np.uint8)))
    gb.group_topk_idx.copy_(torch.from_numpy(idx))
    gb.group_topk_weights.copy_(torch.from_numpy(w))
    bufs.tokens_per_expert.copy_(torch.from_numpy(tpe))
    gb.perm_slot_to_row.fill_(-7)
    gb.permute()
    assert bufs.status() == 0
    eq(bufs.expert_offsets.cpu().numpy(), o["expert_offsets"], "expert_offsets")
    eq(bufs.recv_x[:R].cpu().numpy(), o["recv_x"][:R].view(np.uint8), "rows")
    eq(gb.perm_src_idx[:R].cpu().numpy(), o["recv_src_idx"][:R], "recv_src_idx")
    eq(bufs.recv_weights[:R].cpu().numpy(), o["recv_weights"][:R], "recv_weights")
    eq(gb.perm_slot_to_row.cpu().numpy(), o["slot_to_row"], "slot_to_row")


ERROR_CASES = {
    # the local permutation on the block-pull copy, and on the push scatter
    "pull_permute": lambda: W.make_workload("err_pull", 600, 512, 64, 8, 8, seed=86),
    "push_permute": lambda: W.make_workload("err_push", 100, 256, 8, 2, 2, seed=87),
}


@pytest.mark.parametrize("name", list(ERROR_CASES))
def test_group_path_inconsistent_counts_are_reported(dev, name):
    """tokens_per_group, then tokens_per_expert, changed so that they disagree
    with the routing: ep_dispatch_groups and ep_group_permute report
    BAD_LAYOUT, write every handle entry (a row or -1), and no handle names a
    row outside its receive buffer."""
    wl = ERROR_CASES[name]()
    shape = GH.shape_of(wl)
    assert M.ep_plan_query(shape)["permute_pull"] == (name == "pull_permute")
    bufs = M.EpBuffers(shape, dev)
    gb = M.EpGroupBuffers(bufs)
    inp = GH.GpuInputs(wl, dev)
    bufs.layout(inp.topk_idx)
    assert bufs.status() == 0
    _say(f"[groups-err] {name}: group counts")
    good = bufs.tokens_per_group.clone()
    bufs.tokens_per_group[0] += 3
    bufs.tokens_per_group[1] -= 1
    gb.token_group_row.fill_(-7)
    gb.dispatch_groups(inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights)
    assert bufs.status() & M.binding.DEV_BAD_LAYOUT
    tgr = gb.token_group_row.cpu().numpy()
    assert tgr.min() >= -1 and tgr.max() < gb.capacity

    _say(f"[groups-err] {name}: expert counts")
    bufs.tokens_per_group.copy_(good)
    gb.dispatch_groups(inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights)
    assert bufs.status() == 0
    bufs.tokens_per_expert[0] += 2
    bufs.tokens_per_expert[wl.E - 1] -= 1
    gb.perm_slot_to_row.fill_(-7)
    gb.permute()
    assert bufs.status() & M.binding.DEV_BAD_LAYOUT
    p = gb.perm_slot_to_row.cpu().numpy()
    assert p.min() >= -1 and p.max() < wl.T * wl.k


def test_group_reduce_and_combine_report_bad_handles(dev):
    """A handle entry past the rows it indexes, and a row whose source no
    longer names its group row (reduce) or token (group combine): each call
    raises BAD_HANDLE and skips those slots (no load through them)."""
    wl = W.make_workload("grp_bad_handle", 64, 256, 16, 4, 4, seed=89)
    bufs = M.EpBuffers(GH.shape_of(wl), dev)
    gb = M.EpGroupBuffers(bufs)
    inp = GH.GpuInputs(wl, dev)
    bufs.layout(inp.topk_idx)
    gb.dispatch_groups(inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights)
    gb.permute()
    assert bufs.status() == 0
    cap = gb.capacity
    _say("[groups-err] reduce handle")
    p = gb.perm_slot_to_row
    p[0, 0] = wl.T * wl.k + 50                  # past the expert rows
    row1 = p[1].cpu().numpy()
    gb.perm_src_idx[int(row1[row1 >= 0][0])] = 0  # no longer names group row 1
    eo = bufs.recv_x.view(torch.bfloat16)
    red = torch.empty((cap, wl.H), dtype=torch.float32, device=dev)
    gb.reduce(eo, red, M.FP32)
    assert bufs.status() & M.binding.DEV_BAD_HANDLE
    _say("[groups-err] group combine handle")
    t = gb.token_group_row
    t[3, 0] = cap + 9                           # past the group rows
    row7 = t[7].cpu().numpy()
    gb.group_src_idx[int(row7[row7 >= 0][0])] = 0  # no longer names token 7
    grows = torch.zeros((cap, wl.H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.float32, device=dev)
    gb.combine_groups(grows, out, M.FP32)
    assert bufs.status() & M.binding.DEV_BAD_HANDLE
    assert torch.count_nonzero(out) == 0        # every other slot summed its zero rows
