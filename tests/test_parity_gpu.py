"""GPU parity of libmoedisp against the CPU oracle (needs an MI355X).

Bit-exact: layout counts, bitmap, offsets, slot_to_row, recv_src_idx,
recv_weights, received rows and scales.  Combine: bit for bit in fp32 and in
its bf16 rounding (the kernel sums in the oracle's order by fused
multiply-add), on every token of every case, the full sizes included (they run in the same launch configuration as the
benchmark).  Shapes with at least 256 tokens and at most 512 experts take the
block-pull dispatch (blocks of tokens per XCD, a sorted list per block);
smaller ones take the push scatter; both are covered here.
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


# --- small and mid-sized cases: every output compared ---------------------

MID = {
    "tiny": lambda: W.config(1),
    "decode_fp8": lambda: W.config(4),
    "dsv3_ragged": lambda: W.make_workload("dsv3_ragged", 601, 7168, 256, 8, 8, seed=31, expert_kind="scale_by_id"),
    "zipf_ragged": lambda: W.make_workload("zipf_ragged", 777, 7168, 256, 8, 8, seed=32, routing="zipf",
                                           mask_frac=0.05, expert_kind="scale_by_id"),
    "mixtral_ragged": lambda: W.make_workload("mixtral_ragged", 3001, 4096, 8, 8, 2, seed=33,
                                              expert_kind="double_odd"),
}


@pytest.mark.parametrize("name", list(MID))
def test_parity_every_output(orc, dev, name):
    wl = MID[name]()
    _say(f"[parity] {name} T={wl.T} H={wl.H} E={wl.E} G={wl.G} k={wl.k} {wl.x_dtype}")
    r = GH.full_parity(orc, wl, dev)
    _say(f"[parity] {name} ok R={r['R']} max_ulp={r['max_ulp']} exact_f32={r['exact_f32']:.4f}")


# --- full sizes, bench launch configuration --------------------------------

@pytest.mark.parametrize("cid", [2, 3, 5])
def test_parity_full_size(orc, dev, cid):
    wl = W.config(cid)
    _say(f"[parity-full] config {cid} {wl.name} T={wl.T} H={wl.H} E={wl.E} k={wl.k}")
    r = GH.full_parity(orc, wl, dev)
    _say(f"[parity-full] config {cid} ok R={r['R']} max_ulp={r['max_ulp']} exact_f32={r['exact_f32']:.4f}")


# --- edge cases ------------------------------------------------------------

EDGE = {
    "T0": lambda: W.make_workload("T0", 0, 64, 8, 2, 2, seed=41),
    "T1": lambda: W.make_workload("T1", 1, 64, 8, 2, 2, seed=42),
    "all_masked": lambda: W.make_workload("all_masked", 37, 64, 8, 2, 2, seed=43, mask_frac=1.0),
    "half_masked": lambda: W.make_workload("half_masked", 300, 64, 16, 4, 4, seed=44, mask_frac=0.5),
    "k1": lambda: W.make_workload("k1", 257, 64, 8, 2, 1, seed=45),
    "G1": lambda: W.make_workload("G1", 100, 64, 32, 1, 4, seed=46),
    "G_eq_E": lambda: W.make_workload("G_eq_E", 100, 64, 32, 32, 4, seed=47),
    "row16_bf16": lambda: W.make_workload("row16_bf16", 200, 8, 8, 2, 2, seed=48),
    "row16_fp8": lambda: W.make_workload("row16_fp8", 200, 16, 8, 2, 2, seed=49, x_dtype=W.X_FP8, scale_block=16),
    "k3_odd": lambda: W.make_workload("k3_odd", 123, 96, 12, 3, 3, seed=50),
    "k32": lambda: W.make_workload("k32", 50, 64, 64, 8, 32, seed=51),
    "E4096": lambda: W.make_workload("E4096", 300, 64, 4096, 32, 8, seed=52, routing="zipf", mask_frac=0.1),
    "E1": lambda: W.make_workload("E1", 70, 64, 1, 1, 1, seed=53),
    "tokens_per_tile_edges": lambda: W.make_workload("tile_edges", 1025, 256, 64, 8, 6, seed=54),
    "groups_of_3": lambda: W.make_workload("groups_of_3", 300, 64, 24, 8, 4, seed=55),
    "groups_of_6_zipf": lambda: W.make_workload("groups_of_6", 513, 64, 12, 2, 3, seed=56, routing="zipf",
                                                mask_frac=0.2),
    "groups_of_96": lambda: W.make_workload("groups_of_96", 200, 64, 3072, 32, 8, seed=57, routing="zipf"),
    # 875 units per row: column ranges of 63 (k = 8), 125 (k = 4) units, and
    # the generic-k gather (k = 5), each with a shorter last range
    "ragged_columns_k8": lambda: W.make_workload("ragged_cols_k8", 300, 7000, 64, 8, 8, seed=58),
    "ragged_columns_k4": lambda: W.make_workload("ragged_cols_k4", 200, 7000, 32, 4, 4, seed=59, mask_frac=0.2),
    "ragged_columns_k5": lambda: W.make_workload("ragged_cols_k5", 150, 7000, 40, 5, 5, seed=60, routing="zipf"),
    # 2500 units per row and enough tokens that rows are not split into
    # column ranges: more than one pass of the scatter's widest workgroup
    # (1024 lanes x 2 units), with a ragged last pass
    "wide_rows": lambda: W.make_workload("wide_rows", 1024, 20000, 16, 4, 4, seed=61),
    # block-pull boundaries: the smallest pulled T (8 blocks of 32 tokens,
    # the last one shorter), 512 experts with k = 32 (the largest expert
    # table and sorted list of the sort), fp8 rows with scales, masked
    # slots, rows wider than one pass of the copy workgroup, and 256 blocks
    # (a row's count prefix spans all 64 lanes of a wave)
    "pull_T255": lambda: W.make_workload("pull_T255", 255, 512, 64, 8, 8, seed=62),
    "pull_E512_k32": lambda: W.make_workload("pull_E512_k32", 2048, 256, 512, 32, 32, seed=63, routing="zipf",
                                             mask_frac=0.05),
    "pull_fp8": lambda: W.make_workload("pull_fp8", 1500, 7168, 256, 8, 8, seed=64, x_dtype=W.X_FP8,
                                        scale_block=128),
    "pull_masked": lambda: W.make_workload("pull_masked", 2000, 2048, 128, 8, 6, seed=65, mask_frac=0.3),
    "pull_wide_rows": lambda: W.make_workload("pull_wide_rows", 2000, 40000, 16, 4, 2, seed=66),
    "pull_256_blocks": lambda: W.make_workload("pull_256_blocks", 32768, 256, 64, 8, 32, seed=67),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_parity_edge_cases(orc, dev, name):
    wl = EDGE[name]()
    _say(f"[edge] {name} T={wl.T} H={wl.H} E={wl.E} G={wl.G} k={wl.k}")
    GH.full_parity(orc, wl, dev)


# --- properties -----------------------------------------------------------

def test_dispatch_deterministic_under_repeats(orc, dev):
    """Skewed routing, 20 dispatches on one workspace: every output identical
    (no scheduling order may leak into the result: the sorts rank slots by
    ballots and popcounts of token masks; their atomics only add and OR,
    which commute)."""
    wl = W.make_workload("det", 2048, 1024, 256, 8, 8, seed=61, routing="zipf", mask_frac=0.05)
    _say("[determinism] 20 repeats")
    bufs, inputs, st = GH.gpu_layout_dispatch(wl, dev)
    assert st == 0
    ref, R = GH.fetch_dispatch(bufs, wl)
    for i in range(20):
        bufs.recv_x.zero_()
        bufs.slot_to_row.fill_(-7)
        bufs.dispatch(inputs.x, inputs.x_scales, inputs.topk_idx, inputs.topk_weights)
        g, _ = GH.fetch_dispatch(bufs, wl)
        for key in ("expert_offsets", "slot_to_row", "recv_src_idx", "recv_weights", "recv_x"):
            assert np.array_equal(g[key], ref[key]), (i, key)
    assert bufs.status() == 0
    GH.assert_dispatch_equal(ref, GH.oracle_run(orc, wl), wl)


def test_notify_then_scatter_equals_dispatch(orc, dev):
    """The two phases called apart give exactly what ep_dispatch gives."""
    for wl in (W.make_workload("phases_bf16", 700, 512, 64, 8, 4, seed=91, routing="zipf", mask_frac=0.1),
               W.make_workload("phases_fp8", 90, 1024, 32, 8, 8, seed=92, x_dtype=W.X_FP8, scale_block=128)):
        shape = GH.shape_of(wl)
        inputs = GH.GpuInputs(wl, dev)
        b = M.EpBuffers(shape, dev)
        b.layout(inputs.topk_idx)
        b.dispatch_notify(inputs.topk_idx)
        b.dispatch_scatter(inputs.x, inputs.x_scales, inputs.topk_idx, inputs.topk_weights)
        assert b.status() == 0
        g, _ = GH.fetch_dispatch(b, wl)
        GH.assert_dispatch_equal(g, GH.oracle_run(orc, wl), wl)


def test_round_trip_identity_experts(dev):
    """dispatch -> identity experts (the received rows themselves) -> combine
    with weights summing to one returns x within one bf16 ulp."""
    wl = W.config(1)
    bufs, inputs, st = GH.gpu_layout_dispatch(wl, dev)
    assert st == 0
    eo = bufs.recv_x.view(torch.bfloat16)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
    bufs.combine(eo, out, M.BF16)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert GH.bf16_ulp_distance(got, wl.x).max() <= 1


def test_workspace_reuse_across_shapes(orc, dev):
    """One workspace serves a large call, then smaller and different ones;
    counts left by an earlier call must not leak into a later one."""
    big = W.make_workload("ws_big", 1500, 512, 64, 8, 4, seed=71)
    shape = GH.shape_of(big)
    bufs = M.EpBuffers(shape, dev)
    for wl in [big, W.make_workload("ws_small", 333, 512, 64, 8, 4, seed=72), big,
               W.make_workload("ws_fewer_experts", 700, 512, 16, 4, 4, seed=73)]:
        sub = GH.shape_of(wl)
        inputs = GH.GpuInputs(wl, dev)
        b = M.EpBuffers(sub, dev)
        b.ws = bufs.ws  # shared workspace, large enough for every shape here
        b.layout(inputs.topk_idx)
        b.dispatch(inputs.x, inputs.x_scales, inputs.topk_idx, inputs.topk_weights)
        assert b.status() == 0
        g, _ = GH.fetch_dispatch(b, wl)
        GH.assert_dispatch_equal(g, GH.oracle_run(orc, wl), wl)


# --- device-detected errors -------------------------------------------------

def test_bad_and_duplicate_expert_ids_match_oracle(orc, dev):
    wl = W.make_workload("bad_ids", 400, 64, 16, 4, 4, seed=81)
    idx = wl.topk_idx
    idx[3, 1] = 16      # out of range
    idx[10, 2] = -5     # negative, not -1
    idx[20, 3] = idx[20, 0]  # repeat within a token
    o = GH.oracle_run(orc, wl)
    assert o["status"] == (M.binding.DEV_BAD_EXPERT_ID | M.binding.DEV_DUPLICATE_EXPERT)
    bufs, inputs, st = GH.gpu_layout_dispatch(wl, dev)
    assert st == o["status"]
    g, _ = GH.fetch_dispatch(bufs, wl)
    GH.assert_dispatch_equal(g, o, wl)


def test_inconsistent_layout_is_reported(dev):
    wl = W.make_workload("bad_layout", 300, 64, 16, 4, 4, seed=82)
    bufs, inputs, st = GH.gpu_layout_dispatch(wl, dev)
    assert st == 0
    bufs.tokens_per_expert[0] += 5
    bufs.tokens_per_expert[3] -= 1
    bufs.dispatch(inputs.x, inputs.x_scales, inputs.topk_idx, inputs.topk_weights)
    assert bufs.status() & M.binding.DEV_BAD_LAYOUT
    s2r = bufs.slot_to_row.cpu().numpy()
    assert s2r.max() < wl.T * wl.k  # every written row stayed inside the buffer


def test_corrupt_pull_list_is_reported_and_skipped(orc, dev):
    """Block-pull scatter over a list that does not belong to this routing
    (entries naming slots of another block, or experts past E): reported as
    BAD_LAYOUT, the bad entries are neither followed nor written, and every
    entry of the untouched blocks is still copied exactly."""
    wl = W.make_workload("bad_list", 700, 512, 64, 8, 4, seed=84)
    shape = GH.shape_of(wl)
    q = M.ep_plan_query(shape)
    assert q["pull"] == 1 and q["pull_nblk"] >= 2
    inputs = GH.GpuInputs(wl, dev)
    b = M.EpBuffers(shape, dev)
    b.layout_notify(inputs.topk_idx)
    ent = b.ws[q["ws_pull_ent_offset"]:q["ws_pull_end"]].view(torch.int32).view(-1, 2)
    tb = q["pull_tb"]
    ent[0, 0] = wl.T * wl.k + 7        # a slot past the routed ones
    ent[1, 0] = tb * wl.k              # block 1's first slot, listed in block 0
    ent[2, 1] = wl.E + 3               # an expert id past E
    b.slot_to_row.fill_(-7)
    b.dispatch_scatter(inputs.x, inputs.x_scales, inputs.topk_idx, inputs.topk_weights)
    assert b.status() & M.binding.DEV_BAD_LAYOUT
    o = GH.oracle_run(orc, wl)
    s2r = b.slot_to_row.cpu().numpy().reshape(-1)
    want = o["slot_to_row"].reshape(-1)
    later = slice(tb * wl.k, wl.T * wl.k)  # blocks 1.. are untouched
    assert np.array_equal(s2r[later], want[later])
    assert s2r.max() < wl.T * wl.k


def test_bad_handle_is_reported_and_skipped(dev):
    wl = W.make_workload("bad_handle", 64, 64, 8, 2, 2, seed=83)
    bufs, inputs, st = GH.gpu_layout_dispatch(wl, dev)
    assert st == 0
    bufs.slot_to_row[5, 0] = wl.T * wl.k + 100   # outside the receive buffer
    r = int(bufs.slot_to_row[9, 1].item())
    bufs.recv_src_idx[r] = 0                     # row no longer names token 9
    eo = bufs.recv_x.view(torch.bfloat16)
    out = torch.empty((wl.T, wl.H), dtype=torch.float32, device=dev)
    bufs.combine(eo, out, M.FP32)
    assert bufs.status() & M.binding.DEV_BAD_HANDLE


@pytest.mark.parametrize("shuffled", [False, True])
def test_probe_fill(dev, shuffled):
    """Every 16-byte unit i is written exactly with {i, i >> 32, ~i, 0x5EED},
    in either chunk order (a chunk the permutation missed would stay zero)."""
    n = 2 * 32768 * 14336  # 917504 KiB: 229376 chunks of 4 KiB
    dst = torch.zeros(n // 4, dtype=torch.int32, device=dev)
    M.ep_probe_fill(dst, n, shuffled)
    torch.cuda.synchronize()
    i = torch.arange(n // 16, dtype=torch.int64, device=dev)
    lo = (i & 0xFFFFFFFF).to(torch.int64)
    want = torch.stack([lo, i >> 32, lo ^ 0xFFFFFFFF, torch.full_like(i, 0x5EED)], dim=1)
    want = torch.where(want >= 2**31, want - 2**32, want).to(torch.int32)
    assert torch.equal(dst.view(-1, 4), want)


def test_probe_copy(dev):
    n = 64 << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    M.ep_probe_copy(dst, src, n)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_probe_copy_ragged(dev):
    """A size that ends inside a workgroup's chunk: every byte copied, none
    past the end."""
    n16 = 3 * 1024 + 7
    src = torch.randint(0, 255, (n16 * 16,), dtype=torch.uint8, device=dev)
    dst = torch.zeros(n16 * 16 + 4096, dtype=torch.uint8, device=dev)
    M.ep_probe_copy(dst, src, n16 * 16)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n16 * 16], src)
    assert not dst[n16 * 16:].any()


def test_probe_read(dev):
    """The read probe stores its lane's fold only when it equals the fixed
    pattern: planted in the last, partial chunk, it reaches the sink."""
    n16 = 3 * 1024 + 7
    src = torch.zeros((n16, 4), dtype=torch.int64, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    M.ep_probe_read(src.to(torch.int32), n16 * 16, sink)
    torch.cuda.synchronize()
    assert not sink.any()
    want = [0x9E3779B9, 0x7F4A7C15, 11, 12]
    src[3 * 1024 + 3] = torch.tensor(want, dtype=torch.int64)
    s32 = torch.where(src >= 2**31, src - 2**32, src).to(torch.int32).contiguous()
    M.ep_probe_read(s32, n16 * 16, sink)
    torch.cuda.synchronize()
    assert sink.cpu().numpy().view(np.uint32).tolist() == want
