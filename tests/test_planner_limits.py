"""Host planners against the limits their kernels assume, over many shapes
(no GPU): T in [0, 1e6], E up to 4096, G up to 32, k up to 32, bf16 and fp8
rows from 16 bytes to 80 KB.  Through ep_plan_query, for every shape the
library accepts:
  - every launch's dynamic plus static LDS <= 64 KiB (the small path's
    tables <= 60 KiB), lanes whole waves <= 1024 (grids of 2^32 lanes or
    more are rejected by the launchers' own check);
  - push scatter: slots per workgroup <= kMaxBlockSlots, a workgroup's tokens
    inside one count tile, tiles cover T, tiles <= the count table's stride,
    column ranges cover the row, one lane per slot;
  - block-pull copy: blocks of >= 32 tokens that cover T, 8 <= blocks <= 256,
    a block's slots <= 4096 and its source rows <= 3.5 MiB, the sort's token
    masks within bounds, an fp8 row's scales one per lane; the same for the
    group rows' permutation (compact lists), whose copy grid is 8 workgroups
    per XCD slot, at most one per entry an XCD's blocks can hold;
  - workspace: 256-byte-aligned regions in order, each large enough for the
    table the kernels index (layout partials, the largest per-tile count
    table, the pull tables), all inside ep_workspace_bytes."""
import ctypes as C
import itertools

import numpy as np
import pytest

import combine_ep_get_dispatch_amd as M
from combine_ep_get_dispatch_amd import binding as B

LDS = 64 * 1024
L2_BLOCK = 3584 * 1024


def shapes():
    Ts = [0, 1, 2, 7, 31, 32, 100, 127, 128, 255, 256, 257, 600, 1000, 2047, 2048, 2049, 4096, 4097, 10000,
          16384, 32768, 65536, 100000, 262144, 1000000]
    EGs = [(1, 1), (2, 2), (3, 1), (8, 2), (8, 8), (16, 4), (64, 8), (100, 4), (256, 8), (256, 32), (384, 8),
           (512, 8), (513, 1), (1024, 32), (4096, 32)]
    ks = [1, 2, 3, 6, 8, 9, 16, 32]
    rows = [(8, 0), (64, 0), (1000, 0), (2048, 0), (4096, 0), (7168, 0), (40000, 0),
            (128, 128), (2048, 128), (7168, 128), (7168, 32)]
    full = [(T, H, E, G, k, sb) for T in Ts for (E, G) in EGs for k in ks for (H, sb) in rows if k <= E]
    rng = np.random.default_rng(7)
    pick = rng.choice(len(full), size=min(len(full), 12000), replace=False)
    sel = [full[i] for i in sorted(pick)]
    # every combination at the DeepSeek-V3 row and at the largest T
    sel += [s for s in full if s[1] == 7168 and s[5] == 0 or s[0] == 1000000]
    return sorted(set(sel))


def check_launch(name, l, lds_cap=LDS):
    """A grid of 2^32 lanes or more is allowed: every launcher checks it and
    the entry point returns UNSUPPORTED before launching anything."""
    assert l.blocks >= 1, name
    assert 1 <= l.threads <= 1024 and l.threads % 64 == 0, (name, l.threads)
    assert l.lds_bytes + l.static_lds_bytes <= lds_cap, (name, l.lds_bytes, l.static_lds_bytes)


def check_push(name, sh, q, launch, k, tile_tokens, tiles, tile_stride, block_tokens, row16, ctx):
    check_launch(name, launch)
    bt = block_tokens
    assert bt * k <= q.max_block_slots, (ctx, name, bt, k)
    assert tile_tokens % bt == 0, (ctx, name, tile_tokens, bt)          # a workgroup inside one tile
    assert tile_tokens * k <= q.max_tile_slots, (ctx, name)
    assert tiles * tile_tokens >= sh.num_tokens, (ctx, name)
    assert tiles <= tile_stride and tile_stride % 4 == 0, (ctx, name, tiles, tile_stride)
    assert launch.threads >= min(bt * k, 1024), (ctx, name)            # one lane per slot


def check(L, sh, q):
    T, H, E, G, k = sh.num_tokens, sh.hidden, sh.num_experts, sh.num_groups, sh.topk
    rb = H * (1 if sh.x_dtype == M.FP8_E4M3 else 2)
    row16 = rb // 16
    ctx = (T, H, E, G, k, sh.x_dtype, sh.scale_block)
    assert q.struct_bytes == C.sizeof(B.moedisp_plan_info)
    # layout (and the launch with the notify phase / block sorts folded in)
    check_launch("layout", q.layout)
    check_launch("layout_reduce", q.layout_reduce)
    assert q.layout_tokens_per_block * k <= 1024
    assert q.layout.blocks * q.layout_tokens_per_block >= T, ctx
    check_launch("layout_notify", q.layout_notify)
    # push scatter and its count tiles
    check_launch("count", q.count)
    assert q.count.blocks == q.tiles
    assert q.split_units * q.col_splits >= row16 > (q.col_splits - 1) * q.split_units, ctx
    assert q.block_slots == q.block_tokens * k
    check_push("scatter", sh, q, q.scatter, k, q.tile_tokens, q.tiles, q.tile_stride, q.block_tokens, row16, ctx)
    # block-pull
    if q.pull:
        tb, nblk, cap = q.pull_tb, q.pull_nblk, q.pull_cap_b
        assert tb >= 32 and 8 <= nblk <= q.pull_max_blocks, ctx
        assert nblk * tb >= T > (nblk - 1) * tb, ctx
        assert cap == tb * k <= q.pull_max_block_slots, ctx
        assert tb * rb <= L2_BLOCK, ctx
        assert E <= 512 and E * ((tb + 63) // 64) <= 4096, ctx
        assert q.pull_cnt_stride >= nblk and q.pull_cnt_stride % 4 == 0, ctx
        check_launch("pull_notify", q.pull_notify)
        check_launch("pull_copy", q.pull_copy)
        wpb = -(-cap // q.pull_rows_per_wg)
        assert q.pull_copy.blocks == 8 * wpb * -(-nblk // 8), ctx
        if sh.scale_block:
            assert H // sh.scale_block <= q.pull_copy.threads, ctx
    else:
        assert q.pull_copy.blocks == 0 and q.pull_nblk == 0
    # quantising scatter (same tiles), group dispatch, local permutation
    if sh.x_dtype == M.BF16 and H % 32 == 0:
        check_push("scatter_quant", sh, q, q.scatter_quant, k, q.tile_tokens, q.tiles, q.tile_stride,
                   q.quant_block_slots // k, row16, ctx)
    else:
        assert q.scatter_quant.blocks == 0
    assert q.group_rows == T * min(G, k)
    check_launch("groups_count", q.groups_count)
    assert q.groups_block_slots <= q.max_block_slots and q.groups_tiles <= q.groups_tile_stride, ctx
    check_launch("groups_scatter", q.groups_scatter)
    if q.permute_pull:
        TR = q.group_rows
        tb, nblk, cap = q.permute_pull_tb, q.permute_pull_nblk, q.permute_pull_cap_b
        assert tb >= 32 and 8 <= nblk <= q.pull_max_blocks, ctx
        assert nblk * tb >= TR > (nblk - 1) * tb, ctx
        assert cap == tb * k <= q.pull_max_block_slots, ctx
        assert tb * rb <= L2_BLOCK, ctx
        assert E <= 512 and E * ((tb + 63) // 64) <= 4096, ctx
        assert q.permute_pull_cnt_stride >= nblk and q.permute_pull_cnt_stride % 4 == 0, ctx
        check_launch("permute_pull_notify", q.permute_pull_notify)
        check_launch("permute_pull_copy", q.permute_pull_copy)
        wq = q.permute_pull_wgs_per_xcd
        assert 1 <= wq <= cap * -(-nblk // 8), ctx
        assert q.permute_pull_copy.blocks == 8 * wq, ctx
        assert q.permute_pull_notify.blocks == nblk + 1, ctx
        if sh.scale_block:
            assert H // sh.scale_block <= q.permute_pull_copy.threads, ctx
        assert q.permute_scatter.blocks == 0 and q.permute_count.blocks == 0, ctx
    else:
        assert q.permute_pull_copy.blocks == 0 and q.permute_pull_nblk == 0
        check_launch("permute_count", q.permute_count)
        assert q.permute_block_slots <= q.max_block_slots and q.permute_tiles <= q.permute_tile_stride, ctx
        check_launch("permute_scatter", q.permute_scatter)
        assert q.permute_tile_stride % 4 == 0
    # combines
    if T > 0:
        for n in ("combine", "group_reduce", "combine_groups"):
            check_launch(n, getattr(q, n))
        assert q.combine.blocks == T * q.combine_col_splits, ctx
    # small path
    if q.small:
        assert T * k <= 8192, ctx
        check_launch("small", q.small_fused, 60 * 1024 + q.small_fused.static_lds_bytes)
    # workspace
    assert q.ws_total == L.ep_workspace_bytes(C.byref(sh)), ctx
    offs = [q.ws_partial_offset, q.ws_counts_offset, q.ws_pull_cnt_offset, q.ws_pull_ls_offset,
            q.ws_pull_n_offset, q.ws_pull_ent_offset]
    assert q.ws_partial_offset >= 256
    assert all(o % 256 == 0 for o in offs[1:]) and offs == sorted(offs), (ctx, offs)
    assert q.ws_counts_offset >= q.ws_partial_offset + q.ws_partial_bytes, ctx
    assert q.ws_partial_bytes == q.layout.blocks * (E + G) * 4
    need = max(q.ws_counts_needed_flat, q.ws_counts_needed_groups, q.ws_counts_needed_rows)
    assert q.ws_counts_bytes >= need, (ctx, q.ws_counts_bytes, need)
    assert q.ws_counts_needed_flat == q.tile_stride * E * 4 and q.ws_counts_needed_groups == q.groups_tile_stride * G * 4
    if q.pull:
        assert q.ws_pull_ls_offset >= q.ws_pull_cnt_offset + E * q.pull_cnt_stride * 4, ctx
        assert q.ws_pull_n_offset >= q.ws_pull_ls_offset + q.pull_nblk * E * 4, ctx
        assert q.ws_pull_ent_offset >= q.ws_pull_n_offset + q.pull_nblk * 4, ctx
        assert q.ws_pull_end == q.ws_pull_ent_offset + q.pull_nblk * q.pull_cap_b * 8, ctx
    assert q.ws_pull_end <= q.ws_total, ctx
    # the permutation's tables: from the same base as the flat ones
    poffs = [q.ws_permute_pull_cnt_offset, q.ws_permute_pull_ls_offset, q.ws_permute_pull_n_offset,
             q.ws_permute_pull_ent_offset]
    assert poffs[0] == q.ws_pull_cnt_offset, ctx
    assert all(o % 256 == 0 for o in poffs) and poffs == sorted(poffs), (ctx, poffs)
    if q.permute_pull:
        nblk = q.permute_pull_nblk
        assert poffs[1] >= poffs[0] + E * q.permute_pull_cnt_stride * 4, ctx
        assert poffs[2] >= poffs[1] + nblk * E * 4, ctx
        assert poffs[3] >= poffs[2] + nblk * 4, ctx
        assert q.ws_permute_pull_end == poffs[3] + nblk * q.permute_pull_cap_b * 8, ctx
    assert q.ws_permute_pull_end <= q.ws_total, ctx


def test_planner_limits_over_shapes():
    L = M.load()
    q = B.moedisp_plan_info()
    n_ok = n_pull = n_small = n_perm = 0
    for (T, H, E, G, k, sb) in shapes():
        for dt in ((M.BF16,) if sb == 0 else (M.FP8_E4M3,)):
            sh = M.moedisp_shape.make(T, H, E, G, k, dt, sb)
            rc = L.ep_plan_query(C.byref(sh), C.byref(q), C.sizeof(q))
            if rc != B.OK:
                assert rc in (B.ERR_INVALID_ARG, B.ERR_UNSUPPORTED)
                continue
            check(L, sh, q)
            n_ok += 1
            n_pull += q.pull
            n_small += q.small
            n_perm += q.permute_pull
    # the sweep reaches every planner branch
    assert n_ok > 5000 and n_pull > 500 and n_small > 500 and n_perm > 500, (n_ok, n_pull, n_small, n_perm)


def test_plan_query_rejects_like_the_entry_points():
    L = M.load()
    q = B.moedisp_plan_info()
    assert L.ep_plan_query(C.byref(M.moedisp_shape.make(16, 64, 8, 2, 2)), C.byref(q), 8) == B.ERR_INVALID_ARG
    assert L.ep_plan_query(C.byref(M.moedisp_shape.make(16, 64, 8, 2, 2)), None, C.sizeof(q)) == B.ERR_INVALID_ARG
    assert L.ep_plan_query(C.byref(M.moedisp_shape.make(16, 64, 255, 2, 2)), C.byref(q), C.sizeof(q)) == \
        B.ERR_INVALID_ARG
    assert q.ws_total == 0  # left zero
    assert L.ep_plan_query(C.byref(M.moedisp_shape.make(16, 64, 8192, 32, 2)), C.byref(q), C.sizeof(q)) == \
        B.ERR_UNSUPPORTED


def test_plan_struct_matches_header():
    """The binding's ctypes layout of moedisp_plan_info is the header's."""
    import os
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    h = open(os.path.join(root, "include", "moedisp_tools.h")).read()
    body = h[h.index("typedef struct moedisp_plan_info {"):h.index("} moedisp_plan_info;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    body = body[body.index("{") + 1:]
    fields = []
    for decl in body.split(";"):
        decl = " ".join(decl.split())
        if decl:
            typ, rest = decl.split(None, 1)
            fields += [(typ, n.strip()) for n in rest.split(",")]
    mine = [("moedisp_launch_info" if t is B.moedisp_launch_info else "int64_t", n)
            for n, t in B.moedisp_plan_info._fields_]
    assert fields == mine
    assert M.ep_plan_query(M.moedisp_shape.make(4096, 7168, 256, 8, 8))["struct_bytes"] == C.sizeof(B.moedisp_plan_info)
