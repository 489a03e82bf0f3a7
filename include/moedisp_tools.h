/* libmoedisp tools: entry points that are not part of the dispatch / combine
 * path, exported by the same library.
 *
 * Calibration probes measure the part's achievable HBM bandwidth in the same
 * process as a benchmark and give kernels of known traffic against which
 * hardware byte counters are scaled.  Each probe runs on `stream` (NULL: the
 * null stream) and returns a host code of moedisp.h (MOEDISP_OK, or
 * INVALID_ARG / UNSUPPORTED / MISALIGNED when the arguments break the rules
 * stated below, before anything is launched; HIP when the launch fails).
 * Buffers are device memory that the caller owns.  The read and copy probes
 * give every workgroup of 512 lanes one 16 KiB chunk (two 16-byte units per
 * lane, non-temporal loads and stores) and exit: the shape that measured
 * fastest on this part among one-chunk-per-workgroup and grid-stride kernels
 * with 256 to 1024 lanes, 1 to 8 loads in flight per lane and chunks of
 * 4 KiB to 256 KiB.
 *
 * The plan query reports, for a shape, the launch geometry, LDS and
 * workspace layout the path's entry points would use, so that host-side
 * limits can be checked over many shapes without a GPU. */
#ifndef MOEDISP_TOOLS_H
#define MOEDISP_TOOLS_H

#include <stddef.h>
#include <stdint.h>

#include "moedisp.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read-only stream: reads `bytes` from `src` (a multiple of 16; 16-byte
 * aligned) and folds them by XOR; `sink` (16 bytes, 16-byte aligned) is
 * written only if the fold hits a fixed 64-bit pattern, so the reads cannot
 * be dropped.  The ceiling of kernels that mostly read (a gather-sum). */
int ep_probe_read(const void* src, size_t bytes, void* sink, void* stream);

/* Copy of `bytes` (a multiple of 16; both pointers 16-byte aligned, buffers
 * not overlapping) from `src` to `dst`.  The ceiling of kernels that read
 * and write in equal parts, and the known traffic (bytes read, bytes
 * written) that scales hardware byte counters. */
int ep_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Writes `bytes` (a multiple of 4096; dst 16-byte aligned) in 4 KiB chunks,
 * one workgroup per chunk, the chunks in address order (shuffled = 0) or in
 * a fixed permuted order (shuffled = 1).  16-byte unit i of the buffer
 * receives the four 32-bit words {i mod 2^32, i / 2^32, ~(i mod 2^32),
 * 0x5EED}, whatever the order.  Measures the HBM write bandwidth of
 * sequential against scattered write streams, the two ends between which a
 * row scatter's writes fall.  Returns UNSUPPORTED for a size that is not a
 * multiple of 4096 or a `shuffled` other than 0 or 1. */
int ep_probe_fill(void* dst, size_t bytes, int32_t shuffled, void* stream);

/* One kernel launch: workgroups, lanes per workgroup, dynamic LDS bytes and
 * an upper bound of the kernel's static LDS bytes. */
typedef struct moedisp_launch_info {
    int64_t blocks;
    int64_t threads;
    int64_t lds_bytes;
    int64_t static_lds_bytes;
} moedisp_launch_info;

/* What the entry points of moedisp.h would launch for one shape.  Launches a
 * shape does not make (the pull copy of a push shape, the small path of a
 * large one) are reported all zero. */
typedef struct moedisp_plan_info {
    int64_t struct_bytes;          /* sizeof(moedisp_plan_info) */
    /* ep_get_dispatch_layout */
    moedisp_launch_info layout, layout_reduce;
    int64_t layout_tokens_per_block;
    /* ep_get_dispatch_layout_notify: 1 if the dispatch's tile counts are
     * folded into the layout's workgroups; the layout launch it makes (with
     * the tile counts, and with the block sorts when the pull copy serves) */
    int64_t layout_notify_fused;
    moedisp_launch_info layout_notify;
    /* flat dispatch, push scatter: count tiles and the copy */
    int64_t tile_tokens, tiles, tile_stride;
    int64_t block_tokens, block_slots, col_splits, split_units, units_per_lane;
    moedisp_launch_info count, scatter;
    /* flat dispatch, block-pull copy (pull = 1 when it serves the shape) */
    int64_t pull, pull_tb, pull_nblk, pull_cap_b, pull_cnt_stride, pull_rows_per_wg, pull_units;
    moedisp_launch_info pull_notify, pull_copy;
    /* quantising scatter (its tiles are the flat dispatch's) */
    int64_t quant_block_slots;
    moedisp_launch_info scatter_quant;
    /* group path: group dispatch, local permutation, reduce, group combine */
    int64_t group_rows;
    int64_t groups_tile_stride, groups_tiles, groups_block_slots;
    int64_t permute_tile_stride, permute_tiles, permute_block_slots;
    moedisp_launch_info groups_count, groups_scatter, permute_count, permute_scatter, group_reduce, combine_groups;
    /* local permutation by block-pull copy over blocks of group rows with
     * compact lists (permute_pull = 1 when it serves the shape; the permute_
     * push fields above are then zero): block sorts with the offsets scan,
     * then permute_pull_wgs_per_xcd copy workgroups per XCD */
    int64_t permute_pull, permute_pull_tb, permute_pull_nblk, permute_pull_cap_b, permute_pull_cnt_stride;
    int64_t permute_pull_units, permute_pull_wgs_per_xcd;
    moedisp_launch_info permute_pull_notify, permute_pull_copy;
    /* ep_combine */
    int64_t combine_col_splits, combine_units_per_lane;
    moedisp_launch_info combine;
    /* ep_layout_dispatch_small (small = 1 when the shape is supported) */
    int64_t small;
    moedisp_launch_info small_fused;
    /* workspace (byte offsets into ws; ws_total = ep_workspace_bytes) */
    int64_t ws_total, ws_partial_offset, ws_partial_bytes, ws_counts_offset, ws_counts_bytes;
    int64_t ws_counts_needed_flat, ws_counts_needed_groups, ws_counts_needed_rows;
    int64_t ws_pull_cnt_offset, ws_pull_ls_offset, ws_pull_n_offset, ws_pull_ent_offset, ws_pull_end;
    /* the permutation's tables share the flat tables' base (never one call) */
    int64_t ws_permute_pull_cnt_offset, ws_permute_pull_ls_offset, ws_permute_pull_n_offset;
    int64_t ws_permute_pull_ent_offset, ws_permute_pull_end;
    /* limits the kernels assume */
    int64_t max_block_slots, max_tile_slots, max_threads, pull_max_block_slots, pull_max_blocks;
} moedisp_plan_info;

/* Fills *info for `shape` (all fields; zero where a launch is not made).
 * Returns the shape check's code (INVALID_ARG / UNSUPPORTED for shapes the
 * entry points reject; *info is then left zero), or INVALID_ARG when info is
 * NULL or info_bytes is not sizeof(moedisp_plan_info).  Touches no device. */
int ep_plan_query(const moedisp_shape* shape, moedisp_plan_info* info, size_t info_bytes);

#ifdef __cplusplus
}
#endif

#endif /* MOEDISP_TOOLS_H */
