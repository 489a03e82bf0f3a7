// Internal declarations of libmoedisp (gfx950): workspace layout, launch plans
// and kernel launchers.  Not part of the public ABI (include/moedisp.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moedisp.h"

namespace moedisp {

// 16-byte unit of a row (one global_load/store_dwordx4 per lane).
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Streaming store of one 16-byte unit into a row that is written once and
// not read again by this kernel: buffer_store_dwordx4 with the non-temporal
// and both system-coherence bits (sc0 sc1 nt).  For the row copy of the
// scatter (k full-row writes per loaded row) this measured slightly faster
// on gfx950 than the plain non-temporal global store.  `row` (the row's base
// address) must be the same in every lane of the wave: it becomes the buffer
// descriptor (scalar registers).
constexpr int kStreamStorePolicy = 1 | 2 | 16;  // sc0 | nt | sc1
// Last word of a raw (untyped) buffer descriptor: data format 32 bits (field
// value 4 at bits 15..18), no swizzle, no index stride.  Accesses past
// `row_bytes` are dropped by the hardware; the callers stay inside the row.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kCombineStorePolicy = 16;  // sc1: the combine's bf16 output rows
__device__ inline void stream_store(v4u v, v4u* row, uint32_t row_bytes, int unit) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(row, (short)0, (int)row_bytes, kRawBufferWord3);
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, unit * 16, 0, kStreamStorePolicy);
}

constexpr int kThreads = 256;              // threads per workgroup (4 wave64s)
constexpr int kLayoutThreads = 1024;       // layout: one lane per slot, kLayoutThreads / k tokens per workgroup
constexpr int kReduceThreads = 512;        // layout reduce: one column of the partials per lane at E + G <= 512
constexpr int kMaxExperts = 4096;
constexpr int kMaxTopk = 32;
constexpr int kMaxGroups = 32;
constexpr int kMaxTileSlots = 4096;        // dispatch tile: tile_tokens * k routing ids in LDS
constexpr int kMaxTiles = 256;             // dispatch aims for at most this many tiles
constexpr int kMaxBlockTokens = 16;        // dispatch tokens copied per workgroup
constexpr int kMaxBlockSlots = 512;        // >= kMaxBlockTokens * kMaxTopk

// First 256 bytes of the workspace.
struct WsHeader {
    uint32_t status;           // MOEDISP_DEV_* bits, or-ed by kernels
    uint32_t reserved0;        // unused (kept zero)
    uint32_t reserved[62];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");

// How one dispatch splits work.  The count kernel runs one workgroup per tile
// of `tile_tokens` tokens and stores per-tile expert counts (expert-major,
// `tile_stride` >= tiles ints per expert, a multiple of 4).  The scatter kernel
// runs `blocks` workgroups of `threads` lanes: each computes the rows of and
// copies `block_tokens` consecutive tokens (inside one tile), restricted to
// one of `col_splits` column ranges of `split_units` lane units each (the
// last one may be shorter), `units_per_lane` units per lane and pass.  A lane
// unit is 16 bytes of the row for the copy and 16 channels for the
// quantising scatter.  The tile plan depends only on the shape, so the count
// kernel serves both scatter kernels.
struct DispatchPlan {
    int tile_tokens;
    int tiles;
    int tile_stride;
    int block_tokens;
    int col_splits;
    int split_units;
    int blocks;
    int threads;
    int units_per_lane;  // 1 or 2
};

constexpr int kMaxDispatchThreads = 1024;

// Static LDS of a push scatter workgroup (both scatter kernels).
struct ScatterSmem {
    int32_t pre[kMaxBlockSlots];   // counts of the slot's expert in earlier tiles
    int32_t base[kMaxBlockSlots];  // expert_offsets[e]
    int32_t len[kMaxBlockSlots];   // tokens_per_expert[e]
    int32_t rows[kMaxBlockSlots + 8];  // receive row of each slot of the workgroup, -1 if none
                                       // (8 spare entries: the stores read rows 8 at a time)
    int32_t routed_tok[kMaxBlockTokens];  // nonzero if the token has a receive row
    int32_t routed;
    uint32_t err;
};

// Block-pull dispatch.  The tokens are cut into nblk blocks of tb tokens
// (the last one may be shorter), and block b is copied by workgroups that the
// hardware's round-robin dispatch places on XCD b % kXcds: a block's source
// rows (tb * row bytes, kept below kPullL2Bytes) are read from HBM once and
// then served by that XCD's L2 for each of their k copies, and the block's
// receive rows are written in ascending address order, one run per expert.
// The notify phase sorts each block's slots by (expert, slot) into a list of
// cap_b = tb * k entries (routed entries first, then the masked ones); copy
// workgroup j of a block writes the receive rows of list entries
// [j * rpw, (j + 1) * rpw).  Shapes this does not fit (small T, many experts,
// very large T) take the push scatter (DispatchPlan).
struct PullPlan {
    int use;          // 0: the push scatter serves this shape
    int tb;           // tokens per block
    int nblk;         // blocks (8 <= nblk <= kPullMaxBlocks)
    int cap_b;        // list entries per block (tb * k <= kPullMaxBlockSlots)
    int cnt_stride;   // ints per expert column of the per-block counts (>= nblk, multiple of 4)
    int rpw;          // list entries (receive rows) per copy workgroup (1)
    int threads;      // copy workgroup lanes
    int units;        // 16-byte units per lane and pass (2, or 3 for rows over 512 units; 4 when compact)
    int wpb;          // copy workgroups per block: ceil(cap_b / rpw)
    long long blocks; // copy grid: kXcds * wpb * ceil(nblk / kXcds), or kXcds * wq when compact
    int compact;      // 1: lists hold the routed entries only; the sort writes masked slots' handles
    int wq;           // compact: copy workgroups per XCD (each takes every wq-th entry of its XCD)
};

constexpr int kXcds = 8;                          // XCDs of an MI355X (round-robin workgroup dispatch)
constexpr long long kPullL2Bytes = 3584 * 1024;   // source bytes per block: below one XCD's 4 MB L2
constexpr int kPullMaxExperts = 512;              // per-wave expert tables of the sort fit LDS
constexpr int kPullMaxBlockSlots = 4096;          // slots of one block sorted in LDS
constexpr int kPullMaxBlocks = 256;               // a row's count prefix is one 16-byte load per lane of a wave
constexpr int kPullMinBlockTokens = 32;
constexpr int kPullMaskWords = 4096;              // the sort's token masks: E * ceil(tb / 64) 64-bit words at most
constexpr int kPullCompactUnits = 4;              // 16-byte units per lane of the compact-list copy
constexpr int kNotifyThreads = 1024;              // lanes of a notify workgroup (16 waves)

__host__ __device__ inline int sort_mask_words(int tb) { return (tb + 63) / 64; }

// LDS words of the sort: token masks [E][mask words] (64-bit; one word of
// padding so that they start 8-byte aligned wherever the area starts), ids
// [cap_b], expert counts [E], masked counts per 64 slots [cap_b / 64 + 1],
// the routed total and a repeat flag.
__host__ __device__ inline size_t sort_lds_words(int tb, int cap_b, int E) {
    return 1 + 2 * (size_t)E * sort_mask_words(tb) + (size_t)cap_b + (size_t)E + (size_t)cap_b / 64 + 3;
}

// One entry of a block's sorted list: flat slot t * k + j and its expert
// (-1 for a masked or invalid slot).
struct PullEnt {
    int32_t slot;
    int32_t expert;
};

struct CombinePlan {
    int col_splits;
    int blocks;
    int threads;
    int units_per_lane;  // 1 or 2 (16-byte units per lane, one pass)
};

constexpr int kMaxCombineThreads = 1024;

struct WsPlan {
    int layout_blocks;
    size_t partial_offset;   // int32 [layout_blocks][E + G]
    size_t counts_offset;    // int32 [E][tile_stride]: per-tile expert counts of the dispatch
    size_t pull_cnt_offset;  // block-pull: int32 [E][cnt_stride] routed slots per (expert, block)
    size_t pull_ls_offset;   // block-pull: int32 [nblk][E] first list entry of each expert in a block
    size_t pull_n_offset;    // block-pull: int32 [nblk] routed entries per block
    size_t pull_ent_offset;  // block-pull: PullEnt [nblk][cap_b] sorted lists
    // the same four tables of the group rows' local expert permutation
    // (compact lists), laid out from the same base: the two are never used
    // by one call, so the region is the larger of the two
    size_t perm_cnt_offset, perm_ls_offset, perm_n_offset, perm_ent_offset;
    size_t total;
};

DispatchPlan plan_dispatch(const moedisp_shape& s);
PullPlan plan_pull(const moedisp_shape& s, long long compact_entries = 0);
PullPlan plan_pull_permute(const moedisp_shape& s);
DispatchPlan plan_dispatch_quant(const moedisp_shape& s);
DispatchPlan plan_dispatch_groups(const moedisp_shape& s);
moedisp_shape group_rows_shape(const moedisp_shape& s);
CombinePlan plan_combine(const moedisp_shape& s, int loads_per_row);
WsPlan plan_workspace(const moedisp_shape& s);

struct SmallPlan {
    int supported;    // T * k and the LDS tables within the path's bounds
    int col_splits, split_units, threads;
    long long blocks;
    size_t lds_bytes;
};
SmallPlan plan_small(const moedisp_shape& s);

struct LayoutNotifyPlan {
    int fused;       // tile counts in the layout's workgroups (else two calls)
    int tile_shift;  // log2 of the dispatch tile
};
LayoutNotifyPlan plan_layout_notify(const moedisp_shape& s);
inline int layout_tokens_per_block(const moedisp_shape& s) { return kLayoutThreads / s.topk; }
// LDS of a layout workgroup (tiles_per_block > 0 with the notify phase folded in)
inline size_t layout_lds_bytes(int E, int G, int k, int tokens_per_block, int tiles_per_block) {
    return ((size_t)E + G + (size_t)tokens_per_block * (k + 1) + (size_t)tiles_per_block * E) * sizeof(int32_t);
}

inline size_t row_bytes(const moedisp_shape& s) {
    return (size_t)s.hidden * (s.x_dtype == MOEDISP_FP8_E4M3 ? 1 : 2);
}
inline int scales_per_row(const moedisp_shape& s) {
    return s.x_dtype == MOEDISP_FP8_E4M3 ? s.hidden / s.scale_block : 0;
}

struct LayoutArgs {
    int T, k, E, G;
    int id_bits;        // bits of an expert id (ceil(log2 E))
    int pg_shift;       // log2(E/G) if E/G is a power of two, else -1
    uint32_t pg_magic;  // floor(2^32 / (E/G)) + 1 otherwise
    int k_shift;        // lane / k the same way
    uint32_t k_magic;
    int tokens_per_block;  // kLayoutThreads / k
    const int32_t* topk_idx;
    int32_t* tokens_per_expert;
    int32_t* tokens_per_group;
    uint32_t* is_token_in_group;
    WsHeader* hdr;
    int32_t* partials;
    int blocks;
    // the dispatch's notify phase in the same launches (ep_get_dispatch_layout_notify)
    // when tile_counts != nullptr: per-tile expert counts in the dispatch's tile
    // geometry (2^tile_shift tokens per tile, dividing tokens_per_block; tiles
    // tiles; tile_stride ints per expert) and expert_offsets [E+1]
    int32_t* tile_counts;
    int tile_shift;
    int tiles;
    int tile_stride;
    int32_t* expert_offsets;
    int capacity;
};

struct DispatchArgs {
    int T, k, E;
    int row16;         // 16-byte units per source row
    int out16;         // 16-byte units per received row (quantising scatter)
    int scale_words;   // fp32 scales per row of an fp8 input (0 without scales)
    int q_block_lanes;     // quantising scatter: lanes (16 channels each) per scale block
    int q_scales_per_row;  // quantising scatter: scale blocks per row
    int capacity;      // T * k receive rows
    DispatchPlan plan;
    const v4u* x;
    const float* x_scales;
    const int32_t* topk_idx;
    const float* topk_weights;
    const int32_t* tokens_per_expert;
    v4u* recv_x;
    float* recv_scales;
    int32_t* recv_src_idx;
    float* recv_weights;
    int32_t* expert_offsets;
    int32_t* slot_to_row;
    void* recv_qscales;  // quantising scatter: fp32 or UE8M0 bytes [rows][q_scales_per_row]
    // group mode (group-deduplicated dispatch) when bitmap != nullptr: the
    // "experts" are the G groups, slot g of token t is routed iff bit g of
    // bitmap[t] is set, k = E = G, and each row also gets the token's src_k
    // slots restricted to its group (recv_topk_idx / recv_topk_weights)
    const uint32_t* bitmap;
    int src_k;
    int experts_per_group;
    int32_t* recv_topk_idx;
    float* recv_topk_weights;
    WsHeader* hdr;
    int32_t* tile_counts;
    // block-pull tables (pull.use != 0)
    PullPlan pull;
    int32_t* pull_cnt;
    int32_t* pull_ls;
    int32_t* pull_n;
    PullEnt* pull_ent;
};

// The notify launch of the block-pull dispatch: one launch whose workgroups
// take one of three roles by index: [0, sort_wgs) sort one block each;
// [sort_wgs, sort_wgs + count_wgs) count one dispatch tile each (the tables
// of the push path, which the quantising scatter reads), tile 0 also writing
// expert_offsets when count_offsets is set; a last workgroup, if reduce is
// set, sums the layout's partial counts (tokens_per_expert, tokens_per_group,
// expert_offsets).  No role waits for another.
struct NotifyArgs {
    DispatchArgs d;
    LayoutArgs lay;
    int id_bits;        // bits of an expert id (ceil(log2 E))
    int sort_wgs;
    int count_wgs;
    int count_offsets;
    int reduce;         // last workgroup: 0 none, 1 the layout's reduce, 2 the offsets scan
};

// The layout's workgroups and the block-pull sort's in one launch.
struct LayoutSortArgs {
    LayoutArgs lay;
    DispatchArgs d;
    int id_bits;
    int sort_wgs;
};

struct CombineArgs {
    int T, k;
    int row16;
    int capacity;
    int col_splits;
    int threads;
    int units_per_lane;
    const v4u* expert_out;
    const int32_t* recv_src_idx;
    const float* recv_weights;  // nullptr: every weight is 1 (plain sum)
    const int32_t* slot_to_row;
    const int32_t* row_limit;   // if set, output rows >= *row_limit are skipped (not written)
    void* out;
    WsHeader* hdr;
};

// Small-batch path: layout and dispatch in one launch (every workgroup
// stages the whole routing table, so T*k is bounded).
constexpr int kFusedMaxSlots = 8192;

struct FusedArgs {
    int T, k, E, G;
    int experts_per_group;
    int pg_shift;       // log2(E/G) if E/G is a power of two, else -1
    uint32_t pg_magic;  // floor(2^32 / (E/G)) + 1 otherwise (exact for ids < 4096)
    int row16;
    int scale_words;
    int capacity;
    int col_splits, split_units, threads;
    // padded layout (pad_s > 0): expert e's slots take rows e*pad_s + pad_b + i
    // for i < pad_c (i = the slot's rank among e's routed slots)
    int pad_c, pad_s, pad_b;
    const v4u* x;
    const float* x_scales;
    const int32_t* topk_idx;
    const float* topk_weights;
    int32_t* tokens_per_expert;
    int32_t* tokens_per_group;
    uint32_t* is_token_in_group;
    v4u* recv_x;
    float* recv_scales;
    int32_t* recv_src_idx;
    float* recv_weights;
    int32_t* expert_offsets;
    int32_t* slot_to_row;
    WsHeader* hdr;
};

// A dispatch packet holds the grid size in work-items as 32 bits: a launch of
// `blocks` workgroups of `threads` lanes must stay below 2^32 work-items.
// Launchers return hipErrorInvalidConfiguration otherwise (the C ABI reports
// MOEDISP_ERR_UNSUPPORTED).
inline bool grid_fits(long long blocks, long long threads) {
    return blocks >= 1 && blocks <= 0x7FFFFFFFll && blocks * threads <= 0xFFFFFFFFll;
}

// reduce = false: the partial counts only (moedisp_layout), no reduce launch
hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream, bool reduce = true);
hipError_t launch_dispatch_fused(const FusedArgs& a, hipStream_t stream);
hipError_t launch_dispatch_notify(const DispatchArgs& a, hipStream_t stream);
hipError_t launch_dispatch_scatter(const DispatchArgs& a, hipStream_t stream);
hipError_t launch_notify(const NotifyArgs& a, hipStream_t stream);
hipError_t launch_layout_sort(const LayoutSortArgs& a, hipStream_t stream);
hipError_t launch_layout_reduce(const LayoutArgs& a, hipStream_t stream);
hipError_t launch_scatter_pull(const DispatchArgs& a, hipStream_t stream);
size_t notify_lds_bytes(const NotifyArgs& a);
hipError_t launch_dispatch_scatter_quant(const DispatchArgs& a, int scale_fmt, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, bool f32_out, hipStream_t stream);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_set_word(uint32_t* p, uint32_t value, hipStream_t stream);
hipError_t launch_probe_copy(v4u* dst, const v4u* src, size_t n16, hipStream_t stream);
hipError_t launch_probe_read(const v4u* src, size_t n16, v4u* sink, hipStream_t stream);
hipError_t launch_probe_fill(v4u* dst, size_t chunks, size_t mult, hipStream_t stream);

}  // namespace moedisp
