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
__device__ inline void stream_store(v4u v, v4u* row, uint32_t row_bytes, int unit) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(row, (short)0, (int)row_bytes, kRawBufferWord3);
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, unit * 16, 0, kStreamStorePolicy);
}

constexpr int kThreads = 256;              // threads per workgroup (4 wave64s)
constexpr int kLayoutThreads = 1024;       // layout: one lane per slot, kLayoutThreads / k tokens per workgroup
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
    size_t total;
};

DispatchPlan plan_dispatch(const moedisp_shape& s);
DispatchPlan plan_dispatch_quant(const moedisp_shape& s);
DispatchPlan plan_dispatch_groups(const moedisp_shape& s);
moedisp_shape group_rows_shape(const moedisp_shape& s);
CombinePlan plan_combine(const moedisp_shape& s, int loads_per_row);
WsPlan plan_workspace(const moedisp_shape& s);
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

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream);
hipError_t launch_dispatch_fused(const FusedArgs& a, hipStream_t stream);
hipError_t launch_dispatch_notify(const DispatchArgs& a, hipStream_t stream);
hipError_t launch_dispatch_scatter(const DispatchArgs& a, hipStream_t stream);
hipError_t launch_dispatch_scatter_quant(const DispatchArgs& a, int scale_fmt, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, bool f32_out, hipStream_t stream);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_set_word(uint32_t* p, uint32_t value, hipStream_t stream);
hipError_t launch_copy(v4u* dst, const v4u* src, size_t n16, hipStream_t stream);
hipError_t launch_probe_fill(v4u* dst, size_t chunks, size_t mult, hipStream_t stream);

}  // namespace moedisp
