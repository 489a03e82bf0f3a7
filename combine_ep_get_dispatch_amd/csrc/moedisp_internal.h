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

constexpr int kThreads = 256;              // threads per workgroup (4 wave64s)
constexpr int kLayoutTokensPerBlock = 256; // layout: one token per thread
constexpr int kMaxExperts = 4096;
constexpr int kMaxTopk = 32;
constexpr int kMaxGroups = 32;
constexpr int kMaxTileTokens = 32;         // dispatch look-back tile
constexpr int kMaxBlockTokens = 16;        // dispatch tokens copied per workgroup
constexpr uint32_t kDefaultSpinLimit = 1u << 18;

// Look-back words: [63:32] epoch of the dispatch call, [31:30] flag, [29:0] value.
constexpr uint32_t kFlagAggregate = 1u;  // value = this tile's count for the expert
constexpr uint32_t kFlagPrefix = 2u;     // value = inclusive prefix through this tile
constexpr uint32_t kValueMask = (1u << 30) - 1u;

// First 256 bytes of the workspace.
struct WsHeader {
    uint32_t status;           // MOEDISP_DEV_* bits, or-ed by kernels
    uint32_t layout_done;      // layout workgroups finished (the last one reduces)
    uint32_t dispatch_ticket;  // dispatch workgroup order (taken at start)
    uint32_t dispatch_done;    // dispatch workgroups finished
    uint32_t epoch;            // dispatch calls completed; tags look-back words
    uint32_t spin_limit;       // 0 = kDefaultSpinLimit
    uint32_t reserved[58];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");

// How one dispatch launch splits work.  Tokens are grouped in look-back
// tiles of `tile_tokens`; each tile is served by `parts` workgroups: every
// workgroup copies `block_tokens` consecutive tokens of the tile, restricted
// to one of `col_splits` equal column ranges of the row.
struct DispatchPlan {
    int tile_tokens;
    int block_tokens;
    int col_splits;
    int parts;
    int tiles;
    int blocks;
};

struct CombinePlan {
    int col_splits;
    int blocks;
};

struct WsPlan {
    int layout_blocks;
    size_t partial_offset;   // int32 [layout_blocks][E + G]
    size_t lookback_offset;  // uint64 [tiles][E]
    size_t total;
};

DispatchPlan plan_dispatch(const moedisp_shape& s);
CombinePlan plan_combine(const moedisp_shape& s);
WsPlan plan_workspace(const moedisp_shape& s);

inline size_t row_bytes(const moedisp_shape& s) {
    return (size_t)s.hidden * (s.x_dtype == MOEDISP_FP8_E4M3 ? 1 : 2);
}
inline int scales_per_row(const moedisp_shape& s) {
    return s.x_dtype == MOEDISP_FP8_E4M3 ? s.hidden / s.scale_block : 0;
}

struct LayoutArgs {
    int T, k, E, G;
    const int32_t* topk_idx;
    int32_t* tokens_per_expert;
    int32_t* tokens_per_group;
    uint32_t* is_token_in_group;
    WsHeader* hdr;
    int32_t* partials;
    int blocks;
};

struct DispatchArgs {
    int T, k, E;
    int row16;         // 16-byte units per row
    int scale_words;   // fp32 scales per row (0 without scales)
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
    WsHeader* hdr;
    uint64_t* lookback;
};

struct CombineArgs {
    int T, k;
    int row16;
    int capacity;
    int col_splits;
    const v4u* expert_out;
    const int32_t* recv_src_idx;
    const float* recv_weights;
    const int32_t* slot_to_row;
    void* out;
    WsHeader* hdr;
};

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream);
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, bool f32_out, hipStream_t stream);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_set_word(uint32_t* p, uint32_t value, hipStream_t stream);
hipError_t launch_copy(v4u* dst, const v4u* src, size_t n16, hipStream_t stream);

}  // namespace moedisp
