// Dispatch: per-tile expert counts (count kernel), then receive rows and the
// row scatter (scatter kernel).
//
// What is computed ("MSCCLPP EP implementation - #852": PR description,
// "Scope", intranode dispatch; commit message fixing internode combine for the
// receiver-side bookkeeping that combine later consumes): every routed slot
// (t,j) with expert e gets the receive row
//     expert_offsets[e] + #{t' < t : token t' routes to e},
// so each expert's rows are contiguous and in token order, and the token's row
// bytes are copied there.  Rows move in 16-byte units (the page's warp-geometry
// commits and code-scanning excerpt count hidden rows in int4 units).
//
// The device-wide scan is a reduce-then-scan split across the two kernels,
// with the kernel boundary as its only synchronisation:
//  - count kernel, one workgroup per tile of `tile_tokens` tokens: counts the
//    tile's slots per expert in LDS and stores them expert-major (one
//    expert's counts over the tiles are contiguous).  Tile 0 also stores
//    expert_offsets, the exclusive scan of tokens_per_expert.
//  - scatter kernel, one workgroup per `block_tokens` tokens (and column
//    range): for each of its slots with expert e, the row is
//      expert_offsets[e] + (counts of e in the earlier tiles, summed by
//      several lanes with 16-byte loads from the L2-resident count table)
//      + (the number of earlier slots of its own tile with expert e, counted
//      from an LDS copy of the tile's routing).
//    Every workgroup does this small prefix sum for itself, so no workgroup
//    ever waits for another: on a multi-XCD part a cross-workgroup wait (a
//    chained or decoupled look-back) costs a cross-XCD round trip per hop,
//    and while the copy saturates HBM those polls queue behind the stores.
//    No atomics decide any order, so the result is deterministic.
// The scatter then streams: each lane loads U 16-byte units of the source row
// (U = 1 by default, up to 1024 lanes per workgroup) once - the first pass is
// issued before the row computation - and stores them,
// non-temporally, to each of the token's k destination rows.  Workgroups of
// column range 0 write the handle (slot_to_row, recv_src_idx, recv_weights)
// and fp8 scales.  Rows outside their expert's segment (or the buffer) are not
// written and raise BAD_LAYOUT; workgroup 0 also checks that the routed slots
// add up to the sum of tokens_per_expert.
#include "moedisp_internal.h"

namespace moedisp {
namespace {

// Exclusive scan of in[0..n) into out (LDS), by the whole workgroup.  Returns
// the total; sets *bad if an entry is negative.
__device__ long long block_exclusive_scan(const int32_t* __restrict__ in, int n, int32_t* out,
                                          long long* s_wave, bool* bad) {
    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int per = (n + nth - 1) / nth;
    const int lo = min(n, tid * per);
    const int hi = min(n, lo + per);
    long long sum = 0;
    for (int i = lo; i < hi; ++i) {
        const int v = in[i];
        if (v < 0) *bad = true;
        sum += v;
    }
    long long incl = sum;
    for (int d = 1; d < 64; d <<= 1) {
        const long long o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    long long run = incl - sum;
    long long total = 0;
    for (int w = 0; w < nth / 64; ++w) {
        if (w < wave) run += s_wave[w];
        total += s_wave[w];
    }
    for (int i = lo; i < hi; ++i) {
        out[i] = (int32_t)run;
        run += in[i];
    }
    __syncthreads();
    return total;
}

__global__ __launch_bounds__(kThreads) void moedisp_count(DispatchArgs a) {
    const DispatchPlan& P = a.plan;
    extern __shared__ int32_t dyn[];  // hist[E]
    int32_t* s_hist = dyn;
    __shared__ long long s_wave[kThreads / 64];
    __shared__ uint32_t s_err;
    const int tid = threadIdx.x;
    const int k = a.k;
    const int E = a.E;
    const int tile = blockIdx.x;
    const int tile_t0 = tile * P.tile_tokens;
    const int tile_slots = max(0, min(P.tile_tokens, a.T - tile_t0)) * k;

    for (int e = tid; e < E; e += kThreads) s_hist[e] = 0;
    if (tid == 0) s_err = 0;
    __syncthreads();
    uint32_t err = 0;
    for (int s = tid; s < tile_slots; s += kThreads) {
        const int id = a.topk_idx[(size_t)tile_t0 * k + s];
        if (id >= 0 && id < E)
            atomicAdd(&s_hist[id], 1);
        else if (id != -1)
            err |= MOEDISP_DEV_BAD_EXPERT_ID;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) a.tile_counts[(size_t)e * P.tile_stride + tile] = s_hist[e];
    if (tile == 0) {
        __syncthreads();  // s_hist is reused as the scan output
        bool bad = false;
        const long long total = block_exclusive_scan(a.tokens_per_expert, E, s_hist, s_wave, &bad);
        if (bad || total > a.capacity) err |= MOEDISP_DEV_BAD_LAYOUT;
        for (int e = tid; e < E; e += kThreads) a.expert_offsets[e] = s_hist[e];
        if (tid == 0) a.expert_offsets[E] = (int32_t)total;
    }
    if (err) atomicOr(&s_err, err);
    __syncthreads();
    if (tid == 0 && s_err) atomicOr(&a.hdr->status, s_err);
}

// U: 16-byte units per lane per pass.
template <int U>
__global__ __launch_bounds__(kMaxDispatchThreads) void moedisp_scatter(DispatchArgs a) {
    const DispatchPlan& P = a.plan;
    extern __shared__ int32_t dyn[];  // routing of the tile up to this workgroup's last slot
    int32_t* s_ids = dyn;
    __shared__ int32_t s_pre[kMaxBlockSlots];   // counts of the slot's expert in earlier tiles
    __shared__ int32_t s_base[kMaxBlockSlots];  // expert_offsets[e]
    __shared__ int32_t s_len[kMaxBlockSlots];   // tokens_per_expert[e]
    __shared__ int32_t s_rows[kMaxBlockSlots];
    __shared__ int32_t s_routed;
    __shared__ uint32_t s_err;

    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const int k = a.k;
    const int E = a.E;
    const int tok = blockIdx.x / P.col_splits;
    const int split = blockIdx.x - tok * P.col_splits;
    const int blk_t0 = tok * P.block_tokens;
    const int blk_nt = max(0, min(P.block_tokens, a.T - blk_t0));
    const int blk_slots = blk_nt * k;
    const int tile = blk_t0 / P.tile_tokens;  // tile_tokens is a multiple of block_tokens
    const int tile_t0 = tile * P.tile_tokens;
    const int first = (blk_t0 - tile_t0) * k;  // slots of the tile before this workgroup's
    const int per_split = (a.row16 + P.col_splits - 1) / P.col_splits;
    const int c0 = split * per_split;
    const int c1 = min(a.row16, c0 + per_split);

    // first pass of source units: independent of the rows, so issued first
    v4u pre[U];
    if (blk_nt > 0) {
        const v4u* src = a.x + (size_t)blk_t0 * a.row16;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cc = c0 + tid + u * nth;
            if (cc < c1) pre[u] = src[cc];
        }
    }
    for (int i = tid; i < first + blk_slots; i += nth) {
        const int id = a.topk_idx[(size_t)tile_t0 * k + i];
        s_ids[i] = (id >= 0 && id < E) ? id : -1;
    }
    for (int q = tid; q < blk_slots; q += nth) s_pre[q] = 0;
    if (tid == 0) {
        s_routed = 0;
        s_err = 0;
    }
    __syncthreads();

    // counts of each slot's expert in the earlier tiles: L lanes per slot,
    // 16-byte loads of the expert's contiguous count column
    if (blk_slots > 0) {
        const int L = nth / blk_slots;  // >= 1: the plan keeps blk_slots <= threads
        if (tid < L * blk_slots) {
            const int q = tid / L;
            const int l = tid - q * L;
            const int e = s_ids[first + q];
            if (e >= 0) {
                const int32_t* col = a.tile_counts + (size_t)e * P.tile_stride;  // 16-byte aligned
                const int n4 = tile >> 2;
                int32_t sum = 0;
                for (int c = l; c < n4; c += 4 * L) {
                    int4 v[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        v[u] = (c + u * L < n4) ? reinterpret_cast<const int4*>(col)[c + u * L] : make_int4(0, 0, 0, 0);
#pragma unroll
                    for (int u = 0; u < 4; ++u) sum += v[u].x + v[u].y + v[u].z + v[u].w;
                }
                if (l == 0) {
                    for (int j = n4 * 4; j < tile; ++j) sum += col[j];
                    s_base[q] = a.expert_offsets[e];
                    s_len[q] = a.tokens_per_expert[e];
                }
                if (sum) atomicAdd(&s_pre[q], sum);
            }
        }
    }
    __syncthreads();

    // rows of this workgroup's slots
    uint32_t err = 0;
    for (int q = tid; q < blk_slots; q += nth) {
        const int s = first + q;
        const int e = s_ids[s];
        int row = -1;
        if (e >= 0) {
            int before = 0;
            for (int u = 0; u < s; ++u) before += s_ids[u] == e;
            const long long base = s_base[q];
            const long long r = base + s_pre[q] + before;
            if (r < 0 || r < base || r >= base + s_len[q] || r >= a.capacity)
                err |= MOEDISP_DEV_BAD_LAYOUT;
            else
                row = (int)r;
        }
        s_rows[q] = row;
    }
    __syncthreads();

    // handle: slot -> row, row -> source token and weight, fp8 scales
    if (split == 0) {
        for (int q = tid; q < blk_slots; q += nth) {
            const size_t slot = (size_t)blk_t0 * k + q;
            const int row = s_rows[q];
            a.slot_to_row[slot] = row;
            if (row >= 0) {
                a.recv_src_idx[row] = blk_t0 + q / k;
                a.recv_weights[row] = a.topk_weights[slot];
            }
        }
        if (a.scale_words) {
            const int n = blk_slots * a.scale_words;
            for (int i = tid; i < n; i += nth) {
                const int q = i / a.scale_words;
                const int c = i - q * a.scale_words;
                const int row = s_rows[q];
                if (row >= 0)
                    a.recv_scales[(size_t)row * a.scale_words + c] =
                        a.x_scales[(size_t)(blk_t0 + q / k) * a.scale_words + c];
            }
        }
    }

    // row scatter: each 16-byte unit is loaded once and stored k times
    for (int tt = 0; tt < blk_nt; ++tt) {
        const v4u* src = a.x + (size_t)(blk_t0 + tt) * a.row16;
        const int32_t* rows = s_rows + tt * k;
        for (int c = c0 + tid; c < c1; c += U * nth) {
            v4u v[U];
            if (tt == 0 && c == c0 + tid) {
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = pre[u];
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int cc = c + u * nth;
                    if (cc < c1) v[u] = src[cc];
                }
            }
            for (int j = 0; j < k; ++j) {
                const int r = rows[j];
                if (r < 0) continue;
                v4u* dst = a.recv_x + (size_t)r * a.row16;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int cc = c + u * nth;
                    if (cc < c1) __builtin_nontemporal_store(v[u], dst + cc);
                }
            }
        }
    }

    // workgroup 0: the routed slots must add up to the layout's total
    if (blockIdx.x == 0) {
        const int n = a.T * k;
        int32_t routed = 0;
        for (int i0 = tid; i0 < n; i0 += 8 * nth) {
            int32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = (i0 + u * nth < n) ? a.topk_idx[i0 + u * nth] : -1;
#pragma unroll
            for (int u = 0; u < 8; ++u) routed += (v[u] >= 0 && v[u] < E);
        }
        if (routed) atomicAdd(&s_routed, routed);
        __syncthreads();
        if (tid == 0 && s_routed != a.expert_offsets[E]) err |= MOEDISP_DEV_BAD_LAYOUT;
    }
    if (err) atomicOr(&s_err, err);
    __syncthreads();
    if (tid == 0 && s_err) atomicOr(&a.hdr->status, s_err);
}

}  // namespace

hipError_t launch_dispatch_notify(const DispatchArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(moedisp_count, dim3(a.plan.tiles), dim3(kThreads), (size_t)a.E * sizeof(int32_t), stream, a);
    return hipGetLastError();
}

hipError_t launch_dispatch_scatter(const DispatchArgs& a, hipStream_t stream) {
    const DispatchPlan& p = a.plan;
    const size_t lds = (size_t)p.tile_tokens * a.k * sizeof(int32_t);
    const dim3 grid(p.blocks), block(p.threads);
    switch (p.units_per_lane) {
        case 1: hipLaunchKernelGGL((moedisp_scatter<1>), grid, block, lds, stream, a); break;
        case 2: hipLaunchKernelGGL((moedisp_scatter<2>), grid, block, lds, stream, a); break;
        default: hipLaunchKernelGGL((moedisp_scatter<4>), grid, block, lds, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace moedisp
