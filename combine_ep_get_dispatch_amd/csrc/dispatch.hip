// Dispatch kernel: row offsets by a single-pass scan with decoupled look-back,
// fused with the row scatter.
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
// How.  Tokens form look-back tiles of `tile_tokens`.  Workgroups take a ticket
// from a workspace counter when they start, so a ticket's predecessors are
// already running; ticket -> (tile, part).  Part 0 of each tile ("publisher")
// builds the tile's per-expert histogram in LDS, publishes it as an aggregate
// word per expert, walks back over predecessor tiles (eight words per poll)
// until it meets an inclusive prefix, and publishes its own inclusive prefix.
// Tile 0 seeds the chain with the exclusive scan of tokens_per_expert, so
// every published prefix already includes the expert's base offset.  The other
// parts of a tile wait for that tile's prefix of the experts they need.  Within
// a tile, a slot's rank is the number of earlier slots in the tile with the
// same expert, counted from the LDS copy of the tile's routing: no atomics
// decide any order, so the result is deterministic.
//
// Each workgroup then copies its tokens: every lane loads U 16-byte units of
// the source row once and stores them to each of the token's k destination
// rows (one load, k coalesced stores per unit).  Look-back words carry the
// call's epoch so words left by earlier calls read as "not ready"; the last
// workgroup to finish advances the epoch and resets the ticket counters.
// Every wait is bounded; a wait that gives up raises SPIN_TIMEOUT and the
// workgroup continues, so the grid always drains.
#include "moedisp_internal.h"

namespace moedisp {
namespace {

constexpr int kLookWindow = 8;

__device__ inline uint64_t pack_word(uint32_t epoch, uint32_t flag, uint32_t value) {
    return ((uint64_t)epoch << 32) | ((uint64_t)flag << 30) | (uint64_t)(value & kValueMask);
}
__device__ inline uint32_t word_epoch(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ inline uint32_t word_flag(uint64_t w) { return (uint32_t)(w >> 30) & 3u; }
__device__ inline uint32_t word_value(uint64_t w) { return (uint32_t)w & kValueMask; }

__device__ inline uint64_t load_word(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void store_word(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive scan of in[0..n) into out (LDS), by the whole workgroup.  Returns
// the total; sets *bad if an entry is negative.
__device__ long long block_exclusive_scan(const int32_t* __restrict__ in, int n, int32_t* out,
                                          long long* s_wave, bool* bad) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int per = (n + kThreads - 1) / kThreads;
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
    for (int w = 0; w < kThreads / 64; ++w) {
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

template <bool kNT>
__device__ inline void store16(v4u* p, v4u v) {
    if constexpr (kNT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

template <int U, bool kNT>
__global__ __launch_bounds__(kThreads) void moedisp_dispatch(DispatchArgs a) {
    extern __shared__ int32_t dyn[];  // hist[E], excl[E], off[E]
    int32_t* s_hist = dyn;
    int32_t* s_excl = dyn + a.E;
    int32_t* s_off = dyn + 2 * a.E;
    __shared__ int32_t s_ids[kMaxTileTokens * kMaxTopk];
    __shared__ int32_t s_rows[kMaxBlockTokens * kMaxTopk];
    __shared__ long long s_wave[kThreads / 64];
    __shared__ uint32_t s_ticket, s_epoch, s_limit, s_err;

    const int tid = threadIdx.x;
    const int k = a.k;
    const int E = a.E;
    const DispatchPlan& P = a.plan;

    if (tid == 0) {
        s_ticket = atomicAdd(&a.hdr->dispatch_ticket, 1u);
        s_epoch = __hip_atomic_load(&a.hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
        const uint32_t lim = __hip_atomic_load(&a.hdr->spin_limit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_limit = lim ? lim : kDefaultSpinLimit;
        s_err = 0;
    }
    __syncthreads();
    const uint32_t ticket = s_ticket;
    const uint32_t epoch = s_epoch;
    const uint32_t limit = s_limit;
    if (ticket >= (uint32_t)a.plan.blocks) {
        // counters left by an overlapping call on this workspace: touch nothing
        if (tid == 0) atomicOr(&a.hdr->status, MOEDISP_DEV_WORKSPACE_RACE);
        return;
    }
    const int tile = (int)(ticket / (uint32_t)P.parts);
    const int part = (int)(ticket % (uint32_t)P.parts);
    const int split = part % P.col_splits;
    const int tile_t0 = tile * P.tile_tokens;
    const int tile_nt = max(0, min(P.tile_tokens, a.T - tile_t0));
    const int tile_slots = tile_nt * k;
    const int blk_t0 = tile_t0 + (part / P.col_splits) * P.block_tokens;
    const int blk_nt = max(0, min(P.block_tokens, a.T - blk_t0));
    const int blk_slots = blk_nt * k;
    const bool publisher = part == 0;
    uint32_t err = 0;

    // routing of the whole tile -> LDS; ids outside {-1} U [0,E) become -1
    for (int s = tid; s < tile_slots; s += kThreads) {
        int id = a.topk_idx[(size_t)tile_t0 * k + s];
        if (id < -1 || id >= E) {
            err |= MOEDISP_DEV_BAD_EXPERT_ID;
            id = -1;
        }
        s_ids[s] = id;
    }
    if (publisher)
        for (int e = tid; e < E; e += kThreads) s_hist[e] = 0;
    __syncthreads();

    if (publisher) {
        for (int s = tid; s < tile_slots; s += kThreads) {
            const int id = s_ids[s];
            if (id >= 0) atomicAdd(&s_hist[id], 1);
        }
        __syncthreads();
        uint64_t* mine = a.lookback + (size_t)tile * E;
        if (tile == 0) {
            bool bad = false;
            const long long total = block_exclusive_scan(a.tokens_per_expert, E, s_excl, s_wave, &bad);
            if (bad || total > a.capacity) err |= MOEDISP_DEV_BAD_LAYOUT;
            for (int e = tid; e < E; e += kThreads) {
                store_word(mine + e, pack_word(epoch, kFlagPrefix, (uint32_t)(s_excl[e] + s_hist[e])));
                a.expert_offsets[e] = s_excl[e];
            }
            if (tid == 0) a.expert_offsets[E] = (int32_t)total;
        } else {
            for (int e = tid; e < E; e += kThreads)
                store_word(mine + e, pack_word(epoch, kFlagAggregate, (uint32_t)s_hist[e]));
            for (int e = tid; e < E; e += kThreads) {
                uint32_t acc = 0;
                int j = tile - 1;
                uint32_t polls = 0;
                while (true) {
                    uint64_t w[kLookWindow];
#pragma unroll
                    for (int q = 0; q < kLookWindow; ++q)
                        w[q] = (j - q >= 0) ? load_word(a.lookback + (size_t)(j - q) * E + e) : 0ull;
                    int q = 0;
                    bool done = false;
                    for (; q < kLookWindow && j - q >= 0; ++q) {
                        if (word_epoch(w[q]) != epoch || word_flag(w[q]) == 0u) break;
                        acc += word_value(w[q]);
                        if (word_flag(w[q]) == kFlagPrefix) {
                            done = true;
                            break;
                        }
                    }
                    if (done) break;
                    j -= q;
                    if (j < 0) {  // tile 0 always publishes a prefix; cannot happen
                        err |= MOEDISP_DEV_BAD_LAYOUT;
                        break;
                    }
                    if (q == 0) {
                        if (++polls > limit) {
                            err |= MOEDISP_DEV_SPIN_TIMEOUT;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
                s_excl[e] = (int32_t)acc;
                store_word(mine + e, pack_word(epoch, kFlagPrefix, acc + (uint32_t)s_hist[e]));
            }
        }
        if (tile == P.tiles - 1) {
            // the last tile's inclusive prefix must land on expert_offsets[e+1]
            bool bad = false;
            block_exclusive_scan(a.tokens_per_expert, E, s_off, s_wave, &bad);
            for (int e = tid; e < E; e += kThreads)
                if ((long long)s_excl[e] + s_hist[e] != (long long)s_off[e] + a.tokens_per_expert[e])
                    err |= MOEDISP_DEV_BAD_LAYOUT;
        }
        __syncthreads();
    }

    // rows of this workgroup's slots
    for (int q = tid; q < blk_slots; q += kThreads) {
        const int s = (blk_t0 - tile_t0) * k + q;  // slot within the tile
        const int e = s_ids[s];
        int row = -1;
        if (e >= 0) {
            int before = 0, in_tile = 0;
            for (int u = 0; u < tile_slots; ++u) {
                const int v = s_ids[u];
                in_tile += v == e;
                before += (v == e) & (u < s);
            }
            long long base;
            if (publisher) {
                base = s_excl[e];
            } else {
                const uint64_t* p = a.lookback + (size_t)tile * E + e;
                uint32_t polls = 0;
                uint64_t w = load_word(p);
                while (word_epoch(w) != epoch || word_flag(w) != kFlagPrefix) {
                    if (++polls > limit) {
                        err |= MOEDISP_DEV_SPIN_TIMEOUT;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                    w = load_word(p);
                }
                base = (long long)word_value(w) - in_tile;
            }
            const long long r = base + before;
            if (r < 0 || r >= a.capacity)
                err |= MOEDISP_DEV_BAD_LAYOUT;
            else
                row = (int)r;
        }
        s_rows[q] = row;
    }
    __syncthreads();

    // handle: slot -> row, row -> source token and weight, fp8 scales
    if (split == 0) {
        for (int q = tid; q < blk_slots; q += kThreads) {
            const int t = blk_t0 + q / k;
            const size_t slot = (size_t)blk_t0 * k + q;
            const int row = s_rows[q];
            a.slot_to_row[slot] = row;
            if (row >= 0) {
                a.recv_src_idx[row] = t;
                a.recv_weights[row] = a.topk_weights[slot];
            }
        }
        if (a.scale_words) {
            const int n = blk_slots * a.scale_words;
            for (int i = tid; i < n; i += kThreads) {
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
    const int per_split = (a.row16 + P.col_splits - 1) / P.col_splits;
    const int c0 = split * per_split;
    const int c1 = min(a.row16, c0 + per_split);
    for (int tt = 0; tt < blk_nt; ++tt) {
        const v4u* src = a.x + (size_t)(blk_t0 + tt) * a.row16;
        const int32_t* rows = s_rows + tt * k;
        for (int c = c0 + tid; c < c1; c += U * kThreads) {
            v4u v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int cc = c + u * kThreads;
                if (cc < c1) v[u] = src[cc];
            }
            for (int j = 0; j < k; ++j) {
                const int r = rows[j];
                if (r < 0) continue;
                v4u* dst = a.recv_x + (size_t)r * a.row16;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int cc = c + u * kThreads;
                    if (cc < c1) store16<kNT>(dst + cc, v[u]);
                }
            }
        }
    }

    if (err) atomicOr(&s_err, err);
    __syncthreads();
    if (tid == 0) {
        if (s_err) atomicOr(&a.hdr->status, s_err);
        __threadfence();
        const uint32_t prev = atomicAdd(&a.hdr->dispatch_done, 1u);
        if (prev == (uint32_t)(P.blocks - 1)) {
            __hip_atomic_store(&a.hdr->epoch, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.hdr->dispatch_ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.hdr->dispatch_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream) {
    const size_t lds = (size_t)3 * a.E * sizeof(int32_t);
    hipLaunchKernelGGL((moedisp_dispatch<4, true>), dim3(a.plan.blocks), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace moedisp
