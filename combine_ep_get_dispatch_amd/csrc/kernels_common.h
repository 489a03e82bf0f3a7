// Device helpers shared by the layout, notify and dispatch kernels of
// libmoedisp (gfx950, wave64).  Every function is static inline, so each
// translation unit that includes this header gets its own copy.
#pragma once

#include "moedisp_internal.h"

namespace moedisp {

// Lanes among `active` whose key equals this lane's key (keys < 2^nbits,
// nbits <= 12).  Every lane of the wave must execute this (it issues nbits
// ballots).
static __device__ inline uint64_t match_peers(uint32_t key, int nbits, uint64_t active) {
    uint64_t peers = active;
#pragma unroll
    for (int b = 0; b < 12; ++b) {
        if (b < nbits) {  // nbits is uniform
            const bool bit = (key >> b) & 1u;
            const uint64_t ones = __ballot(bit);
            peers &= bit ? ones : ~ones;
        }
    }
    return peers;
}

// x / d for a host-computed (shift, magic) pair: a shift when d is a power of
// two, else a multiply-high (exact for the ranges the host checks).
static __device__ inline uint32_t div_const(uint32_t x, int shift, uint32_t magic) {
    return shift >= 0 ? x >> shift : __umulhi(x, magic);
}

// Inclusive scan over the wave with DPP moves (no LDS round trip): sums
// inside each 16-lane row (row_shr 1, 2, 4, 8), then row 0's total into
// rows 1 and 3 and row 1's running total into rows 2 and 3 (row_bcast 15
// and 31).  Lane i gets the sum of lanes 0..i; the wave sum is lane 63's.
// Whole wave, all lanes active.
static __device__ inline int32_t wave_inclusive_scan_dpp(int32_t v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return v;
}

// Sum of v over the 64 lanes of the wave (every lane gets it, in a scalar
// register); whole wave, all lanes active.
static __device__ inline int32_t wave_sum_dpp(int32_t v) {
    return __builtin_amdgcn_readlane(wave_inclusive_scan_dpp(v), 63);
}

// Exclusive scan of in[0..n) (global or LDS) into out (LDS), by the whole
// workgroup (any size that is a multiple of 64, s_wave holding one entry per
// wave).  Returns the total; sets *bad if an entry is negative.  Has barriers.
static __device__ inline long long block_exclusive_scan(const int32_t* in, int n, int32_t* out, long long* s_wave,
                                                 bool* bad) {
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
        const int v = in[i];
        out[i] = (int32_t)run;
        run += v;
    }
    __syncthreads();
    return total;
}

// Expert (or, in group mode, group) of flat slot s = t*k + j, -1 if masked;
// sets BAD_EXPERT_ID in *err for an id outside {-1} U [0,E).
static __device__ inline int slot_id(const DispatchArgs& a, size_t s, uint32_t* err) {
    if (a.bitmap) {
        const size_t t = s / (unsigned)a.k;
        const int g = (int)(s - t * a.k);
        return ((a.bitmap[t] >> g) & 1u) ? g : -1;
    }
    const int id = a.topk_idx[s];
    if (id >= 0 && id < a.E) return id;
    if (id != -1) *err |= MOEDISP_DEV_BAD_EXPERT_ID;
    return -1;
}

// expert_offsets: the exclusive scan of tokens_per_expert, [E] = the total
// (BAD_LAYOUT for a negative count or a total beyond the receive capacity).
// Whole workgroup; s holds E ints.  Returns this lane's status bits.  Has
// barriers.
static __device__ inline uint32_t offsets_scan(const DispatchArgs& a, int32_t* s, long long* s_wave) {
    bool bad = false;
    const long long total = block_exclusive_scan(a.tokens_per_expert, a.E, s, s_wave, &bad);
    for (int e = threadIdx.x; e < a.E; e += blockDim.x) a.expert_offsets[e] = s[e];
    if (threadIdx.x == 0) a.expert_offsets[a.E] = (int32_t)total;
    return (bad || total > a.capacity) ? (uint32_t)MOEDISP_DEV_BAD_LAYOUT : 0u;
}

// One dispatch tile's expert counts, stored expert-major (the push path's
// per-tile table); with `offsets`, tile 0 also writes expert_offsets, the
// exclusive scan of tokens_per_expert.  Whole workgroup (any size that is a
// multiple of 64); s_hist holds E ints, s_wave one entry per wave.  Returns
// this lane's status bits.  Has barriers.
static __device__ inline uint32_t count_tile(const DispatchArgs& a, int tile, bool offsets, int32_t* s_hist,
                                      long long* s_wave) {
    const DispatchPlan& P = a.plan;
    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const int k = a.k;
    const int E = a.E;
    const int tile_t0 = tile * P.tile_tokens;
    const int tile_slots = max(0, min(P.tile_tokens, a.T - tile_t0)) * k;
    for (int e = tid; e < E; e += nth) s_hist[e] = 0;
    __syncthreads();
    uint32_t err = 0;
    for (int s = tid; s < tile_slots; s += nth) {
        const int id = slot_id(a, (size_t)tile_t0 * k + s, &err);
        if (id >= 0) atomicAdd(&s_hist[id], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += nth) a.tile_counts[(size_t)e * P.tile_stride + tile] = s_hist[e];
    if (offsets && tile == 0) {
        __syncthreads();  // s_hist is reused as the scan output
        err |= offsets_scan(a, s_hist, s_wave);
    }
    return err;
}

// Sum of the layout's partial counts in workgroup order (one workgroup; the
// kernel boundary orders it after every partial), 32 independent loads in
// flight per lane: tokens_per_expert, tokens_per_group, and, when
// a.expert_offsets is set, their exclusive scan into expert_offsets.  s_tot
// holds E ints, s_wave one entry per wave.  Has barriers (uniform branches).
static __device__ inline void layout_reduce(const LayoutArgs& a, int32_t* s_tot, int32_t* s_wave) {
    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const int EG = a.E + a.G;
    constexpr int kBatch = 32;
    for (int i = tid; i < EG; i += nth) {
        int32_t sum = 0;
        for (int b0 = 0; b0 < a.blocks; b0 += kBatch) {
            int32_t v[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q)
                v[q] = (b0 + q < a.blocks) ? a.partials[(size_t)(b0 + q) * EG + i] : 0;
#pragma unroll
            for (int q = 0; q < kBatch; ++q) sum += v[q];
        }
        if (i < a.E) {
            a.tokens_per_expert[i] = sum;
            s_tot[i] = sum;
        } else {
            a.tokens_per_group[i - a.E] = sum;
        }
    }
    if (!a.expert_offsets) return;  // uniform
    // expert_offsets: exclusive scan of the totals, a contiguous run per lane
    __syncthreads();
    const int lane = tid & 63, wave = tid >> 6;
    const int per = (a.E + nth - 1) / nth;
    const int lo = min(a.E, tid * per), hi = min(a.E, lo + per);
    int32_t run = 0;
    for (int i = lo; i < hi; ++i) run += s_tot[i];
    const int32_t incl = wave_inclusive_scan_dpp(run);
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int32_t off = incl - run, total = 0;
    for (int w = 0; w < nth / 64; ++w) {
        if (w < wave) off += s_wave[w];
        total += s_wave[w];
    }
    for (int i = lo; i < hi; ++i) {
        a.expert_offsets[i] = off;
        off += s_tot[i];
    }
    if (tid == 0) {
        a.expert_offsets[a.E] = total;
        if (total > a.capacity) atomicOr(&a.hdr->status, (uint32_t)MOEDISP_DEV_BAD_LAYOUT);
    }
}

// Sort of one token block for the block-pull dispatch ("MSCCLPP EP
// implementation - #852": a rank's received rows are ordered by local expert,
// and within an expert by source token).  For block b (tokens [b * tb,
// b * tb + nt)) the routed slots s = t * k + j are listed in (expert, s)
// order - a stable counting sort - followed by the block's masked slots in
// slot order; per-(expert, block) counts, each expert's first list position
// ls_b[e] and the block's routed total are stored beside the list.
//
// A routed slot's position is ls_b[e] plus the number of earlier routed slots
// of the block with the same expert.  With a bitmask per expert of the
// block's tokens that route to it (LDS, built by 64-bit ORs), that number is
// the popcount of the mask below the slot's token.  A token that repeats an
// expert (invalid routing, which the layout reports) breaks that count; the
// OR that finds the token's bit already set flags the block, which then
// counts each slot's earlier same-expert slots one by one instead (slow, but
// the same order).  ls_b is one scan over the experts by
// one wave; a masked slot's position follows the routed ones, from one
// ballot per 64 slots and one scan over those counts.  No atomic decides any
// order (the ORs and the histogram adds commute), so the lists are
// deterministic.  Whole workgroup of kNotifyThreads lanes (16 waves, so that
// the 64-slot chunks of a pass over the slots are whole waves); lds holds
// sort_lds_words(tb, cap_b, E) ints.  Returns this lane's status bits.  Has
// barriers.
constexpr int kNotifyWaves = kNotifyThreads / 64;

// Exclusive scan of v[0..n) in place by one wave (n <= 64 * 64), returning
// the total in every lane.
static __device__ inline int32_t wave_exclusive_scan(int32_t* v, int n) {
    const int lane = threadIdx.x & 63;
    const int per = (n + 63) / 64;
    const int lo = min(n, lane * per), hi = min(n, lo + per);
    int32_t run = 0;
    for (int i = lo; i < hi; ++i) run += v[i];
    const int32_t incl = wave_inclusive_scan_dpp(run);
    int32_t off = incl - run;
    for (int i = lo; i < hi; ++i) {
        const int32_t c = v[i];
        v[i] = off;
        off += c;
    }
    return __builtin_amdgcn_readlane(incl, 63);
}

static __device__ inline uint32_t pull_sort(const DispatchArgs& a, int b, int32_t* lds) {
    const PullPlan& P = a.pull;
    const int tid = threadIdx.x;
    const int nth = blockDim.x;  // kNotifyThreads
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int k = a.k;
    const int E = a.E;
    const int t0 = b * P.tb;
    const int nt = max(0, min(P.tb, a.T - t0));
    const int ns = nt * k;
    const int mw = sort_mask_words(P.tb);
    const int nchunks = (ns + 63) / 64;
    // 64-bit LDS ORs need 8-byte alignment, which the caller's area (a
    // dynamic LDS array that may sit after 4-byte static variables) does
    // not promise: skip one word where it starts at 4 mod 8
    lds += (reinterpret_cast<uintptr_t>(lds) >> 2) & 1;
    uint64_t* s_mask = reinterpret_cast<uint64_t*>(lds);       // [E][mw]
    int32_t* s_id = lds + 2 * E * mw;                           // [cap_b]
    int32_t* s_cnt = s_id + P.cap_b;                             // [E]: counts, then ls_b
    int32_t* s_mc = s_cnt + E;                                   // [cap_b / 64 + 1]: masked per chunk
    int32_t* s_total = s_mc + P.cap_b / 64 + 1;                  // routed total
    int32_t* s_rep = s_total + 1;                                // a token repeats an expert
    const size_t slot0 = (size_t)t0 * k;
    const uint64_t below = (1ull << lane) - 1ull;

    // stage the block's ids (invalid ids become masked slots); clear tables
    uint32_t err = 0;
    for (int i = tid; i < ns; i += nth) {
        int id = a.topk_idx[slot0 + i];
        if (id < -1 || id >= E) {
            err |= MOEDISP_DEV_BAD_EXPERT_ID;
            id = -1;
        }
        s_id[i] = id;
    }
    for (int i = tid; i < E * mw; i += nth) s_mask[i] = 0ull;
    for (int e = tid; e < E; e += nth) s_cnt[e] = 0;
    if (tid == 0) *s_rep = 0;
    __syncthreads();

    // expert counts and token masks; masked slots per 64-slot chunk (chunk
    // c = i / 64 is one whole wave of one pass)
    for (int base = 0; base < ns; base += nth) {
        const int i = base + tid;
        const bool valid = i < ns;
        const int e = valid ? s_id[i] : -1;
        if (e >= 0) {
            const int t = i / k;
            atomicAdd(&s_cnt[e], 1);
            // the token's bit already set: it repeats the expert
            const unsigned long long bit = 1ull << (t & 63);
            if (atomicOr(reinterpret_cast<unsigned long long*>(&s_mask[e * mw + (t >> 6)]), bit) & bit) *s_rep = 1;
        }
        const uint64_t masked = __ballot(valid && e < 0);
        if (lane == 0 && base + wave * 64 < ns) s_mc[(base >> 6) + wave] = (int32_t)__popcll(masked);
    }
    __syncthreads();

    // wave 0: per-block counts out, ls_b = exclusive scan of the counts;
    // wave 1: exclusive scan of the masked counts over the chunks
    if (wave == 0) {
        for (int e = lane; e < E; e += 64) a.pull_cnt[(size_t)e * P.cnt_stride + b] = s_cnt[e];
        const int32_t total = wave_exclusive_scan(s_cnt, E);
        for (int e = lane; e < E; e += 64) a.pull_ls[(size_t)b * E + e] = s_cnt[e];
        if (lane == 0) {
            a.pull_n[b] = total;
            *s_total = total;
        }
    } else if (wave == 1) {
        wave_exclusive_scan(s_mc, nchunks);
    }
    __syncthreads();

    // place every slot at its list position
    PullEnt* list = a.pull_ent + (size_t)b * P.cap_b;
    const int routed_total = *s_total;
    const bool repeats = *s_rep != 0;
    for (int base = 0; base < ns; base += nth) {
        const int i = base + tid;
        const bool valid = i < ns;
        const int e = valid ? s_id[i] : -1;
        const uint64_t masked = __ballot(valid && e < 0);
        if (!valid) continue;
        PullEnt en;
        en.slot = (int32_t)(slot0 + i);
        if (e < 0 && P.compact) {  // compact lists: the masked slot's handle here
            a.slot_to_row[en.slot] = -1;
            continue;
        }
        int pos;
        if (e >= 0) {
            int r = 0;
            if (!repeats) {
                const int t = i / k;
                const uint64_t* m = s_mask + e * mw;
                r = (int)__popcll(m[t >> 6] & ((1ull << (t & 63)) - 1ull));
                for (int w = 0; w < (t >> 6); ++w) r += (int)__popcll(m[w]);
            } else {
                for (int q = 0; q < i; ++q) r += s_id[q] == e ? 1 : 0;
            }
            en.expert = e;
            pos = s_cnt[e] + r;
        } else {
            en.expert = -1;
            pos = routed_total + s_mc[i >> 6] + (int)__popcll(masked & below);
        }
        list[pos] = en;
    }
    return err;
}

}  // namespace moedisp
