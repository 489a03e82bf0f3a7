// Layout kernel: tokens per expert, tokens per group and the token-in-group
// bitmap ("counts + token-in-rank" of the high-throughput layout kernel on the
// "MSCCLPP EP implementation - #852" page, review file table).
//
// One lane per routing slot: a workgroup of kLayoutThreads lanes covers
// kLayoutThreads / k whole tokens, so at T = 4096, k = 8 the grid has 32
// workgroups of 16 waves and every wave handles the 64 slots of 8 tokens at
// once.  Each lane loads its slot's expert id (coalesced) and:
//   - expert counts: the lanes of a wave with the same expert find each other
//     with one ballot per bit of the expert id, and only the lowest such lane
//     adds the popcount of its peer mask to an LDS-private histogram - one LDS
//     atomic per distinct expert per wave;
//   - token masks: an LDS atomicOr of the slot's group bit into its token's
//     word; repeated experts: a comparison with the token's earlier slots
//     (LDS copy of the ids, 8 reads in flight);
// then each token's mask is the bitmap word and group counts are popcounts of
// one ballot per group.  Each workgroup writes its partial counts to the
// workspace, and a second, one-workgroup kernel sums them in workgroup order:
// the kernel boundary is the only synchronisation.  (A last-workgroup finish
// inside one kernel needs a device-scope fence and a same-address atomic per
// workgroup; measured on this part, those serialise across the XCDs and cost
// more than the second launch.)
//
// With the dispatch's notify phase folded in (ep_get_dispatch_layout_notify),
// each workgroup also counts its slots per (dispatch tile, expert): the lanes
// of one tile are a contiguous range of the wave, so the expert peer mask
// restricted to that range gives the tile count with no further ballots; the
// counts are stored expert-major as the count kernel would, and the reduce
// kernel also writes expert_offsets, the exclusive scan of the totals.
#include "moedisp_internal.h"

namespace moedisp {
namespace {

// Lanes among `active` whose key equals this lane's key (keys < 2^nbits,
// nbits <= 12).  Every lane of the wave must execute this (it issues nbits
// ballots).
__device__ inline uint64_t match_peers(uint32_t key, int nbits, uint64_t active) {
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
__device__ inline uint32_t div_const(uint32_t x, int shift, uint32_t magic) {
    return shift >= 0 ? x >> shift : __umulhi(x, magic);
}

__global__ __launch_bounds__(kLayoutThreads) void moedisp_layout(LayoutArgs a) {
    // LDS: counts [E + G], ids [tokens * k], token masks [tokens], and with
    // the notify phase tile counts [tiles per workgroup][E]
    extern __shared__ int32_t dyn[];
    const int EG = a.E + a.G;
    const int k = a.k;
    const int tpb = a.tokens_per_block;
    int32_t* s_cnt = dyn;
    int32_t* s_ids = dyn + EG;
    uint32_t* s_mask = reinterpret_cast<uint32_t*>(s_ids + tpb * k);
    int32_t* s_tile = reinterpret_cast<int32_t*>(s_mask + tpb);
    const int tpw = a.tile_counts ? (tpb >> a.tile_shift) : 0;  // tiles per workgroup
    __shared__ uint32_t s_err;

    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const int lane = tid & 63;
    const int t0 = blockIdx.x * tpb;
    const int nt = max(0, min(tpb, a.T - t0));
    const int ns = nt * k;

    // this lane's slot (coalesced), validated
    uint32_t err = 0;
    int id = -1;
    if (tid < ns) {
        id = a.topk_idx[(size_t)t0 * k + tid];
        if (id < -1 || id >= a.E) {
            err |= MOEDISP_DEV_BAD_EXPERT_ID;
            id = -1;
        }
    }
    for (int i = tid; i < EG; i += nth) s_cnt[i] = 0;
    for (int i = tid; i < nt; i += nth) s_mask[i] = 0;
    for (int i = tid; i < tpw * a.E; i += nth) s_tile[i] = 0;
    if (tid < ns) s_ids[tid] = id;
    if (tid == 0) s_err = 0;
    __syncthreads();

    // expert counts: one ballot-match round per wave
    const bool routed = id >= 0;
    const uint64_t below = (1ull << lane) - 1ull;
    const uint64_t active = __ballot(routed);
    const uint64_t peers = match_peers(routed ? (uint32_t)id : 0u, a.id_bits, active);
    if (routed && (peers & below) == 0) atomicAdd(&s_cnt[id], (int32_t)__popcll(peers));
    // tile counts: the peers whose slots lie in this lane's tile (slots
    // [tile * 2^tile_shift * k, (tile + 1) * 2^tile_shift * k) of the
    // workgroup, a contiguous lane range of the wave)
    if (tpw > 0 && routed) {
        const int tile = (int)div_const((uint32_t)tid, a.k_shift, a.k_magic) >> a.tile_shift;
        const int span = (k << a.tile_shift);
        const int w0 = tid - lane;
        const int lo = max(tile * span - w0, 0);
        const int hi = min((tile + 1) * span - w0, 64);
        const uint64_t range = (hi >= 64 ? ~0ull : ((1ull << hi) - 1ull)) & ~((1ull << lo) - 1ull);
        const uint64_t tp = peers & range;
        if ((tp & below) == 0) atomicAdd(&s_tile[tile * a.E + id], (int32_t)__popcll(tp));
    }
    // token masks and repeated experts
    if (routed) {
        const int tl = (int)div_const((uint32_t)tid, a.k_shift, a.k_magic);
        const int base = tl * k;
        atomicOr(&s_mask[tl], 1u << div_const((uint32_t)id, a.pg_shift, a.pg_magic));
        for (int u0 = base; u0 < tid; u0 += 8) {  // 8 clamped reads per step, no branch
            int v[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) v[m] = s_ids[min(u0 + m, tid - 1)];
#pragma unroll
            for (int m = 0; m < 8; ++m)
                if (u0 + m < tid && v[m] == id) err |= MOEDISP_DEV_DUPLICATE_EXPERT;
        }
    }
    __syncthreads();

    // bitmap and group counts (one ballot per group and wave)
    const uint32_t mask = tid < nt ? s_mask[tid] : 0u;  // nt <= tpb <= threads
    if (tid < nt) a.is_token_in_group[t0 + tid] = mask;
    for (int g = 0; g < a.G; ++g) {
        const uint64_t in_g = __ballot((mask >> g) & 1u);
        if (lane == 0 && in_g) atomicAdd(&s_cnt[a.E + g], (int32_t)__popcll(in_g));
    }
    if (err) atomicOr(&s_err, err);
    __syncthreads();

    int32_t* mine = a.partials + (size_t)blockIdx.x * EG;
    for (int i = tid; i < EG; i += nth) mine[i] = s_cnt[i];
    if (tpw > 0) {  // expert-major, this workgroup's tiles contiguous per expert
        const int tile0 = blockIdx.x * tpw;
        const int ntl = min(tpw, a.tiles - tile0);
        for (int i = tid; i < a.E * ntl; i += nth) {
            const int e = i / ntl;
            const int q = i - e * ntl;
            a.tile_counts[(size_t)e * a.tile_stride + tile0 + q] = s_tile[q * a.E + e];
        }
    }
    if (tid == 0 && s_err) atomicOr(&a.hdr->status, s_err);
}

// Sum of the partial counts in workgroup order (one workgroup; the kernel
// boundary orders it after every partial), 32 independent loads in flight:
// one round trip for up to 32 partial rows.
__global__ __launch_bounds__(kThreads) void moedisp_layout_reduce(LayoutArgs a) {
    __shared__ int32_t s_tot[kMaxExperts];  // expert totals, for expert_offsets
    __shared__ int32_t s_wave[kThreads / 64];
    const int EG = a.E + a.G;
    constexpr int kBatch = 32;
    for (int i = threadIdx.x; i < EG; i += kThreads) {
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
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (a.E + kThreads - 1) / kThreads;
    const int lo = min(a.E, tid * per), hi = min(a.E, lo + per);
    int32_t run = 0;
    for (int i = lo; i < hi; ++i) run += s_tot[i];
    int32_t incl = run;
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int32_t off = incl - run, total = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
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

}  // namespace

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream) {
    const size_t lds = layout_lds_bytes(a.E, a.G, a.k, a.tokens_per_block,
                                        a.tile_counts ? (a.tokens_per_block >> a.tile_shift) : 0);
    if (!grid_fits(a.blocks, kLayoutThreads)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(moedisp_layout, dim3(a.blocks), dim3(kLayoutThreads), lds, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moedisp_layout_reduce, dim3(1), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace moedisp
