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
#include "kernels_common.h"

namespace moedisp {
namespace {

// One layout workgroup (index wg) of kLayoutThreads lanes.  LDS (dyn):
// counts [E + G], ids [tokens * k], token masks [tokens], and with the
// notify phase tile counts [tiles per workgroup][E]; s_err one word.
static __device__ void layout_body(const LayoutArgs& a, int wg, int32_t* dyn, uint32_t& s_err) {
    const int EG = a.E + a.G;
    const int k = a.k;
    const int tpb = a.tokens_per_block;
    int32_t* s_cnt = dyn;
    int32_t* s_ids = dyn + EG;
    uint32_t* s_mask = reinterpret_cast<uint32_t*>(s_ids + tpb * k);
    int32_t* s_tile = reinterpret_cast<int32_t*>(s_mask + tpb);
    const int tpw = a.tile_counts ? (tpb >> a.tile_shift) : 0;  // tiles per workgroup

    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const int lane = tid & 63;
    const int t0 = wg * tpb;
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

    int32_t* mine = a.partials + (size_t)wg * EG;
    for (int i = tid; i < EG; i += nth) mine[i] = s_cnt[i];
    if (tpw > 0) {  // expert-major, this workgroup's tiles contiguous per expert
        const int tile0 = wg * tpw;
        const int ntl = min(tpw, a.tiles - tile0);
        for (int i = tid; i < a.E * ntl; i += nth) {
            const int e = i / ntl;
            const int q = i - e * ntl;
            a.tile_counts[(size_t)e * a.tile_stride + tile0 + q] = s_tile[q * a.E + e];
        }
    }
    if (tid == 0 && s_err) atomicOr(&a.hdr->status, s_err);
}

// Both kernels name one dynamic LDS array (a function-scope extern declares
// the same entity), so both declare it alike.
__global__ __launch_bounds__(kLayoutThreads) void moedisp_layout(LayoutArgs a) {
    extern __shared__ __attribute__((aligned(16))) int32_t dyn[];
    __shared__ uint32_t s_err;
    layout_body(a, blockIdx.x, dyn, s_err);
}

// The layout's workgroups and the block-pull sort's in one launch (both read
// only topk_idx): workgroups [0, lay.blocks) are layout workgroups, the next
// sort_wgs sort one token block each.
__global__ __launch_bounds__(kLayoutThreads) void moedisp_layout_sort(LayoutSortArgs a) {
    extern __shared__ __attribute__((aligned(16))) int32_t dyn[];  // the sort's 64-bit masks first
    __shared__ uint32_t s_err;
    if ((int)blockIdx.x < a.lay.blocks) {
        layout_body(a.lay, blockIdx.x, dyn, s_err);
        return;
    }
    if (threadIdx.x == 0) s_err = 0;
    __syncthreads();
    const uint32_t err = pull_sort(a.d, blockIdx.x - a.lay.blocks, dyn);
    if (err) atomicOr(&s_err, err);
    __syncthreads();
    if (threadIdx.x == 0 && s_err) atomicOr(&a.d.hdr->status, s_err);
}

// Sum of the partial counts in workgroup order (one workgroup; the kernel
// boundary orders it after every partial), and expert_offsets when requested.
__global__ __launch_bounds__(kReduceThreads) void moedisp_layout_reduce(LayoutArgs a) {
    __shared__ int32_t s_tot[kMaxExperts];  // expert totals, for expert_offsets
    __shared__ int32_t s_wave[kReduceThreads / 64];
    layout_reduce(a, s_tot, s_wave);
}

}  // namespace

hipError_t launch_layout_sort(const LayoutSortArgs& a, hipStream_t stream) {
    const LayoutArgs& l = a.lay;
    size_t lds = layout_lds_bytes(l.E, l.G, l.k, l.tokens_per_block,
                                  l.tile_counts ? (l.tokens_per_block >> l.tile_shift) : 0);
    const size_t sort = sort_lds_words(a.d.pull.tb, a.d.pull.cap_b, a.d.E) * sizeof(int32_t);
    if (sort > lds) lds = sort;
    const long long blocks = (long long)l.blocks + a.sort_wgs;
    if (!grid_fits(blocks, kLayoutThreads)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(moedisp_layout_sort, dim3((unsigned)blocks), dim3(kLayoutThreads), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_layout_reduce(const LayoutArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(moedisp_layout_reduce, dim3(1), dim3(kReduceThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream, bool reduce) {
    const size_t lds = layout_lds_bytes(a.E, a.G, a.k, a.tokens_per_block,
                                        a.tile_counts ? (a.tokens_per_block >> a.tile_shift) : 0);
    if (!grid_fits(a.blocks, kLayoutThreads)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(moedisp_layout, dim3(a.blocks), dim3(kLayoutThreads), lds, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !reduce) return e;
    hipLaunchKernelGGL(moedisp_layout_reduce, dim3(1), dim3(kReduceThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace moedisp
