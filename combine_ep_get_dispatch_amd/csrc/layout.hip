// Layout kernel: tokens per expert, tokens per group and the token-in-group
// bitmap ("counts + token-in-rank" of the high-throughput layout kernel on the
// "MSCCLPP EP implementation - #852" page, review file table).
//
// One thread per token, 256 tokens per workgroup.  The workgroup's routing
// rows are staged in LDS (padded to an odd stride so a wave reading one slot
// of 64 tokens hits distinct banks).  Expert counts go to an LDS-private
// histogram: for each slot, the lanes of a wave that carry the same expert
// find each other with one ballot per bit of the expert id, and only the
// lowest such lane adds the popcount of its peer mask - one LDS atomic per
// distinct expert per wave instead of one per lane, which matters under skewed
// routing.  Group counts are popcounts of one ballot per group.  Each
// workgroup writes its partial counts to the workspace; the last workgroup to
// finish sums them in workgroup order and resets the finish counter.
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

// Group of expert id: id / (E/G) by a shift (power-of-two group sizes) or by
// a multiply-high with a host-computed reciprocal (exact for id, E <= 4096).
__device__ inline uint32_t group_of(uint32_t id, const LayoutArgs& a) {
    return a.pg_shift >= 0 ? id >> a.pg_shift : __umulhi(id, a.pg_magic);
}

// KMAX: compile-time bound on k; a token's routing row lives in registers.
template <int KMAX>
__global__ __launch_bounds__(kThreads) void moedisp_layout(LayoutArgs a) {
    extern __shared__ int32_t dyn[];  // [E + G] counts, then the staged routing rows
    const int EG = a.E + a.G;
    int32_t* s_cnt = dyn;
    int32_t* s_ids = dyn + EG;
    __shared__ uint32_t s_err;
    __shared__ uint32_t s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int k = a.k;
    const int kp = k | 1;  // odd LDS stride
    const int t0 = blockIdx.x * kLayoutTokensPerBlock;
    const int nt = max(0, min(kLayoutTokensPerBlock, a.T - t0));

    for (int i = tid; i < EG; i += kThreads) s_cnt[i] = 0;
    if (tid == 0) s_err = 0;
    // stage the routing rows: 8 independent coalesced loads in flight per lane
    constexpr int kStage = 8;
    const int n = nt * k;
    for (int i0 = 0; i0 < n; i0 += kStage * kThreads) {
        int32_t v[kStage];
#pragma unroll
        for (int q = 0; q < kStage; ++q) {
            const int i = i0 + q * kThreads + tid;
            v[q] = i < n ? a.topk_idx[(size_t)t0 * k + i] : 0;
        }
#pragma unroll
        for (int q = 0; q < kStage; ++q) {
            const int i = i0 + q * kThreads + tid;
            if (i < n) {
                const int tt = i / k;
                s_ids[tt * kp + (i - tt * k)] = v[q];
            }
        }
    }
    __syncthreads();

    const bool have = tid < nt;
    const uint64_t below = (1ull << lane) - 1ull;
    uint32_t gmask = 0;
    uint32_t err = 0;
    int ids[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        int id = (have && j < k) ? s_ids[tid * kp + j] : -1;
        if (id < -1 || id >= a.E) {
            err |= MOEDISP_DEV_BAD_EXPERT_ID;
            id = -1;
        }
        ids[j] = id;
    }
#pragma unroll
    for (int j = 1; j < KMAX; ++j)
#pragma unroll
        for (int jj = 0; jj < j; ++jj)
            if (ids[j] >= 0 && ids[j] == ids[jj]) err |= MOEDISP_DEV_DUPLICATE_EXPERT;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j < k) {  // k is uniform
            const int id = ids[j];
            const bool routed = id >= 0;
            if (routed) gmask |= 1u << group_of((uint32_t)id, a);
            const uint64_t active = __ballot(routed);
            const uint64_t peers = match_peers(routed ? (uint32_t)id : 0u, a.id_bits, active);
            if (routed && (peers & below) == 0) atomicAdd(&s_cnt[id], (int32_t)__popcll(peers));
        }
    }
    for (int g = 0; g < a.G; ++g) {
        const uint64_t in_g = __ballot((gmask >> g) & 1u);
        if (lane == 0 && in_g) atomicAdd(&s_cnt[a.E + g], (int32_t)__popcll(in_g));
    }
    if (have) a.is_token_in_group[t0 + tid] = gmask;
    if (err) atomicOr(&s_err, err);
    __syncthreads();

    int32_t* mine = a.partials + (size_t)blockIdx.x * EG;
    for (int i = tid; i < EG; i += kThreads) mine[i] = s_cnt[i];
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        if (s_err) atomicOr(&a.hdr->status, s_err);
        const uint32_t prev = atomicAdd(&a.hdr->layout_done, 1u);
        s_last = prev == (uint32_t)(a.blocks - 1);
    }
    __syncthreads();
    if (!s_last) return;

    __threadfence();
    // sum the partials in workgroup order, 16 independent loads in flight
    constexpr int kBatch = 16;
    for (int i = tid; i < EG; i += kThreads) {
        int32_t sum = 0;
        for (int b0 = 0; b0 < a.blocks; b0 += kBatch) {
            int32_t v[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q)
                v[q] = (b0 + q < a.blocks) ? a.partials[(size_t)(b0 + q) * EG + i] : 0;
#pragma unroll
            for (int q = 0; q < kBatch; ++q) sum += v[q];
        }
        if (i < a.E)
            a.tokens_per_expert[i] = sum;
        else
            a.tokens_per_group[i - a.E] = sum;
    }
    if (tid == 0) __hip_atomic_store(&a.hdr->layout_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream) {
    const size_t lds = (size_t)(a.E + a.G + kLayoutTokensPerBlock * (a.k | 1)) * sizeof(int32_t);
    if (a.k <= 8)
        hipLaunchKernelGGL((moedisp_layout<8>), dim3(a.blocks), dim3(kThreads), lds, stream, a);
    else if (a.k <= 16)
        hipLaunchKernelGGL((moedisp_layout<16>), dim3(a.blocks), dim3(kThreads), lds, stream, a);
    else
        hipLaunchKernelGGL((moedisp_layout<kMaxTopk>), dim3(a.blocks), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace moedisp
