// Small-batch (decode) path: layout and dispatch in one kernel launch.
//
// What is computed is exactly ep_get_dispatch_layout followed by ep_dispatch
// ("MSCCLPP EP implementation - #852": the layout's counts and token-in-rank
// flags from the review file table; the dispatch of the PR description's
// scope).  The page's low-latency path is its own single kernel with
// send/count phases and a grid-wide synchronisation in between, tuned for
// small batches; here no workgroup waits for another at all.  With at most
// kFusedMaxSlots routing slots, every workgroup stages the whole routing table
// (a few KB, from L2) in LDS and derives from it what it needs:
//   - the expert histogram (LDS atomics) and its exclusive scan, i.e.
//     tokens_per_expert and expert_offsets;
//   - for its own token's slots, the number of earlier slots (flat (t, j)
//     order) with the same expert, L lanes per slot;
// so every workgroup knows its rows without any cross-workgroup traffic and
// copies its token's row (its column range of it) to them with 16-byte
// non-temporal stores, the first pass loaded before the layout work.  One
// extra workgroup writes the layout outputs (counts, bitmap, group counts,
// offsets) and checks ids and repeats, in parallel with the copies; column
// range 0 of each token writes its handle and fp8 scales.
#include "moedisp_internal.h"

namespace moedisp {
namespace {

// Exclusive scan of in[0..n) (non-negative, LDS, total < 2^31) into out
// (LDS); returns the total.  Whole workgroup; has barriers.
__device__ int lds_exclusive_scan(const int32_t* in, int n, int32_t* out, int32_t* s_wave) {
    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int per = (n + nth - 1) / nth;
    const int lo = min(n, tid * per);
    const int hi = min(n, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += in[i];
    int incl = sum;
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int run = incl - sum;
    int total = 0;
    for (int w = 0; w < nth / 64; ++w) {
        if (w < wave) run += s_wave[w];
        total += s_wave[w];
    }
    for (int i = lo; i < hi; ++i) {
        const int v = in[i];
        out[i] = run;
        run += v;
    }
    __syncthreads();
    return total;
}

__global__ __launch_bounds__(kMaxDispatchThreads) void moedisp_dispatch_fused(FusedArgs a) {
    extern __shared__ int32_t dyn[];  // ids [T*k], counts [E], offsets [E], token group masks [T]
    const int n = a.T * a.k;
    int32_t* s_ids = dyn;
    int32_t* s_cnt = dyn + n;
    int32_t* s_off = s_cnt + a.E;
    uint32_t* s_mask = reinterpret_cast<uint32_t*>(s_off + a.E);
    __shared__ int32_t s_pre[kMaxTopk];
    __shared__ int32_t s_row[kMaxTopk];
    __shared__ int32_t s_gcnt[kMaxGroups];
    __shared__ int32_t s_wave[kMaxDispatchThreads / 64];
    __shared__ uint32_t s_err;

    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const int k = a.k;
    const int E = a.E;
    // the last workgroup writes the layout outputs; the others each copy one
    // token's column range
    const bool layout_wg = blockIdx.x == gridDim.x - 1;
    const int t = blockIdx.x / a.col_splits;
    const int split = blockIdx.x - t * a.col_splits;
    const bool copy_wg = !layout_wg;  // then t < T
    const int c0 = split * a.split_units;
    const int c1 = min(a.row16, c0 + a.split_units);

    // first pass of this token's row, independent of the layout
    v4u pre = {0, 0, 0, 0};
    if (copy_wg && c0 + tid < c1) pre = a.x[(size_t)t * a.row16 + c0 + tid];

    for (int i = tid; i < E; i += nth) s_cnt[i] = 0;
    if (tid < kMaxTopk) s_pre[tid] = 0;
    if (tid < kMaxGroups) s_gcnt[tid] = 0;
    if (tid == 0) s_err = 0;
    if (layout_wg)
        for (int i = tid; i < a.T; i += nth) s_mask[i] = 0;
    uint32_t err = 0;
    // stage the routing table: 8 independent loads in flight per lane
    // (clamped indices: the loads carry no branch, so they issue together)
    constexpr int kStage = 8;
    for (int i0 = 0; i0 < n; i0 += kStage * nth) {
        int v[kStage];
#pragma unroll
        for (int q = 0; q < kStage; ++q) v[q] = a.topk_idx[min(i0 + q * nth + tid, n - 1)];
#pragma unroll
        for (int q = 0; q < kStage; ++q) {
            const int i = i0 + q * nth + tid;
            const bool ok = v[q] >= 0 && v[q] < E;
            if (!ok && v[q] != -1 && layout_wg) err |= MOEDISP_DEV_BAD_EXPERT_ID;
            if (i < n) s_ids[i] = ok ? v[q] : -1;
        }
    }
    __syncthreads();

    // expert histogram; the layout workgroup also forms each token's group
    // mask and looks for repeated experts, one slot per lane
    for (int i0 = 0; i0 < n; i0 += 4 * nth) {
        int ev[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) ev[m] = s_ids[min(i0 + m * nth + tid, n - 1)];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int i = i0 + m * nth + tid;
            const int e = ev[m];
            if (i >= n || e < 0) continue;
            atomicAdd(&s_cnt[e], 1);
            if (layout_wg) {
                const int tt = i / k;
                const int base = tt * k;
                const uint32_t g = a.pg_shift >= 0 ? (uint32_t)e >> a.pg_shift : __umulhi((uint32_t)e, a.pg_magic);
                atomicOr(&s_mask[tt], 1u << g);
                for (int u0 = base; u0 < i; u0 += 8) {  // 8 clamped reads per step, no branch
                    int v[8];
#pragma unroll
                    for (int m = 0; m < 8; ++m) v[m] = s_ids[min(u0 + m, i - 1)];
#pragma unroll
                    for (int m = 0; m < 8; ++m)
                        if (u0 + m < i && v[m] == e) err |= MOEDISP_DEV_DUPLICATE_EXPERT;
                }
            }
        }
    }
    // earlier slots (flat (t, j) order) with the same expert, for this token's
    // slots: L lanes each, 8 independent LDS reads per step
    if (copy_wg) {
        const int L = nth / k;  // >= 1: at least 256 lanes, k <= 32
        if (tid < L * k) {
            const int q = tid / L;
            const int l = tid - q * L;
            const int s = t * k + q;
            const int e = s_ids[s];
            if (e >= 0) {
                int32_t c = 0;
                for (int u0 = l; u0 < s; u0 += 8 * L) {
                    int v[8];
#pragma unroll
                    for (int m = 0; m < 8; ++m) v[m] = s_ids[min(u0 + m * L, s - 1)];  // clamped: no branch
#pragma unroll
                    for (int m = 0; m < 8; ++m) c += (u0 + m * L < s && v[m] == e) ? 1 : 0;
                }
                if (c) atomicAdd(&s_pre[q], c);
            }
        }
    }
    __syncthreads();
    const int total = lds_exclusive_scan(s_cnt, E, s_off, s_wave);

    if (copy_wg) {
        // rows of this token's slots (< total <= T*k: always inside the buffer)
        if (tid < k) {
            const int e = s_ids[t * k + tid];
            s_row[tid] = e >= 0 ? s_off[e] + s_pre[tid] : -1;
        }
    } else {
        // layout outputs: counts, offsets, token-in-group bitmap, and tokens
        // per group (one ballot per group and wave)
        for (int e = tid; e < E; e += nth) {
            a.tokens_per_expert[e] = s_cnt[e];
            a.expert_offsets[e] = s_off[e];
        }
        if (tid == 0) a.expert_offsets[E] = total;
        const int lane = tid & 63;
        for (int t0 = 0; t0 < a.T; t0 += nth) {
            const int tt = t0 + tid;
            const uint32_t mask = tt < a.T ? s_mask[tt] : 0u;
            if (tt < a.T) a.is_token_in_group[tt] = mask;
            for (int g = 0; g < a.G; ++g) {
                const uint64_t b = __ballot((mask >> g) & 1u);
                if (lane == 0 && b) atomicAdd(&s_gcnt[g], (int32_t)__popcll(b));
            }
        }
    }
    __syncthreads();
    if (layout_wg)
        for (int g = tid; g < a.G; g += nth) a.tokens_per_group[g] = s_gcnt[g];

    // handle and scales of this token (column range 0)
    if (copy_wg && split == 0) {
        for (int q = tid; q < k; q += nth) {
            const size_t slot = (size_t)t * k + q;
            const int row = s_row[q];
            a.slot_to_row[slot] = row;
            if (row >= 0) {
                a.recv_src_idx[row] = t;
                a.recv_weights[row] = a.topk_weights[slot];
            }
        }
        if (a.scale_words) {
            const int ns = k * a.scale_words;
            for (int i = tid; i < ns; i += nth) {
                const int q = i / a.scale_words;
                const int c = i - q * a.scale_words;
                const int row = s_row[q];
                if (row >= 0)
                    a.recv_scales[(size_t)row * a.scale_words + c] = a.x_scales[(size_t)t * a.scale_words + c];
            }
        }
    }

    // row copy: each 16-byte unit loaded once, stored to every routed slot's row
    if (copy_wg) {
        for (int c = c0 + tid; c < c1; c += nth) {
            const v4u v = (c == c0 + tid) ? pre : a.x[(size_t)t * a.row16 + c];
            for (int j = 0; j < k; ++j) {
                const int r = s_row[j];
                if (r >= 0) __builtin_nontemporal_store(v, a.recv_x + (size_t)r * a.row16 + c);
            }
        }
    }

    if (err) atomicOr(&s_err, err);
    __syncthreads();
    if (tid == 0 && s_err) atomicOr(&a.hdr->status, s_err);
}

}  // namespace

hipError_t launch_dispatch_fused(const FusedArgs& a, hipStream_t stream) {
    const size_t lds = ((size_t)a.T * a.k + 2 * (size_t)a.E + (size_t)a.T) * sizeof(int32_t);
    const unsigned blocks = (unsigned)(a.T * a.col_splits) + 1u;  // + the layout workgroup
    hipLaunchKernelGGL(moedisp_dispatch_fused, dim3(blocks), dim3(a.threads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace moedisp
