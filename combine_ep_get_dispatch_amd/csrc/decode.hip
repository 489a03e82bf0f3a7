// Small-batch (decode) path: layout and dispatch in one kernel launch.
//
// What is computed is exactly ep_get_dispatch_layout followed by ep_dispatch
// ("MSCCLPP EP implementation - #852": the layout's counts and token-in-rank
// flags from the review file table; the dispatch of the PR description's
// scope).  The page's low-latency path is its own single kernel with
// send/count phases and a grid-wide synchronisation in between, tuned for
// small batches; here no workgroup waits for another at all.
//
// A copy workgroup (one token, one column range of its row) needs only its
// token's k receive rows.  The dispatch hands out each expert's rows in flat
// slot order (s = t * k + j), after the rows of every smaller expert, so a
// routed slot s with expert e_s lands before slot (t, j) with expert e iff
// (e_s, s) < (e, t * k + j).  With key(s) = e_s * n + s (n = T * k slots),
//     row(t, j) = #{routed slots s : key(s) < key(t, j)},
// one pass over the routing table (from L2) in which each lane compares its
// share of the keys with the token's k keys (scalar registers), then k sums
// over the workgroup.  No workgroup stages the table, builds a histogram or
// scans it.  The token's first column pass is loaded before that pass.
//
// One extra workgroup writes the layout outputs (counts, offsets, bitmap,
// group counts) and checks ids and repeats, in parallel with the copies, one
// lane per token; column range 0 of each token writes its handle and fp8
// scales.
//
// Padded (low-latency) layout ("MSCCLPP EP implementation - #852": the
// low-latency port gives every expert its own receive slots, sized by a
// maximum token count, with per-expert received counts; a later commit adds
// a rank-major output option).  Expert e owns rows [e*S + B, e*S + B + C);
// slot (t, j) with expert e takes row e*S + B + i, where
//     i = #{routed slots s : e * n <= key(s) < key(t, j)}
// is its rank among e's routed slots, counted in the same pass with a lower
// bound per key; a slot with i >= C gets no row (EXPERT_OVERFLOW).  No
// offsets are needed, so the layout workgroup writes none.
#include "kernels_common.h"

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
    const int incl = wave_inclusive_scan_dpp(sum);
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

// The layout workgroup: tokens_per_expert, expert_offsets, is_token_in_group,
// tokens_per_group and the id checks.  One lane per token holds the token's
// k ids in registers (KM >= k): its group mask and repeated experts come
// from registers, its slots go into the LDS histogram.  LDS (dyn): counts
// [E], offsets [E].
template <int KM>
__device__ void fused_layout(const FusedArgs& a, int32_t* dyn, int32_t* s_gcnt, int32_t* s_wave, uint32_t& err) {
    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const int lane = tid & 63;
    const int k = a.k;
    const int E = a.E;
    int32_t* s_cnt = dyn;
    int32_t* s_off = dyn + E;
    for (int i = tid; i < E; i += nth) s_cnt[i] = 0;
    if (tid < kMaxGroups) s_gcnt[tid] = 0;
    __syncthreads();
    for (int t0 = 0; t0 < a.T; t0 += nth) {  // whole waves in every pass
        const int tt = t0 + tid;
        uint32_t mask = 0;
        if (tt < a.T) {
            int id[KM];
            if (k == KM && (reinterpret_cast<uintptr_t>(a.topk_idx) & 15) == 0) {  // aligned 16-byte groups
                const int4* p4 = reinterpret_cast<const int4*>(a.topk_idx + (size_t)tt * KM);
#pragma unroll
                for (int j = 0; j < KM / 4; ++j) {
                    const int4 q = p4[j];
                    id[4 * j] = q.x;
                    id[4 * j + 1] = q.y;
                    id[4 * j + 2] = q.z;
                    id[4 * j + 3] = q.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < KM; ++j) id[j] = a.topk_idx[(size_t)tt * k + min(j, k - 1)];  // clamped: no branch
            }
#pragma unroll
            for (int j = 0; j < KM; ++j) {
                const int e = id[j];
                if (j < k && (e < -1 || e >= E)) err |= MOEDISP_DEV_BAD_EXPERT_ID;
                if (j < k && e >= 0 && e < E) {
                    atomicAdd(&s_cnt[e], 1);
                    mask |= 1u << (a.pg_shift >= 0 ? (uint32_t)e >> a.pg_shift : __umulhi((uint32_t)e, a.pg_magic));
#pragma unroll
                    for (int j2 = 0; j2 < j; ++j2)
                        if (id[j2] == e) err |= MOEDISP_DEV_DUPLICATE_EXPERT;
                }
            }
            a.is_token_in_group[tt] = mask;
        }
        for (int g = 0; g < a.G; ++g) {
            const uint64_t b = __ballot((mask >> g) & 1u);
            if (lane == 0 && b) atomicAdd(&s_gcnt[g], (int32_t)__popcll(b));
        }
    }
    __syncthreads();
    const int total = lds_exclusive_scan(s_cnt, E, s_off, s_wave);
    for (int e = tid; e < E; e += nth) {
        a.tokens_per_expert[e] = s_cnt[e];
        if (a.expert_offsets) a.expert_offsets[e] = s_off[e];
    }
    if (tid == 0 && a.expert_offsets) a.expert_offsets[E] = total;
    for (int g = tid; g < a.G; g += nth) a.tokens_per_group[g] = s_gcnt[g];
}

// KM: the largest k this instance serves (8 or 32); PAD: the padded layout.
template <int KM, bool PAD>
__global__ __launch_bounds__(kMaxDispatchThreads) void moedisp_dispatch_fused(FusedArgs a) {
    extern __shared__ int32_t dyn[];  // layout workgroup: counts [E], offsets [E]
    __shared__ int32_t s_part[(kMaxDispatchThreads / 64) * KM];  // per-wave counts below the token's keys
    __shared__ int32_t s_key[KM];
    __shared__ int32_t s_row[KM];
    __shared__ int32_t s_gcnt[kMaxGroups];
    __shared__ int32_t s_wave[kMaxDispatchThreads / 64];
    __shared__ uint32_t s_err;

    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int k = a.k;
    const int E = a.E;
    const int n = a.T * k;
    if (tid == 0) s_err = 0;
    uint32_t err = 0;
    // workgroup 0 (dispatched first) writes the layout outputs; the others
    // each copy one token's column range
    if (blockIdx.x == 0) {
        fused_layout<KM>(a, dyn, s_gcnt, s_wave, err);
    } else {
        const int t = (blockIdx.x - 1) / a.col_splits;
        const int split = (blockIdx.x - 1) - t * a.col_splits;
        const int c0 = split * a.split_units;
        const int c1 = min(a.row16, c0 + a.split_units);
        // first pass of this token's row, independent of the rows
        v4u pre = {0, 0, 0, 0};
        if (c0 + tid < c1) pre = a.x[(size_t)t * a.row16 + c0 + tid];
        // the token's keys: lane j < k of every wave loads slot j, and each
        // key is read out of its lane into a scalar register; -1 for a slot
        // past k or masked, whose row is -1 and which no key precedes
        const int sj = t * k + min(lane, k - 1);
        const int ej = a.topk_idx[sj];
        // column range 0 also writes the handle and scales: their loads now
        float wj = 0.0f, scale = 0.0f;
        if (split == 0) {
            if (tid < k) wj = a.topk_weights[sj];
            if (tid < a.scale_words) scale = a.x_scales[(size_t)t * a.scale_words + tid];
        }
        const int kj = (lane < k && ej >= 0 && ej < E) ? ej * n + sj : -1;
        int key_t[KM], lo_t[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) key_t[j] = __builtin_amdgcn_readlane(kj, j);
        if (PAD) {  // the first key of the slot's expert
#pragma unroll
            for (int j = 0; j < KM; ++j) lo_t[j] = key_t[j] >= 0 ? key_t[j] - key_t[j] % n : 0;
        }
        if (tid < KM) s_key[tid] = kj;
        // keys below each of the token's, over this lane's share of the table
        int c[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) c[j] = 0;
        constexpr int kLoads = 8;
        for (int i0 = 0; i0 < n; i0 += kLoads * nth) {
            int v[kLoads];
#pragma unroll
            for (int q = 0; q < kLoads; ++q) v[q] = a.topk_idx[min(i0 + q * nth + tid, n - 1)];
#pragma unroll
            for (int q = 0; q < kLoads; ++q) {
                const int s = i0 + q * nth + tid;
                const int key = (s < n && v[q] >= 0 && v[q] < E) ? v[q] * n + s : 0x7FFFFFFF;
#pragma unroll
                for (int j = 0; j < KM; ++j) c[j] += (key < key_t[j] && (!PAD || key >= lo_t[j])) ? 1 : 0;
            }
        }
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            if (j < k) {  // uniform
                const int w = wave_sum_dpp(c[j]);
                if (lane == 0) s_part[wave * KM + j] = w;
            }
        }
        __syncthreads();
        if (tid < k) {
            int32_t r = -1;
            if (s_key[tid] >= 0) {
                r = 0;
                for (int w = 0; w < nth / 64; ++w) r += s_part[w * KM + tid];
                if (PAD) {  // r is the slot's rank among its expert's slots
                    if (r >= a.pad_c) {
                        err |= MOEDISP_DEV_EXPERT_OVERFLOW;
                        r = -1;
                    } else {
                        r += (s_key[tid] / n) * a.pad_s + a.pad_b;  // < E * pad_s: inside the buffer
                    }
                }
            }
            s_row[tid] = r;  // flat: < the routed total <= T * k, inside the buffer
        }
        __syncthreads();

        // handle and scales of this token (column range 0; the first pass of
        // the scales was loaded with the keys)
        if (split == 0) {
            if (tid < k) {
                const int row = s_row[tid];
                a.slot_to_row[(size_t)t * k + tid] = row;
                if (row >= 0) {
                    a.recv_src_idx[row] = t;
                    a.recv_weights[row] = wj;
                }
            }
            for (int cc = tid; cc < a.scale_words; cc += nth) {
                const float sc = cc == tid ? scale : a.x_scales[(size_t)t * a.scale_words + cc];
                for (int q = 0; q < k; ++q) {
                    const int row = s_row[q];
                    if (row >= 0) a.recv_scales[(size_t)row * a.scale_words + cc] = sc;
                }
            }
        }
        // row copy: each 16-byte unit loaded once, stored to every routed slot's row
        for (int cc = c0 + tid; cc < c1; cc += nth) {
            const v4u v = (cc == c0 + tid) ? pre : a.x[(size_t)t * a.row16 + cc];
            for (int j = 0; j < k; ++j) {
                const int r = s_row[j];
                if (r >= 0) __builtin_nontemporal_store(v, a.recv_x + (size_t)r * a.row16 + cc);
            }
        }
    }
    if (err) atomicOr(&s_err, err);
    __syncthreads();
    if (tid == 0 && s_err) atomicOr(&a.hdr->status, s_err);
}

}  // namespace

hipError_t launch_dispatch_fused(const FusedArgs& a, hipStream_t stream) {
    // the layout workgroup's tables
    const size_t lds = 2 * (size_t)a.E * sizeof(int32_t);
    const unsigned blocks = (unsigned)(a.T * a.col_splits) + 1u;  // + the layout workgroup
    if (a.pad_s > 0) {
        if (a.pad_c < 0 || a.pad_b < 0 || (long long)a.pad_b + a.pad_c > a.pad_s) return hipErrorInvalidValue;
        if (a.k <= 8)
            hipLaunchKernelGGL((moedisp_dispatch_fused<8, true>), dim3(blocks), dim3(a.threads), lds, stream, a);
        else
            hipLaunchKernelGGL((moedisp_dispatch_fused<kMaxTopk, true>), dim3(blocks), dim3(a.threads), lds, stream,
                               a);
    } else if (a.k <= 8) {
        hipLaunchKernelGGL((moedisp_dispatch_fused<8, false>), dim3(blocks), dim3(a.threads), lds, stream, a);
    } else {
        hipLaunchKernelGGL((moedisp_dispatch_fused<kMaxTopk, false>), dim3(blocks), dim3(a.threads), lds, stream, a);
    }
    return hipGetLastError();
}

}  // namespace moedisp
