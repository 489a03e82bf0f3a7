// Combine kernel: gather each token's expert outputs back through the dispatch
// handle and form the weighted top-k sum.
//
// What is computed ("MSCCLPP EP implementation - #852": PR description,
// "Scope", intranode combine; the commit message fixing internode combine says
// combine runs in the reverse direction of dispatch and must consume the
// receiver-side bookkeeping dispatch returned; the commit message on combine
// byte accounting says one returned row is read per routed copy):
//     out[t][h] = sum_{j = 0..k-1, slot routed} recv_weights[r] * expert_out[r][h],
//     r = slot_to_row[t][j],
// accumulated in fp32 by fused multiply-add in ascending j from 0, then rounded
// once to bf16 (nearest-even, v_cvt_pk_bf16_f32) or stored as fp32.  The same
// kernel serves the group path: the local reduce of each (token, group) row
// (rows past a device-side row limit are skipped) and the sum of a token's
// group rows (no weights: a fused multiply-add by 1 is the plain fp32 add).
//
// How.  One workgroup per (token, column range).  The token's k rows and
// weights are uniform across the workgroup, so they come through scalar loads;
// the handle is checked there (row inside the receive buffer and, when
// recv_src_idx is given, naming this token) and a slot that fails is skipped
// at accumulation, with BAD_HANDLE raised.  The token's routed slots are
// compacted (slot order kept) and a switch on their count picks an unrolled
// gather, so no masked slot costs a load.  Each lane owns U 16-byte units (8
// bf16) of the output row (U = 1 with workgroups of 64 lanes for k >= 8 or
// 128 lanes otherwise, so a 7168-wide row at k = 8 is 14 workgroups; U = 2
// and about 256 lanes where a row gathers about one slot): it issues all k*U
// gathered 16-byte loads before the first FMA, so each lane keeps k*U loads
// in flight, then accumulates slot by slot in order.
// With k known at compile time (1, 2, 4, 8) the slot loop is unrolled; other
// k take the generic loop.
#include "moedisp_internal.h"

namespace moedisp {
namespace {

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    const bf2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ inline void fma8(float* acc, float w, v4u v) {
    acc[0] = __builtin_fmaf(w, bf16_lo(v.x), acc[0]);
    acc[1] = __builtin_fmaf(w, bf16_hi(v.x), acc[1]);
    acc[2] = __builtin_fmaf(w, bf16_lo(v.y), acc[2]);
    acc[3] = __builtin_fmaf(w, bf16_hi(v.y), acc[3]);
    acc[4] = __builtin_fmaf(w, bf16_lo(v.z), acc[4]);
    acc[5] = __builtin_fmaf(w, bf16_hi(v.z), acc[5]);
    acc[6] = __builtin_fmaf(w, bf16_lo(v.w), acc[6]);
    acc[7] = __builtin_fmaf(w, bf16_hi(v.w), acc[7]);
}

// One output unit of token t (16 bytes of bf16, or 32 of fp32) at column
// unit cc.  bf16 rows (the path's output) go out as buffer stores from the
// token's row (a wave-uniform base) with the sc1 policy.  At T = 4096,
// H = 7168, k = 8 the combine's reads alone run at the rate of a plain read
// stream (a bare gather-sum without its stores: 68.4 against 68.3 us), and
// its 58.7 MB of output writes cost 20 us more; with sc1 they cost about
// 1.8 us less than with non-temporal stores (median of 5 cold A/B rounds:
// 89.5 against 91.3 us), nt with sc0 and sc1 no better; the same at k = 2.
template <bool kF32>
__device__ inline void store_out(void* out, int row16, int t, int cc, const float* acc) {
    if constexpr (kF32) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        f4* o = reinterpret_cast<f4*>(out) + 2 * ((size_t)t * row16 + cc);
        const f4 a0 = {acc[0], acc[1], acc[2], acc[3]};
        const f4 a1 = {acc[4], acc[5], acc[6], acc[7]};
        __builtin_nontemporal_store(a0, o);
        __builtin_nontemporal_store(a1, o + 1);
    } else {
        v4u r;
        r.x = pack_bf16x2(acc[0], acc[1]);
        r.y = pack_bf16x2(acc[2], acc[3]);
        r.z = pack_bf16x2(acc[4], acc[5]);
        r.w = pack_bf16x2(acc[6], acc[7]);
        v4u* row = reinterpret_cast<v4u*>(out) + (size_t)t * row16;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(row, (short)0, row16 * 16, kRawBufferWord3);
        __builtin_amdgcn_raw_buffer_store_b128(r, rs, cc * 16, 0, kCombineStorePolicy);
    }
}

// Row and weight of slot j of token t, with the handle checks.
__device__ inline int handle_row(const CombineArgs& a, int t, int j, float* w, uint32_t* err) {
    int r = a.slot_to_row[(size_t)t * a.k + j];
    *w = 0.0f;
    if (r < -1 || r >= a.capacity) {
        *err |= MOEDISP_DEV_BAD_HANDLE;
        return -1;
    }
    if (r >= 0) {
        *w = a.recv_weights ? a.recv_weights[r] : 1.0f;
        if (a.recv_src_idx && a.recv_src_idx[r] != t) {
            *err |= MOEDISP_DEV_BAD_HANDLE;
            return -1;
        }
    }
    return r;
}

// Weighted sum over N compacted slots (rows crow[0..N), in slot order) for
// this lane's columns.  All N*U row loads of a pass are issued back to back
// (no per-slot branch), then the weights and source tokens as scalar loads
// that are in flight with them.  A slot whose row fails the source check is
// skipped at accumulation.
template <int N, int U, bool kF32>
__device__ inline void gather_sum(const CombineArgs& a, int t, int c0, int c1, const int* crow, uint32_t* err) {
    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    int c = c0 + tid;
    v4u v[N > 0 ? N : 1][U];
#pragma unroll
    for (int p = 0; p < N; ++p)
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[p][u] = __builtin_nontemporal_load(a.expert_out + (size_t)crow[p] * a.row16 + min(c + u * nth, c1 - 1));
    // weights and source tokens: uniform scalar loads issued after the row
    // loads (a scheduling barrier keeps that order), in flight with them
    __builtin_amdgcn_sched_barrier(0);
    float w[N > 0 ? N : 1];
    int src[N > 0 ? N : 1];
    if (a.recv_weights) {
#pragma unroll
        for (int p = 0; p < N; ++p) w[p] = a.recv_weights[crow[p]];
    } else {
#pragma unroll
        for (int p = 0; p < N; ++p) w[p] = 1.0f;
    }
    if (a.recv_src_idx) {
#pragma unroll
        for (int p = 0; p < N; ++p) src[p] = a.recv_src_idx[crow[p]];
    } else {
#pragma unroll
        for (int p = 0; p < N; ++p) src[p] = t;
    }
    bool ok[N > 0 ? N : 1];
#pragma unroll
    for (int p = 0; p < N; ++p) {
        ok[p] = src[p] == t;
        *err |= ok[p] ? 0u : MOEDISP_DEV_BAD_HANDLE;
    }
    while (c < c1) {
        float acc[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;
#pragma unroll
        for (int p = 0; p < N; ++p) {
            if (!ok[p]) continue;
#pragma unroll
            for (int u = 0; u < U; ++u) fma8(acc[u], w[p], v[p][u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cc = c + u * nth;
            if (cc < c1) store_out<kF32>(a.out, a.row16, t, cc, acc[u]);
        }
        c += U * nth;
        if (c >= c1) break;
#pragma unroll
        for (int p = 0; p < N; ++p)
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[p][u] = __builtin_nontemporal_load(a.expert_out + (size_t)crow[p] * a.row16 +
                                                     min(c + u * nth, c1 - 1));
    }
}

// KC: compile-time k (0 = runtime k, slots gathered one at a time).
template <int KC, int U, bool kF32>
__global__ __launch_bounds__(kMaxCombineThreads) void moedisp_combine(CombineArgs a) {
    const int t = blockIdx.x / a.col_splits;
    const int split = blockIdx.x - t * a.col_splits;
    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const int per_split = (a.row16 + a.col_splits - 1) / a.col_splits;
    const int c0 = split * per_split;
    const int c1 = min(a.row16, c0 + per_split);
    uint32_t err = 0;
    if (a.row_limit && t >= *a.row_limit) return;  // uniform: whole workgroup

    if constexpr (KC > 0) {
        // the token's rows inside the receive buffer, compacted in slot order
        // (uniform values: scalar registers and selects, no indexing)
        int rows[KC];
        bool use[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            const int r = a.slot_to_row[(size_t)t * KC + j];
            if (r < -1 || r >= a.capacity) err |= MOEDISP_DEV_BAD_HANDLE;
            use[j] = r >= 0 && r < a.capacity;
            rows[j] = r;
        }
        int n = 0;
#pragma unroll
        for (int j = 0; j < KC; ++j) n += use[j] ? 1 : 0;
        if (n == KC) {  // every slot routed (the common case): no compaction
            gather_sum<KC, U, kF32>(a, t, c0, c1, rows, &err);
        } else {
        int crow[KC];
#pragma unroll
        for (int p = 0; p < KC; ++p) crow[p] = 0;
        int m = 0;
#pragma unroll
        for (int j = 0; j < KC; ++j) {
#pragma unroll
            for (int p = 0; p <= j; ++p)
                if (use[j] && m == p) crow[p] = rows[j];
            m += use[j] ? 1 : 0;
        }
        switch (n) {
            case 0: gather_sum<0, U, kF32>(a, t, c0, c1, crow, &err); break;
            case 1: gather_sum<(KC >= 1 ? 1 : 0), U, kF32>(a, t, c0, c1, crow, &err); break;
            case 2: gather_sum<(KC >= 2 ? 2 : 0), U, kF32>(a, t, c0, c1, crow, &err); break;
            case 3: gather_sum<(KC >= 3 ? 3 : 0), U, kF32>(a, t, c0, c1, crow, &err); break;
            case 4: gather_sum<(KC >= 4 ? 4 : 0), U, kF32>(a, t, c0, c1, crow, &err); break;
            case 5: gather_sum<(KC >= 5 ? 5 : 0), U, kF32>(a, t, c0, c1, crow, &err); break;
            case 6: gather_sum<(KC >= 6 ? 6 : 0), U, kF32>(a, t, c0, c1, crow, &err); break;
            case 7: gather_sum<(KC >= 7 ? 7 : 0), U, kF32>(a, t, c0, c1, crow, &err); break;
            default: gather_sum<(KC >= 8 ? 8 : 0), U, kF32>(a, t, c0, c1, crow, &err); break;
        }
        }
    } else {
        if (tid == 0)
            for (int j = 0; j < a.k; ++j) {
                float w;
                handle_row(a, t, j, &w, &err);
            }
        uint32_t ignored = 0;
        for (int c = c0 + tid; c < c1; c += U * nth) {
            float acc[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;
            for (int j = 0; j < a.k; ++j) {
                float w;
                const int r = handle_row(a, t, j, &w, &ignored);
                if (r < 0) continue;
                v4u v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int cc = c + u * nth;
                    if (cc < c1) v[u] = __builtin_nontemporal_load(a.expert_out + (size_t)r * a.row16 + cc);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) fma8(acc[u], w, v[u]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int cc = c + u * nth;
                if (cc < c1) store_out<kF32>(a.out, a.row16, t, cc, acc[u]);
            }
        }
    }
    if (err && split == 0 && tid == 0) atomicOr(&a.hdr->status, err);
}

template <int KC, bool kF32>
hipError_t launch_k(const CombineArgs& a, hipStream_t stream) {
    const long long blocks = (long long)a.T * a.col_splits;
    if (!grid_fits(blocks, a.threads)) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks), block(a.threads);
    if (a.units_per_lane == 1)
        hipLaunchKernelGGL((moedisp_combine<KC, 1, kF32>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((moedisp_combine<KC, 2, kF32>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <bool kF32>
hipError_t launch_any(const CombineArgs& a, hipStream_t stream) {
    switch (a.k) {
        case 1: return launch_k<1, kF32>(a, stream);
        case 2: return launch_k<2, kF32>(a, stream);
        case 4: return launch_k<4, kF32>(a, stream);
        case 8: return launch_k<8, kF32>(a, stream);
        default: return launch_k<0, kF32>(a, stream);
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, bool f32_out, hipStream_t stream) {
    return f32_out ? launch_any<true>(a, stream) : launch_any<false>(a, stream);
}

}  // namespace moedisp
