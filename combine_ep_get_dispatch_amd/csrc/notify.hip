// Notify phase of the block-pull dispatch: one launch in which each
// workgroup takes one role (NotifyArgs):
//   - sort one token block: list its slots in (expert, slot) order;
//   - count one dispatch tile of the push path's table (which the quantising
//     scatter reads), tile 0 possibly writing expert_offsets;
//   - sum the layout's partial counts (the layout's reduce, with
//     expert_offsets), when the call folds the layout in, or scan
//     tokens_per_expert into expert_offsets.
// The roles are independent: no workgroup waits for another.
//
// The sort (pull_sort, with the device helpers) lists each block's slots in
// (expert, slot) order; entry i of expert e in block b receives the row
//     expert_offsets[e] + sum_{b' < b} cnt_b'[e] + (i - ls_b[e]),
// which is the row the definition gives: each expert's rows are contiguous
// and in token order, and the tokens of earlier blocks come first.
#include "kernels_common.h"

namespace moedisp {
namespace {

__global__ __launch_bounds__(kNotifyThreads) void moedisp_notify(NotifyArgs a) {
    extern __shared__ __attribute__((aligned(16))) int32_t dyn[];  // the sort's 64-bit masks first
    __shared__ long long s_wave[kNotifyWaves];
    __shared__ uint32_t s_err;
    const int wg = blockIdx.x;
    if (threadIdx.x == 0) s_err = 0;
    __syncthreads();
    uint32_t err = 0;
    if (wg < a.sort_wgs) {
        err = pull_sort(a.d, wg, dyn);
    } else if (wg < a.sort_wgs + a.count_wgs) {
        err = count_tile(a.d, wg - a.sort_wgs, a.count_offsets != 0, dyn, s_wave);
    } else if (a.reduce == 1) {
        layout_reduce(a.lay, dyn, reinterpret_cast<int32_t*>(s_wave));
    } else if (a.reduce == 2) {
        err = offsets_scan(a.d, dyn, s_wave);
    }
    if (err) atomicOr(&s_err, err);
    __syncthreads();
    if (threadIdx.x == 0 && s_err) atomicOr(&a.d.hdr->status, s_err);
}

}  // namespace

size_t notify_lds_bytes(const NotifyArgs& a) {
    size_t words = 0;
    if (a.sort_wgs) words = sort_lds_words(a.d.pull.tb, a.d.pull.cap_b, a.d.E);
    if (a.count_wgs && (size_t)a.d.E > words) words = a.d.E;
    if (a.reduce && (size_t)a.d.E > words) words = a.d.E;
    return words * sizeof(int32_t);
}

hipError_t launch_notify(const NotifyArgs& a, hipStream_t stream) {
    const long long blocks = (long long)a.sort_wgs + a.count_wgs + (a.reduce ? 1 : 0);
    if (!grid_fits(blocks, kNotifyThreads)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(moedisp_notify, dim3((unsigned)blocks), dim3(kNotifyThreads), notify_lds_bytes(a), stream, a);
    return hipGetLastError();
}

}  // namespace moedisp
