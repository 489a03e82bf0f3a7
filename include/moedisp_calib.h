/* libmoedisp calibration probes: kernels that are not part of the dispatch /
 * combine path, exported by the same library so that a benchmark can measure
 * the part's achievable HBM bandwidth in the same process and scale hardware
 * byte counters against a kernel of known traffic.
 *
 * Each probe runs on `stream` (NULL: the null stream) and returns a host code
 * of moedisp.h (MOEDISP_OK, or INVALID_ARG / UNSUPPORTED / MISALIGNED when the
 * arguments break the rules stated below, before anything is launched; HIP
 * when the launch fails).  Buffers are device memory that the caller owns.
 *
 * The read and copy probes give every workgroup of 512 lanes one 16 KiB chunk
 * (two 16-byte units per lane, non-temporal loads and stores) and exit: the
 * shape that measured fastest on this part among one-chunk-per-workgroup and
 * grid-stride kernels with 256 to 1024 lanes, 1 to 8 loads in flight per lane
 * and chunks of 4 KiB to 256 KiB. */
#ifndef MOEDISP_CALIB_H
#define MOEDISP_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read-only stream: reads `bytes` from `src` (a multiple of 16; 16-byte
 * aligned) and folds them by XOR; `sink` (16 bytes, 16-byte aligned) is
 * written only if the fold hits a fixed 64-bit pattern, so the reads cannot
 * be dropped.  The ceiling of kernels that mostly read (a gather-sum). */
int ep_probe_read(const void* src, size_t bytes, void* sink, void* stream);

/* Copy of `bytes` (a multiple of 16; both pointers 16-byte aligned, buffers
 * not overlapping) from `src` to `dst`.  The ceiling of kernels that read
 * and write in equal parts, and the known traffic (bytes read, bytes
 * written) that scales hardware byte counters. */
int ep_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Writes `bytes` (a multiple of 4096; dst 16-byte aligned) in 4 KiB chunks,
 * one workgroup per chunk, the chunks in address order (shuffled = 0) or in
 * a fixed permuted order (shuffled = 1).  16-byte unit i of the buffer
 * receives the four 32-bit words {i mod 2^32, i / 2^32, ~(i mod 2^32),
 * 0x5EED}, whatever the order.  Measures the HBM write bandwidth of
 * sequential against scattered write streams, the two ends between which a
 * row scatter's writes fall.  Returns UNSUPPORTED for a size that is not a
 * multiple of 4096 or a `shuffled` other than 0 or 1. */
int ep_probe_fill(void* dst, size_t bytes, int32_t shuffled, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEDISP_CALIB_H */
