/*
 * moedisp.h - C ABI of libmoedisp: one GPU's share of MoE expert-parallel
 * token layout, dispatch and combine, written for MI355X (gfx950).
 *
 * The operations follow the MSCCL++ EP pull request page ("MSCCLPP EP
 * implementation - #852"):
 *   - PR description, "Scope": get_dispatch_layout, dispatch and combine are
 *     the three calls of the expert-parallel path;
 *   - review file table, high-throughput layout kernel entry: the layout call
 *     produces token counts and token-in-rank flags;
 *   - commit message fixing internode combine: combine runs in the reverse
 *     direction of dispatch and consumes receiver-side bookkeeping that
 *     dispatch returned;
 *   - commit message on combine byte accounting: one returned row per routed
 *     copy;
 *   - warp-geometry commit messages and the code-scanning excerpt: hidden
 *     rows are moved in 16-byte units.
 * A destination rank of the page is a destination GROUP here: a contiguous
 * block of E/G experts whose receive rows are a contiguous range of this
 * GPU's HBM.
 *
 * Conventions shared by every call
 *   - Every pointer argument is DEVICE memory owned by the caller, except the
 *     moedisp_shape pointer and ep_check_status's host_status (host memory).
 *     The library never allocates, never frees and keeps no device memory of
 *     its own; all scratch state lives in the caller's workspace `ws`.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on it and returns; nothing synchronises
 *     except ep_check_status.
 *   - Row buffers (x, recv_x, expert_out, out) must be 16-byte aligned and a
 *     row must be a whole number of 16-byte units (H * element size % 16 == 0).
 *     Index, weight and scale arrays must be 4-byte aligned; ws 256-byte aligned.
 *   - Arguments that can be checked on the host are checked before anything is
 *     enqueued; a failed check returns a negative MOEDISP_ERR_* code and
 *     enqueues nothing.  A failed launch returns MOEDISP_ERR_HIP.  Problems
 *     only visible in device data (bad expert ids, an inconsistent layout or
 *     handle) set bits of a status word in `ws`, read by ep_check_status.
 *     The library never asserts or aborts.
 *   - Calls that share one `ws` must be ordered on one stream; concurrent
 *     calls need distinct workspaces.
 */
#ifndef MOEDISP_H
#define MOEDISP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of token rows. */
typedef enum {
    MOEDISP_BF16 = 0,      /* bfloat16, 2 bytes */
    MOEDISP_FP8_E4M3 = 1,  /* OCP e4m3fn codes, 1 byte, with fp32 scales per block */
    MOEDISP_FP32 = 2       /* float32 (combine output only) */
} moedisp_dtype;

/* Scale formats of quantise-on-dispatch (ep_dispatch_quant). */
typedef enum {
    MOEDISP_SCALE_FP32 = 0,  /* one binary32 scale per block */
    MOEDISP_SCALE_UE8M0 = 1  /* one byte per block: the scale is 2^(byte - 127) */
} moedisp_scale_fmt;

/* Problem shape.  T tokens of H elements, E experts in G groups (E % G == 0,
 * group of expert e = e / (E/G)), top-k slots per token. */
typedef struct {
    int32_t num_tokens;   /* T >= 0 */
    int32_t hidden;       /* H > 0 */
    int32_t num_experts;  /* E in [1, 4096] */
    int32_t num_groups;   /* G in [1, 32], E % G == 0 */
    int32_t topk;         /* k in [1, 32], k <= E */
    int32_t x_dtype;      /* MOEDISP_BF16 or MOEDISP_FP8_E4M3 */
    int32_t scale_block;  /* 0 for bf16; for fp8 the channels per fp32 scale (H % scale_block == 0) */
} moedisp_shape;

/* Host-side return codes. */
#define MOEDISP_OK 0
#define MOEDISP_ERR_INVALID_ARG (-1)          /* null pointer, negative size, E % G != 0, ... */
#define MOEDISP_ERR_UNSUPPORTED (-2)          /* a limit above exceeded, row not whole 16-B units,
                                                T*k >= 2^30, or a launch grid of 2^32 work-items or
                                                more (T*H beyond about 2^35); nothing is launched */
#define MOEDISP_ERR_MISALIGNED (-3)           /* pointer alignment rule broken */
#define MOEDISP_ERR_WORKSPACE_TOO_SMALL (-4)  /* ws_bytes < ep_workspace_bytes(shape) */
#define MOEDISP_ERR_HIP (-5)                  /* a HIP runtime call or launch failed */

/* Device status bits (ep_check_status). */
#define MOEDISP_DEV_BAD_EXPERT_ID 1u     /* id outside {-1} U [0,E); that slot is treated as masked */
#define MOEDISP_DEV_DUPLICATE_EXPERT 2u  /* an expert repeated within one token (each copy still routed) */
#define MOEDISP_DEV_BAD_LAYOUT 4u        /* tokens_per_expert disagrees with topk_idx; bad rows skipped */
#define MOEDISP_DEV_BAD_HANDLE 8u        /* combine handle inconsistent; those slots skipped */
#define MOEDISP_DEV_EXPERT_OVERFLOW 16u  /* padded layout: an expert got more slots than its capacity;
                                            the extra slots get no row (slot_to_row -1) */

/* Bytes of workspace the calls need for `shape`; 0 if the shape is invalid.
 * One workspace serves every call of that shape, and of any other shape whose
 * ep_workspace_bytes is not larger (calls check this and return
 * MOEDISP_ERR_WORKSPACE_TOO_SMALL otherwise). */
size_t ep_workspace_bytes(const moedisp_shape* shape);

/* Zero a workspace before its first use.  The calls keep its counters
 * consistent afterwards; a workspace must not be shared by overlapping calls. */
int ep_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Layout ("counts + token-in-rank" of the high-throughput layout kernel).
 *   topk_idx           int32 [T][k]: expert per slot, -1 = masked slot.
 *   tokens_per_expert  int32 [E]: number of routed slots with that expert.
 *   tokens_per_group   int32 [G]: number of tokens with at least one routed
 *                      slot in the group (a token counts once per group).
 *   is_token_in_group  uint32 [T]: bit g set iff the token reaches group g.
 * Status bits: BAD_EXPERT_ID, DUPLICATE_EXPERT. */
int ep_get_dispatch_layout(const moedisp_shape* shape, const int32_t* topk_idx,
                           int32_t* tokens_per_expert, int32_t* tokens_per_group,
                           uint32_t* is_token_in_group, void* ws, size_t ws_bytes, void* stream);

/* Dispatch: pack every routed copy of a token into its expert's contiguous
 * receive rows.  Expert e owns rows [expert_offsets[e], expert_offsets[e+1]);
 * inside them rows follow token order.  Row of slot (t,j) with expert e:
 *   expert_offsets[e] + #{t' < t : some slot of t' routes to e}.
 *   x                  [T][H] bf16 or fp8 codes (bytes are copied unchanged).
 *   x_scales           fp32 [T][H/scale_block] for fp8, NULL for bf16.
 *   topk_idx, topk_weights  int32 / fp32 [T][k].
 *   tokens_per_expert  int32 [E] from ep_get_dispatch_layout for this topk_idx.
 *   recv_x             [T*k][H] capacity; rows >= R = expert_offsets[E] untouched.
 *   recv_scales        fp32 [T*k][H/scale_block] for fp8, NULL for bf16.
 *   recv_src_idx       int32 [T*k]: source token of each received row.
 *   recv_weights       fp32 [T*k]: topk_weights[t][j] of each received row.
 *   expert_offsets     int32 [E+1]: exclusive prefix of tokens_per_expert; [E] = R.
 *   slot_to_row        int32 [T][k]: row of each slot, -1 if masked.
 * (recv_src_idx, recv_weights, slot_to_row) is the handle ep_combine takes.
 * Status bits: BAD_EXPERT_ID, BAD_LAYOUT. */
int ep_dispatch(const moedisp_shape* shape, const void* x, const float* x_scales,
                const int32_t* topk_idx, const float* topk_weights,
                const int32_t* tokens_per_expert, void* recv_x, float* recv_scales,
                int32_t* recv_src_idx, float* recv_weights, int32_t* expert_offsets,
                int32_t* slot_to_row, void* ws, size_t ws_bytes, void* stream);

/* ep_dispatch for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same kernels, with the workspace in a static device array of the library
 * (8 MiB, one per device, held until the process ends) instead of `ws`: the
 * call allocates nothing, and the caller passes only inputs and outputs.
 * Shapes whose ep_workspace_bytes exceeds 8 MiB return
 * MOEDISP_ERR_WORKSPACE_TOO_SMALL before any HIP call (at H = 7168, E = 256,
 * G = 8, k = 8 every T up to 345856 fits).  The current device must be the stream's.
 * Arguments as for ep_dispatch, except:
 *   status  int32 [1], device: overwritten with this call's status bits
 *           (BAD_EXPERT_ID, BAD_LAYOUT), ready when the stream reaches the
 *           end of the call; read it with an ordinary copy.
 * All calls on one device share its array: calls that overlap on one device
 * (two streams, two threads) race and may return wrong rows. */
int ep_dispatch_noalloc(const moedisp_shape* shape, const void* x, const float* x_scales,
                        const int32_t* topk_idx, const float* topk_weights, const int32_t* tokens_per_expert,
                        void* recv_x, float* recv_scales, int32_t* recv_src_idx, float* recv_weights,
                        int32_t* expert_offsets, int32_t* slot_to_row, int32_t* status, void* stream);

/* The two phases of ep_dispatch, for callers that time or schedule them
 * apart (the page's high-throughput path likewise separates notify_dispatch,
 * which exchanges counts, from dispatch, which moves rows).
 * ep_dispatch_notify: per-tile expert counts of topk_idx (kept in `ws`) and
 *   expert_offsets[E+1] (exclusive scan of tokens_per_expert).
 * ep_dispatch_scatter: everything else ep_dispatch writes; it reads the counts
 *   and expert_offsets that ep_dispatch_notify left for the same topk_idx and
 *   tokens_per_expert in the same `ws` (stream-ordered before it, with no
 *   other dispatch-family call on that `ws` in between: those reuse the
 *   same workspace tables).
 * Arguments, layouts and status bits as for ep_dispatch. */
int ep_dispatch_notify(const moedisp_shape* shape, const int32_t* topk_idx, const int32_t* tokens_per_expert,
                       int32_t* expert_offsets, void* ws, size_t ws_bytes, void* stream);
int ep_dispatch_scatter(const moedisp_shape* shape, const void* x, const float* x_scales,
                        const int32_t* topk_idx, const float* topk_weights,
                        const int32_t* tokens_per_expert, void* recv_x, float* recv_scales,
                        int32_t* recv_src_idx, float* recv_weights, const int32_t* expert_offsets,
                        int32_t* slot_to_row, void* ws, size_t ws_bytes, void* stream);

/* ep_get_dispatch_layout followed by ep_dispatch_notify of the same topk_idx,
 * with exactly their outputs (tokens_per_expert, tokens_per_group,
 * is_token_in_group, expert_offsets, and the per-tile counts that
 * ep_dispatch_scatter reads from `ws`), in the layout's two launches instead
 * of three: the layout workgroups also count their slots per dispatch tile,
 * and the layout's reduce also scans the totals.  Where the dispatch's tiles
 * do not lie inside the layout's workgroups (k that does not divide 1024,
 * very large T) or their counts do not fit in 64 KiB of LDS with the
 * layout's own (large E), it makes the two calls in order.  Arguments and
 * layouts as for the two calls; expert_offsets int32 [E+1].  Status bits:
 * BAD_EXPERT_ID, DUPLICATE_EXPERT, BAD_LAYOUT. */
int ep_get_dispatch_layout_notify(const moedisp_shape* shape, const int32_t* topk_idx,
                                  int32_t* tokens_per_expert, int32_t* tokens_per_group,
                                  uint32_t* is_token_in_group, int32_t* expert_offsets, void* ws,
                                  size_t ws_bytes, void* stream);

/* Small-batch (decode) path: ep_get_dispatch_layout and ep_dispatch in one
 * kernel launch, with exactly their outputs (all of them, bit for bit).  The
 * page's low-latency path is likewise a single kernel tuned for small
 * batches.  Each copy workgroup finds its token's receive rows from one pass
 * of comparisons over the whole topk_idx, so no workgroup waits for another;
 * the work grows with T * (T*k), which bounds the size: T*k <= 8192 and
 * (T*k + 2*E + T) * 4 bytes <= 60 KiB, else MOEDISP_ERR_UNSUPPORTED (use the
 * two calls).  Arguments as for the two calls; tokens_per_expert,
 * tokens_per_group and is_token_in_group are outputs here.  Status bits:
 * BAD_EXPERT_ID, DUPLICATE_EXPERT.  With no host synchronisation and no
 * allocation, the call (and ep_combine after it) can be captured in a HIP
 * graph. */
int ep_layout_dispatch_small(const moedisp_shape* shape, const void* x, const float* x_scales,
                             const int32_t* topk_idx, const float* topk_weights, int32_t* tokens_per_expert,
                             int32_t* tokens_per_group, uint32_t* is_token_in_group, void* recv_x,
                             float* recv_scales, int32_t* recv_src_idx, float* recv_weights,
                             int32_t* expert_offsets, int32_t* slot_to_row, void* ws, size_t ws_bytes,
                             void* stream);

/* Small-batch path with the padded (low-latency) receive layout
 * ("MSCCLPP EP implementation - #852": the commit porting the low-latency
 * kernels gives every expert its own receive slots, sized by a maximum
 * number of dispatched tokens, and signals received counts per expert; a
 * later commit adds a rank-major output option to that path).  Expert e owns
 * the rows [e*expert_stride + row_base, e*expert_stride + row_base +
 * expert_capacity) of receive buffers of E*expert_stride rows; its routed
 * slots take them in ascending slot order (token order), the i-th at
 * e*expert_stride + row_base + i.  A slot past its expert's first
 * expert_capacity gets no row: slot_to_row -1 and status EXPERT_OVERFLOW.
 * Rows no slot takes are not written.  Expert e's received count is
 * min(tokens_per_expert[e], expert_capacity); there are no offsets.  With
 * several sources, source r of N would write its rows at row_base = r*C
 * inside slabs of expert_stride = N*C rows, with no count from any other
 * source needed.
 *   expert_capacity  C >= 0;  row_base >= 0;  row_base + C <= expert_stride;
 *                    E * expert_stride < 2^31 (else INVALID_ARG / UNSUPPORTED)
 *   recv_x           [E*expert_stride][H] (bf16 or fp8 codes), recv_scales
 *                    [E*expert_stride][H/scale_block] for fp8,
 *                    recv_src_idx, recv_weights [E*expert_stride]
 * Other arguments, size limits and status bits as ep_layout_dispatch_small
 * (no expert_offsets).  ep_combine_padded reads these rows back. */
int ep_layout_dispatch_small_padded(const moedisp_shape* shape, int32_t expert_capacity, int32_t expert_stride,
                                    int32_t row_base, const void* x, const float* x_scales,
                                    const int32_t* topk_idx, const float* topk_weights,
                                    int32_t* tokens_per_expert, int32_t* tokens_per_group,
                                    uint32_t* is_token_in_group, void* recv_x, float* recv_scales,
                                    int32_t* recv_src_idx, float* recv_weights, int32_t* slot_to_row, void* ws,
                                    size_t ws_bytes, void* stream);

/* Dispatch with quantisation: as ep_dispatch for a bf16 x, but every
 * received row holds OCP E4M3 codes of the token's row plus one scale per
 * block of `quant_block` channels ("MSCCLPP EP implementation - #852": the
 * PR's commit messages give its low-latency dispatch E4M3 payloads with FP32
 * scales per block of 32 elements, then UE8M0 scale bytes per block, and keep
 * tiny nonzero blocks nonzero at UE8M0 code zero; the review file table lists
 * the E4M3 quantization helpers of that dispatch).  Per block, with amax the
 * largest |x| of its channels:
 *   MOEDISP_SCALE_FP32:  scale = amax / 448 (binary32; 1 for an all-zero
 *                        block); code = E4M3(x / scale), the quotient
 *                        correctly rounded to binary32;
 *   MOEDISP_SCALE_UE8M0: scale = 2^s, s the smallest integer with
 *                        448 * 2^s >= amax, clamped to [-127, 127] (0 for an
 *                        all-zero block), stored as the byte s + 127;
 *                        code = E4M3(x * 2^-s);
 * E4M3(v) is the nearest e4m3fn value, ties to even, saturating at +-448;
 * signs (of zeros too) are kept.  x must be finite.
 *   shape          x_dtype MOEDISP_BF16, scale_block 0.
 *   quant_block    channels per scale: a power of two in [32, 1024] dividing H.
 *   scale_fmt      MOEDISP_SCALE_FP32 or MOEDISP_SCALE_UE8M0.
 *   recv_x         uint8 [T*k][H] E4M3 codes (16-byte aligned).
 *   recv_scales    [T*k][H/quant_block]: float (4-byte aligned) or uint8.
 * The other arguments, the handle and the status bits are those of
 * ep_dispatch; the received rows are in the same order.  Unsupported
 * quant_block or scale_fmt: MOEDISP_ERR_UNSUPPORTED; a block that does not
 * divide H: MOEDISP_ERR_INVALID_ARG.
 * ep_dispatch_scatter_quant is its second phase, after ep_dispatch_notify of
 * the same shape, topk_idx and tokens_per_expert in the same `ws`. */
int ep_dispatch_quant(const moedisp_shape* shape, int32_t quant_block, int32_t scale_fmt, const void* x,
                      const int32_t* topk_idx, const float* topk_weights, const int32_t* tokens_per_expert,
                      void* recv_x, void* recv_scales, int32_t* recv_src_idx, float* recv_weights,
                      int32_t* expert_offsets, int32_t* slot_to_row, void* ws, size_t ws_bytes, void* stream);
int ep_dispatch_scatter_quant(const moedisp_shape* shape, int32_t quant_block, int32_t scale_fmt,
                              const void* x, const int32_t* topk_idx, const float* topk_weights,
                              const int32_t* tokens_per_expert, void* recv_x, void* recv_scales,
                              int32_t* recv_src_idx, float* recv_weights, const int32_t* expert_offsets,
                              int32_t* slot_to_row, void* ws, size_t ws_bytes, void* stream);

/* Group-deduplicated (high-throughput) path.  "MSCCLPP EP implementation -
 * #852": in the high-throughput path the layout's token-in-rank flags decide
 * which ranks receive a token, each such rank receives it once (the bench
 * commits describe the receiver's layout as one row per (token, source rank)
 * pair), and the receiver orders its rows by local expert.  A rank is a
 * destination group here; rows of group g are what GPU g would receive.
 *
 * ep_dispatch_groups: one row per (token, group it reaches), group by group,
 * tokens in order.  Row of (t, g):
 *   group_offsets[g] + #{t' < t : bit g of is_token_in_group[t'] is set}.
 *   is_token_in_group  uint32 [T] and tokens_per_group int32 [G] from
 *                      ep_get_dispatch_layout of the same topk_idx (bits >= G
 *                      are ignored).
 *   recv_x             [T*min(G,k)][H] capacity (bf16 or fp8 bytes, copied).
 *   recv_scales        fp32 [T*min(G,k)][H/scale_block] for fp8, NULL for bf16.
 *   recv_src_idx       int32 [T*min(G,k)]: source token of each row.
 *   recv_topk_idx      int32 [T*min(G,k)][k]: the token's slot j expert where
 *                      that expert lies in the row's group, else -1 (global ids).
 *   recv_topk_weights  fp32 [T*min(G,k)][k]: topk_weights[t][j] where
 *                      recv_topk_idx >= 0, else 0.
 *   group_offsets      int32 [G+1]: exclusive prefix of tokens_per_group;
 *                      [G] = R_g, the number of group rows.
 *   token_group_row    int32 [T][G]: row of (t, g), -1 if t does not reach g.
 * Rows at or past R_g get recv_topk_idx = -1 (all k slots) and are otherwise
 * not written.  Status bits: BAD_LAYOUT.
 *
 * ep_group_permute: the local expert permutation of the group rows, i.e.
 * ep_dispatch applied to the T*min(G,k) group rows as tokens, with
 * recv_topk_idx / recv_topk_weights as their routing and the layout's
 * tokens_per_expert (rows past R_g hold recv_topk_idx = -1, as
 * ep_dispatch_groups leaves them, and route nothing).  Its outputs equal
 * ep_dispatch's for the original tokens byte for byte (expert_offsets,
 * recv_x, recv_scales, recv_weights), except that recv_src_idx names the group
 * row and slot_to_row is [T*min(G,k)][k] over group rows.  recv_x and the
 * other receive buffers hold T*k rows.
 *
 * ep_group_reduce: each group row's weighted sum of its expert outputs, i.e.
 * ep_combine over the group rows through ep_group_permute's handle; rows at or
 * past group_offsets[G] (read on the device) are skipped.
 *   group_out  [T*min(G,k)][H] bf16 or fp32 (out_dtype).
 *
 * ep_combine_groups: out[t][h] = sum over g ascending with
 * token_group_row[t][g] >= 0 of group_rows[that row][h] (bf16), accumulated in
 * fp32 from 0; bf16 output is that sum rounded once to nearest-even.
 *   recv_src_idx  ep_dispatch_groups' recv_src_idx (checks the handle) or NULL.
 * Status bits of the last three: those of ep_dispatch / ep_combine. */
int ep_dispatch_groups(const moedisp_shape* shape, const void* x, const float* x_scales,
                       const int32_t* topk_idx, const float* topk_weights,
                       const uint32_t* is_token_in_group, const int32_t* tokens_per_group, void* recv_x,
                       float* recv_scales, int32_t* recv_src_idx, int32_t* recv_topk_idx,
                       float* recv_topk_weights, int32_t* group_offsets, int32_t* token_group_row,
                       void* ws, size_t ws_bytes, void* stream);
int ep_group_permute(const moedisp_shape* shape, const void* group_x, const float* group_scales,
                     const int32_t* recv_topk_idx, const float* recv_topk_weights,
                     const int32_t* tokens_per_expert, void* recv_x, float* recv_scales,
                     int32_t* recv_src_idx, float* recv_weights, int32_t* expert_offsets,
                     int32_t* slot_to_row, void* ws, size_t ws_bytes, void* stream);
int ep_group_reduce(const moedisp_shape* shape, const void* expert_out, const int32_t* recv_src_idx,
                    const float* recv_weights, const int32_t* slot_to_row, const int32_t* group_offsets,
                    void* group_out, int32_t out_dtype, void* ws, size_t ws_bytes, void* stream);
int ep_combine_groups(const moedisp_shape* shape, const void* group_rows, const int32_t* recv_src_idx,
                      const int32_t* token_group_row, void* out, int32_t out_dtype, void* ws,
                      size_t ws_bytes, void* stream);

/* Combine: the reverse of dispatch through its handle.
 *   out[t][h] = sum over j = 0..k-1 in ascending order, skipping masked slots,
 *               of recv_weights[r] * expert_out[r][h] with r = slot_to_row[t][j],
 *   accumulated in fp32 by fused multiply-add from 0; bf16 output is that sum
 *   rounded once to nearest-even; a token with no routed slot gets +0.
 *   expert_out    bf16 [T*k][H] (rows [0,R) are read).
 *   recv_src_idx  may be NULL; if given, each slot's row must name its token.
 *   out           [T][H] bf16 (out_dtype MOEDISP_BF16) or fp32 (MOEDISP_FP32).
 * Status bits: BAD_HANDLE. */
int ep_combine(const moedisp_shape* shape, const void* expert_out, const int32_t* recv_src_idx,
               const float* recv_weights, const int32_t* slot_to_row, void* out,
               int32_t out_dtype, void* ws, size_t ws_bytes, void* stream);

/* ep_combine over the padded layout of ep_layout_dispatch_small_padded: the
 * same sum, with expert_out bf16 [E*expert_stride][H] and slot_to_row,
 * recv_weights (and recv_src_idx, if given) from that call.  Status bits:
 * BAD_HANDLE (a row outside the E*expert_stride rows, or naming another
 * token). */
int ep_combine_padded(const moedisp_shape* shape, int32_t expert_stride, const void* expert_out,
                      const int32_t* recv_src_idx, const float* recv_weights, const int32_t* slot_to_row,
                      void* out, int32_t out_dtype, void* ws, size_t ws_bytes, void* stream);

/* Wait for `stream`, then return the device status bits accumulated in `ws`
 * since the last check in *host_status and clear them. */
int ep_check_status(void* ws, size_t ws_bytes, void* stream, int32_t* host_status);

/* Text for a host return code. */
const char* ep_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOEDISP_H */
