/*
 * CPU oracle for one GPU's share of MoE expert-parallel
 * get_dispatch_layout -> dispatch -> combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this code; the library under test never
 * does.  It is plain, single-threaded C++17 (in its C subset: loops, arrays
 * and the C math library, no templates or containers) written straight from
 * the definitions, shares no source with the GPU path, and is meant to be
 * checked by eye against the passages cited below.  Every function is
 * exported with C linkage for the ctypes loader.
 *
 * Source: "MSCCLPP EP implementation - #852" (MSCCL++ pull request page).
 *   - PR description, "Scope": the layout call, intranode dispatch and
 *     intranode combine are the three operations of the path.
 *   - Review file table, entry for the high-throughput layout kernel: the
 *     layout produces token counts and the token-in-rank flags.
 *   - Commit message fixing internode combine: combine runs in the reverse
 *     direction of dispatch and consumes the receiver-side bookkeeping that
 *     dispatch returned (the "handle").
 *   - Commit message on combine byte accounting: each expert returns one copy
 *     per dispatched token, so combine reads one row per routed copy.
 *   - Commit messages on warp geometry and the review's code-scanning excerpt:
 *     hidden rows move in 16-byte units.
 *
 * Readings where the page is silent (each is a documented choice):
 *   - a "rank" of the page is a destination group g of this GPU; expert e
 *     belongs to group e / (E/G) (equal, contiguous expert blocks per rank);
 *   - tokens_per_group counts a token once per group it reaches;
 *   - is_token_in_group is one uint32 per token, bit g;
 *   - a masked slot holds -1; any other id outside [0,E) is an error and the
 *     slot is treated as masked;
 *   - received rows are ordered by (expert, token, slot) ascending: each
 *     expert's rows are contiguous and stable in token order;
 *   - recv_src_idx holds the source token index;
 *   - combine sums slots j = 0..k-1 in ascending order with fp32 fused
 *     multiply-add, then rounds once to bf16 (nearest, ties to even); a token
 *     whose every slot is masked gets +0.
 *
 * Quantise-on-dispatch (same page: the commit messages that give the
 * low-latency dispatch E4M3 payloads with FP32 scales per 32 elements, then
 * UE8M0 scale bytes per 32 elements, and that keep tiny nonzero MXFP8 blocks
 * alive at UE8M0 code zero; the review file table's FP8 E4M3 quantization
 * helpers for that dispatch).  The page prints no formula; the readings are:
 *   - payload codes are OCP E4M3 ("e4m3fn": bias 7, 3 fraction bits, no
 *     infinity, largest finite 448);
 *   - a block is B consecutive channels of one token; amax is the largest
 *     |x| in it;
 *   - FP32 scales: scale = amax / 448 rounded to binary32 (1 for an all-zero
 *     block); each element is x / scale rounded to binary32, then to the
 *     nearest E4M3 value, ties to even, magnitudes beyond 448 saturating;
 *   - UE8M0 scales: scale = 2^s with s the smallest integer for which
 *     448 * 2^s >= amax, clamped to [-127, 127] (s = 0 for an all-zero
 *     block); the scale byte is s + 127; each element is x * 2^-s rounded to
 *     binary32 (exact unless far below the E4M3 range), then to E4M3 as above.
 *     Clamping at -127 (code zero) keeps tiny nonzero blocks nonzero.
 *
 * Error codes (bit mask, same meaning as the library's device status bits):
 *   1  an expert id outside {-1} U [0,E)      (slot treated as masked)
 *   2  an expert id repeated within one token  (each copy is its own slot)
 *  16  padded layout only: an expert received more routed slots than its
 *      capacity (the extra slots get no row)
 *  -1  bad shape argument
 *
 * Padded (low-latency) layout (same page: the commit porting the
 * low-latency kernels, whose dispatch signals received counts per expert into
 * per-expert receive slots sized by a maximum token count, and the later
 * commit adding a rank-major output option to that path).  Reading, for one
 * source: expert e owns the C receive rows [e*S + B, e*S + B + C) of a buffer
 * of E*S rows (S >= B + C); its routed slots take them in ascending slot
 * order (token order), the i-th at row e*S + B + i; slots past an expert's
 * first C get no row (slot_to_row -1) and status 16.  Rows of the buffer that
 * no slot takes are left untouched.  With several sources, source r would
 * take B = r*C inside slabs of S = (sources)*C rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

extern "C" {

#define ORACLE_ERR_BAD_EXPERT 1
#define ORACLE_ERR_DUP_EXPERT 2
#define ORACLE_ERR_OVERFLOW 16

/* ------------------------------------------------------------------------ */
/* bf16 <-> binary32.                                                        */
/* bf16 is the upper half of an IEEE binary32: sign, 8 exponent bits and 7   */
/* fraction bits.                                                            */
/* ------------------------------------------------------------------------ */

double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a binary32 value to the nearest bf16 value, ties to even.
 * The bf16 grid near |v| in [2^(p-1), 2^p) is spaced 2^(p-8) (8 significant
 * bits); below the smallest normal 2^-126 the spacing stays 2^-133.  The value
 * is divided by the spacing (exact: a power of two), rounded to an integer
 * with rint() in the default round-to-nearest-even mode, and scaled back.
 * A result of 2^128 or more is +-infinity; NaN maps to the quiet NaN 0x7FC0
 * with the input's sign. */
uint16_t oracle_f32_to_bf16(float v)
{
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    if (isinf(v)) return (uint16_t)(sign | 0x7F80u);
    double d = fabs((double)v);
    if (d == 0.0) return sign;
    int p;
    frexp(d, &p);                 /* d in [2^(p-1), 2^p) */
    if (p < -125) p = -125;       /* subnormal range keeps the 2^-133 spacing */
    double spacing = ldexp(1.0, p - 8);
    double r = rint(d / spacing) * spacing;
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    float rf = (float)r;          /* exact: r is a bf16 value */
    uint32_t ru;
    memcpy(&ru, &rf, sizeof ru);
    return (uint16_t)(sign | (ru >> 16));
}

/* Vector helpers for the harness (convert arrays element by element). */
void oracle_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(in[i]);
}

/* ------------------------------------------------------------------------ */
/* validation                                                               */
/* ------------------------------------------------------------------------ */

static int bad_shape(int T, int k, int E, int G)
{
    if (T < 0 || k < 1 || k > 32 || E < 1 || G < 1 || G > 32) return 1;
    if (E % G != 0) return 1;
    return 0;
}

/* Is slot (t,j) routed, i.e. does it hold an id in [0,E)? */
static int routed(int32_t id, int E) { return id >= 0 && id < E; }

/* Status bits for the routing table: ids out of range and repeats. */
static int routing_status(int T, int k, int E, const int32_t* topk_idx)
{
    int st = 0;
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int32_t id = topk_idx[(int64_t)t * k + j];
            if (id != -1 && !routed(id, E)) st |= ORACLE_ERR_BAD_EXPERT;
            if (!routed(id, E)) continue;
            for (int jj = 0; jj < j; ++jj)
                if (topk_idx[(int64_t)t * k + jj] == id) st |= ORACLE_ERR_DUP_EXPERT;
        }
    }
    return st;
}

/* ------------------------------------------------------------------------ */
/* layout: tokens per expert, tokens per group, token-in-group bitmap        */
/* ------------------------------------------------------------------------ */

int oracle_layout(int T, int k, int E, int G, const int32_t* topk_idx,
                  int32_t* tokens_per_expert, int32_t* tokens_per_group,
                  uint32_t* is_token_in_group)
{
    if (bad_shape(T, k, E, G)) return -1;
    int experts_per_group = E / G;

    /* tokens_per_expert[e] = number of slots (t,j) whose id is e */
    for (int e = 0; e < E; ++e) tokens_per_expert[e] = 0;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int32_t id = topk_idx[(int64_t)t * k + j];
            if (routed(id, E)) tokens_per_expert[id] += 1;
        }

    /* bit g of is_token_in_group[t] = some routed slot of t lands in group g */
    for (int t = 0; t < T; ++t) {
        uint32_t bits = 0;
        for (int j = 0; j < k; ++j) {
            int32_t id = topk_idx[(int64_t)t * k + j];
            if (routed(id, E)) bits |= 1u << (id / experts_per_group);
        }
        is_token_in_group[t] = bits;
    }

    /* tokens_per_group[g] = number of tokens with bit g set */
    for (int g = 0; g < G; ++g) {
        int32_t c = 0;
        for (int t = 0; t < T; ++t) c += (int32_t)((is_token_in_group[t] >> g) & 1u);
        tokens_per_group[g] = c;
    }
    return routing_status(T, k, E, topk_idx);
}

/* ------------------------------------------------------------------------ */
/* dispatch: pack every routed copy into per-expert receive rows             */
/* ------------------------------------------------------------------------ */

/* x: [T][row_bytes] raw row bytes (bf16 or fp8 codes; copied, never read as
 * numbers).  x_scales: [T][scale_row_bytes] or NULL.  Outputs have capacity
 * T*k rows; rows at or past R = expert_offsets[E] are left untouched. */
int oracle_dispatch(int T, int k, int E, int64_t row_bytes, int64_t scale_row_bytes,
                    const uint8_t* x, const uint8_t* x_scales,
                    const int32_t* topk_idx, const float* topk_weights,
                    uint8_t* recv_x, uint8_t* recv_scales,
                    int32_t* recv_src_idx, float* recv_weights,
                    int32_t* expert_offsets, int32_t* slot_to_row)
{
    if (T < 0 || k < 1 || k > 32 || E < 1 || row_bytes < 0 || scale_row_bytes < 0) return -1;

    /* counts and exclusive prefix: expert e owns rows [off[e], off[e+1]) */
    int64_t* cursor = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    if (!cursor) return -1;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int32_t id = topk_idx[(int64_t)t * k + j];
            if (routed(id, E)) cursor[id] += 1;
        }
    int64_t run = 0;
    for (int e = 0; e < E; ++e) {
        int64_t c = cursor[e];
        expert_offsets[e] = (int32_t)run;
        cursor[e] = run;
        run += c;
    }
    expert_offsets[E] = (int32_t)run;

    /* visit slots in (t, j) order; each expert's cursor hands out its rows in
     * that order, so an expert's rows are stable in token order */
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int64_t s = (int64_t)t * k + j;
            int32_t id = topk_idx[s];
            if (!routed(id, E)) {
                slot_to_row[s] = -1;
                continue;
            }
            int64_t r = cursor[id]++;
            memcpy(recv_x + r * row_bytes, x + (int64_t)t * row_bytes, (size_t)row_bytes);
            if (x_scales && recv_scales && scale_row_bytes > 0)
                memcpy(recv_scales + r * scale_row_bytes, x_scales + (int64_t)t * scale_row_bytes,
                       (size_t)scale_row_bytes);
            recv_src_idx[r] = t;
            recv_weights[r] = topk_weights[s];
            slot_to_row[s] = (int32_t)r;
        }
    }
    free(cursor);
    return routing_status(T, k, E, topk_idx);
}

/* ------------------------------------------------------------------------ */
/* padded (low-latency) dispatch: fixed receive slots per expert              */
/* ------------------------------------------------------------------------ */

/* Arguments as oracle_dispatch, plus the per-expert capacity C, the slab
 * stride S and the first row B of this source inside each slab.  recv_x,
 * recv_scales, recv_src_idx and recv_weights have E*S rows.  No offsets are
 * returned: expert e's rows start at e*S + B, and its received count is
 * min(its routed slots, C). */
int oracle_dispatch_padded(int T, int k, int E, int C, int64_t S, int64_t B, int64_t row_bytes,
                           int64_t scale_row_bytes, const uint8_t* x, const uint8_t* x_scales,
                           const int32_t* topk_idx, const float* topk_weights,
                           uint8_t* recv_x, uint8_t* recv_scales,
                           int32_t* recv_src_idx, float* recv_weights, int32_t* slot_to_row)
{
    if (T < 0 || k < 1 || k > 32 || E < 1 || C < 0 || B < 0 || S < 1 || B + C > S || row_bytes < 0 ||
        scale_row_bytes < 0)
        return -1;
    /* how many of each expert's slots have been placed so far */
    int64_t* placed = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    if (!placed) return -1;
    int st = 0;
    /* slots in ascending order s = t*k + j, i.e. token by token */
    for (int64_t s = 0; s < (int64_t)T * k; ++s) {
        int t = (int)(s / k);
        int32_t id = topk_idx[s];
        if (!routed(id, E)) {
            slot_to_row[s] = -1;
            continue;
        }
        int64_t i = placed[id]++;
        if (i >= C) {
            slot_to_row[s] = -1;
            st |= ORACLE_ERR_OVERFLOW;
            continue;
        }
        int64_t q = (int64_t)id * S + B + i;
        const uint8_t* src_row = x + (int64_t)t * row_bytes;
        memcpy(recv_x + q * row_bytes, src_row, (size_t)row_bytes);
        if (x_scales && recv_scales && scale_row_bytes > 0)
            memcpy(recv_scales + q * scale_row_bytes, x_scales + (int64_t)t * scale_row_bytes,
                   (size_t)scale_row_bytes);
        recv_src_idx[q] = (int32_t)t;
        recv_weights[q] = topk_weights[s];
        slot_to_row[s] = (int32_t)q;
    }
    free(placed);
    return st | routing_status(T, k, E, topk_idx);
}

/* ------------------------------------------------------------------------ */
/* combine: weighted top-k sum of the expert outputs, per token               */
/* ------------------------------------------------------------------------ */

/* expert_out: bf16 [R][H]; recv_weights: [R]; slot_to_row: [T][k] (-1 masked).
 * out[t][h] = sum over j = 0..k-1 (ascending) of recv_weights[r] * expert_out[r][h]
 * with r = slot_to_row[t][j] >= 0, accumulated in fp32 by fused multiply-add
 * from 0.0f.  out_f32 receives the fp32 sum, out_bf16 its bf16 rounding;
 * either may be NULL. */
int oracle_combine(int T, int k, int H, int64_t R, const uint16_t* expert_out,
                   const float* recv_weights, const int32_t* slot_to_row,
                   float* out_f32, uint16_t* out_bf16)
{
    if (T < 0 || k < 1 || H < 0 || R < 0) return -1;
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                int32_t r = slot_to_row[(int64_t)t * k + j];
                if (r < 0) continue;
                if ((int64_t)r >= R) return -1;
                float v = (float)oracle_bf16_to_double(expert_out[(int64_t)r * H + h]);
                acc = fmaf(recv_weights[r], v, acc);
            }
            if (out_f32) out_f32[(int64_t)t * H + h] = acc;
            if (out_bf16) out_bf16[(int64_t)t * H + h] = oracle_f32_to_bf16(acc);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* E4M3 (OCP e4m3fn) codes                                                   */
/* Code bits: sign, 4 exponent bits e, 3 fraction bits f.                    */
/*   e >= 1: (1 + f/8) * 2^(e-7);  e = 0: (f/8) * 2^-6;  e = 15, f = 7: NaN. */
/* ------------------------------------------------------------------------ */

double oracle_e4m3_to_double(uint8_t c)
{
    int e = (c >> 3) & 15, f = c & 7;
    double mag;
    if (e == 15 && f == 7) return NAN;
    if (e == 0)
        mag = ldexp(f / 8.0, -6);
    else
        mag = ldexp(1.0 + f / 8.0, e - 7);
    return (c & 0x80) ? -mag : mag;
}

/* Nearest E4M3 value, ties to the even code, |v| beyond 448 saturating to
 * +-448.  The E4M3 grid near |v| in [2^p, 2^(p+1)) is spaced 2^(p-3); below
 * 2^-6 (subnormals) it stays 2^-9.  |v| is divided by the spacing (exact), rounded
 * to an integer by rint() (nearest-even) and scaled back; the encoding of the
 * result then follows from the definition above.  The sign is kept, so a
 * negative value that rounds to zero gives the code 0x80.  NaN gives 0x7F
 * with its sign. */
uint8_t oracle_f32_to_e4m3(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    if (a == 0.0) return sign;
    int p;
    frexp(a, &p);                 /* a in [2^(p-1), 2^p) */
    int lo = p - 1;               /* a in [2^lo, 2^(lo+1)) */
    if (lo < -6) lo = -6;         /* subnormal range keeps the 2^-9 spacing */
    double spacing = ldexp(1.0, lo - 3);
    double r = rint(a / spacing) * spacing;
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -6)) return (uint8_t)(sign | (uint8_t)(r / ldexp(1.0, -9)));
    int q;
    frexp(r, &q);                 /* r in [2^(q-1), 2^q) */
    int ex = q - 1;
    int f = (int)((r / ldexp(1.0, ex) - 1.0) * 8.0);
    return (uint8_t)(sign | (uint8_t)(((ex + 7) << 3) | f));
}

void oracle_f32_to_e4m3_array(const float* in, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_e4m3(in[i]);
}

void oracle_e4m3_to_double_array(const uint8_t* in, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_to_double(in[i]);
}

/* UE8M0 exponent of a block: the smallest s in [-127, 127] with
 * 448 * 2^s >= amax; 0 for amax == 0.  amax is a finite binary32 >= 0. */
int oracle_ue8m0_exponent(float amax)
{
    if (amax == 0.0f) return 0;
    int s = -127;
    while (s < 127 && ldexp(448.0, s) < (double)amax) ++s;
    return s;
}

#define ORACLE_SCALE_FP32 0
#define ORACLE_SCALE_UE8M0 1

/* Quantise T rows of H bf16 values in blocks of B channels.
 * q: E4M3 codes [T][H].  scales: fp32 [T][H/B] (fmt 0) or UE8M0 bytes
 * [T][H/B] (fmt 1).  Returns 0, or -1 for bad arguments. */
int oracle_quant_rows(int T, int H, int B, int fmt, const uint16_t* x, uint8_t* q, uint8_t* scales)
{
    if (T < 0 || H <= 0 || B <= 0 || H % B != 0) return -1;
    if (fmt != ORACLE_SCALE_FP32 && fmt != ORACLE_SCALE_UE8M0) return -1;
    int nb = H / B;
    for (int t = 0; t < T; ++t) {
        for (int b = 0; b < nb; ++b) {
            const uint16_t* xb = x + (int64_t)t * H + (int64_t)b * B;
            uint8_t* qb = q + (int64_t)t * H + (int64_t)b * B;
            float amax = 0.0f;
            for (int i = 0; i < B; ++i) {
                float m = fabsf((float)oracle_bf16_to_double(xb[i]));
                if (m > amax) amax = m;
            }
            if (fmt == ORACLE_SCALE_FP32) {
                float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
                for (int i = 0; i < B; ++i) {
                    float v = (float)oracle_bf16_to_double(xb[i]) / scale;
                    qb[i] = oracle_f32_to_e4m3(v);
                }
                memcpy(scales + ((int64_t)t * nb + b) * 4, &scale, 4);
            } else {
                int sx = oracle_ue8m0_exponent(amax);
                for (int i = 0; i < B; ++i) {
                    float v = ldexpf((float)oracle_bf16_to_double(xb[i]), -sx);
                    qb[i] = oracle_f32_to_e4m3(v);
                }
                scales[(int64_t)t * nb + b] = (uint8_t)(sx + 127);
            }
        }
    }
    return 0;
}

/* Dispatch with quantisation: every token row is quantised once (as
 * oracle_quant_rows), then the codes and the token's scales are dispatched
 * exactly as oracle_dispatch moves rows and scales.  recv_q [T*k][H] codes,
 * recv_scales [T*k][H/B] fp32 or bytes; other outputs and the status as for
 * oracle_dispatch. */
int oracle_dispatch_quant(int T, int k, int E, int H, int B, int fmt,
                          const uint16_t* x, const int32_t* topk_idx, const float* topk_weights,
                          uint8_t* recv_q, uint8_t* recv_scales,
                          int32_t* recv_src_idx, float* recv_weights,
                          int32_t* expert_offsets, int32_t* slot_to_row)
{
    if (T < 0 || H <= 0 || B <= 0 || H % B != 0) return -1;
    int64_t scale_bytes = (int64_t)(H / B) * (fmt == ORACLE_SCALE_FP32 ? 4 : 1);
    uint8_t* q = (uint8_t*)malloc((size_t)T * H + 1);
    uint8_t* sc = (uint8_t*)malloc((size_t)(T * scale_bytes) + 1);
    if (!q || !sc) {
        free(q);
        free(sc);
        return -1;
    }
    int st = oracle_quant_rows(T, H, B, fmt, x, q, sc);
    if (st == 0)
        st = oracle_dispatch(T, k, E, H, scale_bytes, q, sc, topk_idx, topk_weights, recv_q, recv_scales,
                             recv_src_idx, recv_weights, expert_offsets, slot_to_row);
    free(q);
    free(sc);
    return st;
}

/* ------------------------------------------------------------------------ */
/* group-deduplicated dispatch and its combine                               */
/*                                                                           */
/* Same page: in the high-throughput path the layout's token-in-rank flags   */
/* decide which ranks receive a token, each such rank receives it once, and  */
/* the receiver's layout holds one row per (token, source rank) pair (the    */
/* bench commits that change the byte accounting describe that expanded      */
/* receive layout); the receiver then orders rows by its local experts.      */
/* Here a rank is a destination group.  Readings:                            */
/*   - group g's rows are [group_offsets[g], group_offsets[g+1]), one per    */
/*     token whose bit g is set in is_token_in_group, in token order;        */
/*   - each row carries the token index and the token's k slots restricted   */
/*     to the group: the global expert id where the slot's expert lies in    */
/*     g, else -1, and the slot's weight there, else 0;                      */
/*   - token_group_row[t][g] is the row of (t, g), -1 if t does not reach g; */
/*   - the way back: each group row gets the bf16 (nearest-even) rounding of */
/*     its weighted expert sum (fp32 fused multiply-add, ascending slot),    */
/*     and out[t] is the bf16 rounding of the fp32 sum of the token's group  */
/*     rows in ascending g.                                                  */
/* ------------------------------------------------------------------------ */

/* Group-deduplicated dispatch.  is_token_in_group is the layout's bitmap for
 * the same topk_idx (only bits < G are read).  Outputs have capacity
 * T*min(G,k) rows; rows at or past group_offsets[G] are left untouched. */
int oracle_dispatch_groups(int T, int k, int E, int G, int64_t row_bytes, int64_t scale_row_bytes,
                           const uint8_t* x, const uint8_t* x_scales,
                           const int32_t* topk_idx, const float* topk_weights,
                           const uint32_t* is_token_in_group,
                           uint8_t* recv_x, uint8_t* recv_scales, int32_t* recv_src_idx,
                           int32_t* recv_topk_idx, float* recv_topk_weights,
                           int32_t* group_offsets, int32_t* token_group_row)
{
    if (bad_shape(T, k, E, G) || row_bytes < 0 || scale_row_bytes < 0) return -1;
    int experts_per_group = E / G;

    /* rows per group and their exclusive prefix */
    int64_t run = 0;
    for (int g = 0; g < G; ++g) {
        group_offsets[g] = (int32_t)run;
        for (int t = 0; t < T; ++t) run += (is_token_in_group[t] >> g) & 1u;
    }
    group_offsets[G] = (int32_t)run;

    /* group by group, tokens in order */
    for (int g = 0; g < G; ++g) {
        int64_t r = group_offsets[g];
        for (int t = 0; t < T; ++t) {
            if (!((is_token_in_group[t] >> g) & 1u)) {
                token_group_row[(int64_t)t * G + g] = -1;
                continue;
            }
            const uint8_t* row = x + (int64_t)t * row_bytes;
            memcpy(recv_x + r * row_bytes, row, (size_t)row_bytes);
            if (x_scales && recv_scales && scale_row_bytes > 0)
                memcpy(recv_scales + r * scale_row_bytes, x_scales + (int64_t)t * scale_row_bytes,
                       (size_t)scale_row_bytes);
            recv_src_idx[r] = (int32_t)t;
            for (int j = 0; j < k; ++j) {
                int32_t id = topk_idx[(int64_t)t * k + j];
                int here = routed(id, E) && id / experts_per_group == g;
                recv_topk_idx[r * k + j] = here ? id : -1;
                recv_topk_weights[r * k + j] = here ? topk_weights[(int64_t)t * k + j] : 0.0f;
            }
            token_group_row[(int64_t)t * G + g] = (int32_t)r;
            ++r;
        }
    }
    return routing_status(T, k, E, topk_idx);
}

/* Sum of each token's group rows: out[t] = sum over g ascending with
 * token_group_row[t][g] >= 0 of group_rows[that row], accumulated in fp32
 * from 0.0f; out_bf16 is its nearest-even bf16 rounding.  group_rows: bf16
 * [R_g][H].  Either output may be NULL. */
int oracle_combine_groups(int T, int G, int H, int64_t Rg, const uint16_t* group_rows,
                          const int32_t* token_group_row, float* out_f32, uint16_t* out_bf16)
{
    if (T < 0 || G < 1 || H < 0 || Rg < 0) return -1;
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int g = 0; g < G; ++g) {
                int32_t r = token_group_row[(int64_t)t * G + g];
                if (r < 0) continue;
                if ((int64_t)r >= Rg) return -1;
                acc = acc + (float)oracle_bf16_to_double(group_rows[(int64_t)r * H + h]);
            }
            if (out_f32) out_f32[(int64_t)t * H + h] = acc;
            if (out_bf16) out_bf16[(int64_t)t * H + h] = oracle_f32_to_bf16(acc);
        }
    }
    return 0;
}

}  // extern "C"
