// C ABI of libmoedisp: argument checks on the host, then launches on the
// caller's stream.  The checks touch no device and no HIP runtime state, so a
// rejected call enqueues nothing.  Unsupported input is reported as a code,
// never by an assertion (the reviewers of "Add pynccl all-gatherv and
// reducescatterv #20154" ask for a raised error instead of an assert on an
// unsupported argument).
#include <stddef.h>
#include <string.h>

#include <mutex>

#include "moedisp_tools.h"
#include "moedisp_internal.h"

namespace moedisp {

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static int check_shape(const moedisp_shape* s) {
    if (!s) return MOEDISP_ERR_INVALID_ARG;
    if (s->num_tokens < 0 || s->hidden <= 0 || s->num_experts < 1 || s->num_groups < 1 || s->topk < 1)
        return MOEDISP_ERR_INVALID_ARG;
    if (s->num_experts % s->num_groups != 0) return MOEDISP_ERR_INVALID_ARG;
    if (s->topk > s->num_experts) return MOEDISP_ERR_INVALID_ARG;
    if (s->num_groups > kMaxGroups || s->topk > kMaxTopk || s->num_experts > kMaxExperts)
        return MOEDISP_ERR_UNSUPPORTED;
    if (s->x_dtype == MOEDISP_BF16) {
        if (s->scale_block != 0) return MOEDISP_ERR_INVALID_ARG;
    } else if (s->x_dtype == MOEDISP_FP8_E4M3) {
        if (s->scale_block <= 0 || s->hidden % s->scale_block != 0) return MOEDISP_ERR_INVALID_ARG;
    } else {
        return MOEDISP_ERR_UNSUPPORTED;
    }
    if (row_bytes(*s) % 16 != 0) return MOEDISP_ERR_UNSUPPORTED;
    // row byte offsets are 32-bit inside the kernels (buffer descriptors)
    if (row_bytes(*s) >= (1ull << 31)) return MOEDISP_ERR_UNSUPPORTED;
    // receive row indices (T*k of them) are int32 with headroom
    const long long cap = (long long)s->num_tokens * s->topk;
    if (cap >= (1ll << 30)) return MOEDISP_ERR_UNSUPPORTED;
    return MOEDISP_OK;
}

static int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Expert -> group index e / per_group on the device: a shift when per_group is
// a power of two, else a multiply-high by floor(2^32 / per_group) + 1, which
// is exact for e, per_group <= 4096 (the error term e * (per_group - 2^32 mod
// per_group) / (per_group * 2^32) stays below 1 / per_group).
static void group_index_constants(int per_group, int* shift, uint32_t* magic) {
    const uint32_t pg = (uint32_t)per_group;
    *shift = -1;
    *magic = 0;
    if ((pg & (pg - 1)) == 0) {
        *shift = 0;
        while ((1u << *shift) < pg) ++*shift;
    } else {
        *magic = (uint32_t)((1ull << 32) / pg + 1);
    }
}

// Scatter plan for rows of `units` lane units whose k copies write
// `write_per_token` bytes; column ranges are whole multiples of `align` units;
// a lane takes up to `max_per_lane` units per pass; a workgroup copies tokens
// until it stores at least `wg_bytes`.
static DispatchPlan plan_scatter(const moedisp_shape& s, long long write_per_token, int units, int align,
                                 int max_per_lane, long long wg_bytes) {
    DispatchPlan p;
    const int T = s.num_tokens, k = s.topk;
    int bt = 1;
    while (bt < kMaxBlockTokens && write_per_token * bt < wg_bytes && 2 * bt * k <= kMaxDispatchThreads) bt *= 2;
    // count tiles: 16 tokens (>= bt, as bt <= 16), doubled until there are at
    // most kMaxTiles (a slot's row sums one count per earlier tile); this
    // depends only on T and k
    int tt = 16;
    while (tt < bt) tt *= 2;
    while ((long long)tt * kMaxTiles < T && 2 * tt * k <= kMaxTileSlots) tt *= 2;
    p.tile_tokens = tt;
    p.tiles = T > 0 ? ceil_div(T, tt) : 1;
    p.tile_stride = (p.tiles + 3) / 4 * 4;
    // split rows across workgroups while the grid is small (decode-sized T)
    int splits = 1;
    const long long token_blocks = ceil_div(T, bt);
    while (token_blocks * splits < 1024 && units / (splits * 2) >= kThreads / 2) splits *= 2;
    int per = ceil_div(units, splits);
    per = ceil_div(per, align) * align;
    if (per < 1) per = 1;  // rows of no whole unit are rejected by the callers
    p.split_units = per;
    p.col_splits = ceil_div(units, per);
    p.block_tokens = bt;
    // at least one workgroup, so that workgroup 0 runs the total check
    p.blocks = token_blocks > 0 ? (int)(token_blocks * p.col_splits) : 1;
    // lanes: whole waves covering one pass of the column range (up to 1024
    // lanes; wider rows loop), and at least one lane per slot of the
    // workgroup.  A wide range (>= 512 units) takes 2 units per lane where
    // allowed: a 7168-wide bf16 row is then 448 lanes, and smaller workgroups
    // pack the compute units more fully than 896-lane ones.
    const int u = (max_per_lane >= 2 && per >= 2 * kThreads) ? 2 : 1;
    p.units_per_lane = u;
    int threads = ((per + u - 1) / u + 63) / 64 * 64;
    const int slot_lanes = (bt * k + 63) / 64 * 64;
    if (threads < slot_lanes) threads = slot_lanes;
    if (threads < kThreads) threads = kThreads;
    if (threads > kMaxDispatchThreads) threads = kMaxDispatchThreads;
    p.threads = threads;
    return p;
}

// Copy workgroups of one token unless its k rows store less than 16 KiB:
// more tokens per workgroup (the next token's row loaded while this one's is
// stored) measured slower at T = 16384, H = 4096, k = 2 (4 tokens: +1.8 us
// back to back, +14 us with the source rows not in the MALL) and no faster
// at H = 7168, k = 8.
constexpr long long kCopyWorkgroupBytes = 16 * 1024;

DispatchPlan plan_dispatch(const moedisp_shape& s) {
    return plan_scatter(s, (long long)s.topk * (long long)row_bytes(s), (int)(row_bytes(s) / 16), 1, 2,
                        kCopyWorkgroupBytes);
}

// Block-pull copy workgroups: one receive row each, `units` 16-byte units
// per lane.  Measured in the library's cold step (512 MiB read before each)
// at T = 4096, H = 7168, k = 8: 3 units (320 lanes, 5 waves per row) copied
// in 89 us, 2 units (448 lanes) in 94 us, 4 and 5 units (256 and 192 lanes)
// in 98-100 us, 1 unit (896 lanes) in 172 us, and a wave per row (all 14
// units of a lane in one pass, 20 rows per CU in flight) in 103-105 us: the
// more rows a CU writes at once, the further the write stream strays from
// address order, and the fewer, the more each row's dependent loads show.
// With skewed routing (same shape) 3 units took 82.5 against 90.7 us.  Rows
// of at most 512 units (H = 4096 bf16: 72.0 us against 72.8) keep 2 units.
// Two rows per workgroup measured 3 us slower than one.

// Block-pull plan: blocks of tb tokens whose source rows fit one XCD's L2,
// as many blocks as XCDs or a multiple of it (every XCD gets the same number
// of blocks; the last block may be shorter), each block sorted in LDS.
// compact_entries > 0: compact lists (routed entries only) and a copy grid of
// kXcds * wq workgroups sized for that many routed entries plus 1/8 (the
// copy loops where an XCD has more).
PullPlan plan_pull(const moedisp_shape& s, long long compact_entries) {
    PullPlan p;
    memset(&p, 0, sizeof p);
    const long long T = s.num_tokens, k = s.topk, E = s.num_experts;
    const long long rb = (long long)row_bytes(s);
    if (T <= 0 || E > kPullMaxExperts || rb <= 0) return p;
    long long tbmax = kPullL2Bytes / rb;
    if (tbmax > kPullMaxBlockSlots / k) tbmax = kPullMaxBlockSlots / k;
    if (tbmax > 64 * (kPullMaskWords / E)) tbmax = 64 * (kPullMaskWords / E);  // token masks in LDS
    if (tbmax < kPullMinBlockTokens) return p;
    const long long rounds = (T + kXcds * tbmax - 1) / (kXcds * tbmax);
    const long long tb = (T + kXcds * rounds - 1) / (kXcds * rounds);
    const long long nblk = (T + tb - 1) / tb;
    if (tb < kPullMinBlockTokens || nblk < kXcds || nblk > kPullMaxBlocks) return p;
    const int row16 = (int)(rb / 16);
    p.tb = (int)tb;
    p.nblk = (int)nblk;
    p.cap_b = (int)(tb * k);
    p.cnt_stride = (p.nblk + 3) / 4 * 4;
    // compact lists: 4 units per lane (more rows in flight per compute unit)
    p.units = compact_entries > 0 ? kPullCompactUnits : (row16 > 512 ? 3 : 2);
    int threads = ((row16 + p.units - 1) / p.units + 63) / 64 * 64;
    if (threads > kMaxDispatchThreads) threads = kMaxDispatchThreads;
    // an fp8 row's scales travel one per lane with the row
    const int spr = scales_per_row(s);
    if (spr > kMaxDispatchThreads || (compact_entries <= 0 && spr > threads)) return p;
    if (spr > threads) threads = (spr + 63) / 64 * 64;
    p.threads = threads;
    p.rpw = 1;
    p.wpb = (p.cap_b + p.rpw - 1) / p.rpw;
    p.blocks = (long long)kXcds * p.wpb * ((p.nblk + kXcds - 1) / kXcds);
    if (compact_entries > 0) {
        long long wq = ceil_div(compact_entries, kXcds) + ceil_div(compact_entries, 8LL * kXcds);
        const long long most = (long long)p.cap_b * ((p.nblk + kXcds - 1) / kXcds);  // entries one XCD can hold
        if (wq > most) wq = most;
        p.compact = 1;
        p.wq = (int)wq;
        p.blocks = (long long)kXcds * wq;
    }
    p.use = 1;
    return p;
}

// The group rows' local expert permutation: compact lists over blocks of
// group rows, a copy grid sized for the T * k routed slots the group rows
// carry (each routed slot of a token lies in exactly one of its group rows).
// Each group row carries only a few of its k slots, so full lists would
// give mostly empty copy workgroups.
PullPlan plan_pull_permute(const moedisp_shape& s) {
    return plan_pull(group_rows_shape(s), (long long)s.num_tokens * s.topk);
}

// Group-deduplicated dispatch: the scatter over groups (k = E = G slots per
// token, from the layout's bitmap).
static moedisp_shape group_shape(const moedisp_shape& s) {
    moedisp_shape g = s;
    g.topk = s.num_groups;
    g.num_experts = s.num_groups;
    return g;
}

DispatchPlan plan_dispatch_groups(const moedisp_shape& s) { return plan_dispatch(group_shape(s)); }

// The local permutation of group rows: a group row routes about k / (groups
// per token) of its k slots, at least k / min(G, k); size workgroups by that.
static DispatchPlan plan_group_permute(const moedisp_shape& s) {
    const moedisp_shape rs = group_rows_shape(s);
    const int per_row = (s.topk + (s.num_groups < s.topk ? s.num_groups : s.topk) - 1) /
                        (s.num_groups < s.topk ? s.num_groups : s.topk);
    return plan_scatter(rs, (long long)per_row * (long long)row_bytes(rs), (int)(row_bytes(rs) / 16), 1, 2,
                        64 * 1024);
}

// The group rows seen as tokens (T * min(G, k) of them, the capacity of the
// group dispatch), for the local expert permutation and reduce.
moedisp_shape group_rows_shape(const moedisp_shape& s) {
    moedisp_shape g = s;
    g.num_tokens = s.num_tokens * (s.num_groups < s.topk ? s.num_groups : s.topk);
    return g;
}

// Quantising scatter: a lane unit is 16 channels (32 source bytes, 16 code
// bytes); column ranges are whole waves so that no scale block (<= 64 lanes)
// straddles two of them.
DispatchPlan plan_dispatch_quant(const moedisp_shape& s) {
    return plan_scatter(s, (long long)s.topk * (long long)s.hidden, s.hidden / 16, 64, 1, kCopyWorkgroupBytes);
}

// Small-batch path: every workgroup holds the routing table, two per-expert
// arrays and the token masks in LDS (<= 60 KiB); rows are split into column
// ranges while the grid is small, as for the scatter.
SmallPlan plan_small(const moedisp_shape& s) {
    SmallPlan p;
    memset(&p, 0, sizeof p);
    const long long n = (long long)s.num_tokens * s.topk;
    p.lds_bytes = (size_t)(2LL * s.num_experts) * sizeof(int32_t);  // the layout workgroup's tables
    p.supported = n <= kFusedMaxSlots && (size_t)(n + 2LL * s.num_experts + s.num_tokens) * 4 <= 60 * 1024;
    const int row16 = (int)(row_bytes(s) / 16);
    int splits = 1;
    while ((long long)s.num_tokens * splits < 1024 && row16 / (splits * 2) >= kThreads / 2) splits *= 2;
    const int per = ceil_div(row16, splits);
    p.split_units = per;
    p.col_splits = ceil_div(row16, per);
    int threads = (per + 63) / 64 * 64;
    if (threads < kThreads) threads = kThreads;
    if (threads > kMaxDispatchThreads) threads = kMaxDispatchThreads;
    p.threads = threads;
    p.blocks = (long long)s.num_tokens * p.col_splits + 1;  // + the layout workgroup
    return p;
}

// LDS a layout workgroup may use with the notify phase folded in.
constexpr size_t kLayoutNotifyLds = 64 * 1024;

// Whether ep_get_dispatch_layout_notify folds the dispatch's tile counts into
// the layout's workgroups: the tiles (a power of two of tokens) must lie
// inside them and their counts fit the LDS budget with the layout's own.
LayoutNotifyPlan plan_layout_notify(const moedisp_shape& s) {
    LayoutNotifyPlan p;
    const DispatchPlan P = plan_dispatch(s);
    int shift = 0;
    while ((1 << shift) < P.tile_tokens) ++shift;
    const int tpb = layout_tokens_per_block(s);
    p.tile_shift = shift;
    p.fused = s.num_tokens > 0 && (1 << shift) == P.tile_tokens && tpb % P.tile_tokens == 0 &&
              layout_lds_bytes(s.num_experts, s.num_groups, s.topk, tpb, tpb / P.tile_tokens) <= kLayoutNotifyLds;
    return p;
}

CombinePlan plan_combine(const moedisp_shape& s, int loads_per_row) {
    CombinePlan p;
    const int row16 = (int)((size_t)s.hidden * 2 / 16);
    // Each (row, column range) is a workgroup.  Where a row gathers 8 or more
    // rows, one unit per lane (that many loads in flight per lane) and about
    // 64 lanes; where it gathers 2 to 7, one unit and 128 lanes.  Many short
    // workgroups keep loads of other rows issuing while some sum and store;
    // at H = 7168 and k = 8 a row is 14 ranges of 64 units.  Where a row
    // gathers about one (a group row of the local reduce), 2 units per lane
    // and about 256 lanes, so that each lane still has a few loads in flight.
    const int per_lane = loads_per_row >= 2 ? 1 : 2;
    const int target = loads_per_row >= 8 ? 64 : loads_per_row >= 2 ? 128 : 512;
    int splits = (row16 + target - 1) / target;
    if (splits < 1) splits = 1;
    p.col_splits = splits;
    p.blocks = s.num_tokens * splits;
    const int units = (row16 + splits - 1) / splits;
    p.units_per_lane = per_lane;
    int threads = ((units + per_lane - 1) / per_lane + 63) / 64 * 64;
    if (threads > kMaxCombineThreads) threads = kMaxCombineThreads;
    if (threads < 64) threads = 64;
    p.threads = threads;
    return p;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Offsets of one block-pull plan's tables from `base` (all `base` when the
// plan is not used): counts [E][cnt_stride], ls [nblk][E], n [nblk], lists
// [nblk][cap_b]; returns the end of the lists.
static size_t pull_tables(size_t base, const PullPlan& p, int E, size_t off[4]) {
    off[0] = off[1] = off[2] = off[3] = base;
    if (!p.use) return base;
    off[1] = align256(off[0] + (size_t)E * p.cnt_stride * sizeof(int32_t));
    off[2] = align256(off[1] + (size_t)p.nblk * E * sizeof(int32_t));
    off[3] = align256(off[2] + (size_t)p.nblk * sizeof(int32_t));
    return align256(off[3] + (size_t)p.nblk * p.cap_b * sizeof(PullEnt));
}

WsPlan plan_workspace(const moedisp_shape& s) {
    WsPlan w;
    w.layout_blocks = s.num_tokens > 0 ? ceil_div(s.num_tokens, layout_tokens_per_block(s)) : 1;
    w.partial_offset = sizeof(WsHeader);
    const size_t partial_bytes = (size_t)w.layout_blocks * (s.num_experts + s.num_groups) * sizeof(int32_t);
    w.counts_offset = align256(w.partial_offset + partial_bytes);
    // per-tile counts of the largest dispatch the shape allows: over tokens,
    // over groups (group-deduplicated dispatch) or over group rows (their
    // local expert permutation)
    const size_t flat = (size_t)plan_dispatch(s).tile_stride * s.num_experts;
    const size_t groups = (size_t)plan_dispatch_groups(s).tile_stride * s.num_groups;
    const size_t rows = (size_t)plan_dispatch(group_rows_shape(s)).tile_stride * s.num_experts;
    size_t count_words = flat > groups ? flat : groups;
    if (rows > count_words) count_words = rows;
    size_t end = align256(w.counts_offset + count_words * sizeof(int32_t));
    // block-pull tables of the flat dispatch and of the group rows' local
    // expert permutation, from one base
    size_t t[4];
    const size_t end_flat = pull_tables(end, plan_pull(s), s.num_experts, t);
    w.pull_cnt_offset = t[0];
    w.pull_ls_offset = t[1];
    w.pull_n_offset = t[2];
    w.pull_ent_offset = t[3];
    const size_t end_perm = pull_tables(end, plan_pull_permute(s), s.num_experts, t);
    w.perm_cnt_offset = t[0];
    w.perm_ls_offset = t[1];
    w.perm_n_offset = t[2];
    w.perm_ent_offset = t[3];
    w.total = end_flat > end_perm ? end_flat : end_perm;
    return w;
}

static int check_ws(const moedisp_shape* s, void* ws, size_t ws_bytes) {
    if (!ws) return MOEDISP_ERR_INVALID_ARG;
    if (!aligned(ws, 256)) return MOEDISP_ERR_MISALIGNED;
    if (ws_bytes < plan_workspace(*s).total) return MOEDISP_ERR_WORKSPACE_TOO_SMALL;
    return MOEDISP_OK;
}

// hipErrorInvalidConfiguration comes from a launcher's grid-size check (a
// shape whose grid exceeds 2^32 work-items); any other failure is a HIP error.
static int hip_status(hipError_t e) {
    if (e == hipSuccess) return MOEDISP_OK;
    return e == hipErrorInvalidConfiguration ? MOEDISP_ERR_UNSUPPORTED : MOEDISP_ERR_HIP;
}

// Workspace of ep_dispatch_noalloc: one array per device, zero when the code
// object loads and held until the process ends.  Host code never uses the
// name `scratch` as an address (on the host it is a stand-in, not the device
// array): it uses the address hipGetSymbolAddress returns for the current
// device, looked up once per device and kept in scratch_ptr.
constexpr size_t kScratchBytes = (size_t)8 << 20;
constexpr int kScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static void* scratch_ptr[kScratchDevices];
static std::mutex scratch_mu;

static int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return MOEDISP_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOEDISP_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return MOEDISP_OK;
}

}  // namespace moedisp

using namespace moedisp;

extern "C" {

size_t ep_workspace_bytes(const moedisp_shape* s) {
    if (check_shape(s) != MOEDISP_OK) return 0;
    return plan_workspace(*s).total;
}

int ep_workspace_init(void* ws, size_t ws_bytes, void* stream) {
    if (!ws || ws_bytes < sizeof(WsHeader)) return MOEDISP_ERR_INVALID_ARG;
    if (!aligned(ws, 256)) return MOEDISP_ERR_MISALIGNED;
    return hip_status(launch_fill_zero(ws, ws_bytes & ~(size_t)3, (hipStream_t)stream));
}

// Checks of the layout call; fills the launch arguments (notify phase off).
static int layout_args(const moedisp_shape* s, const int32_t* topk_idx, int32_t* tokens_per_expert,
                       int32_t* tokens_per_group, uint32_t* is_token_in_group, void* ws, size_t ws_bytes,
                       LayoutArgs* a) {
    int st = check_shape(s);
    if (st) return st;
    if ((s->num_tokens > 0 && (!topk_idx || !is_token_in_group)) || !tokens_per_expert || !tokens_per_group)
        return MOEDISP_ERR_INVALID_ARG;
    if (!aligned(topk_idx, 4) || !aligned(tokens_per_expert, 4) || !aligned(tokens_per_group, 4) ||
        !aligned(is_token_in_group, 4))
        return MOEDISP_ERR_MISALIGNED;
    if ((st = check_ws(s, ws, ws_bytes))) return st;
    const WsPlan w = plan_workspace(*s);
    a->T = s->num_tokens;
    a->k = s->topk;
    a->E = s->num_experts;
    a->G = s->num_groups;
    a->id_bits = 0;
    while ((1 << a->id_bits) < a->E) ++a->id_bits;
    group_index_constants(a->E / a->G, &a->pg_shift, &a->pg_magic);
    group_index_constants(a->k, &a->k_shift, &a->k_magic);
    a->tokens_per_block = layout_tokens_per_block(*s);
    a->topk_idx = topk_idx;
    a->tokens_per_expert = tokens_per_expert;
    a->tokens_per_group = tokens_per_group;
    a->is_token_in_group = is_token_in_group;
    a->hdr = (WsHeader*)ws;
    a->partials = (int32_t*)((char*)ws + w.partial_offset);
    a->blocks = w.layout_blocks;
    a->tile_counts = nullptr;
    a->tile_shift = 0;
    a->tiles = 0;
    a->tile_stride = 0;
    a->expert_offsets = nullptr;
    a->capacity = s->num_tokens * s->topk;
    return MOEDISP_OK;
}

int ep_get_dispatch_layout(const moedisp_shape* s, const int32_t* topk_idx, int32_t* tokens_per_expert,
                           int32_t* tokens_per_group, uint32_t* is_token_in_group, void* ws, size_t ws_bytes,
                           void* stream) {
    LayoutArgs a;
    const int st = layout_args(s, topk_idx, tokens_per_expert, tokens_per_group, is_token_in_group, ws, ws_bytes, &a);
    if (st) return st;
    return hip_status(launch_layout(a, (hipStream_t)stream));
}

// The block-pull plan and tables of a flat dispatch (off: the push scatter).
static void set_pull(DispatchArgs* a, const moedisp_shape& s, const WsPlan& w, void* ws, bool allow) {
    memset(&a->pull, 0, sizeof a->pull);
    a->pull_cnt = a->pull_ls = a->pull_n = nullptr;
    a->pull_ent = nullptr;
    if (!allow) return;
    a->pull = plan_pull(s);
    if (!a->pull.use) return;
    a->pull_cnt = (int32_t*)((char*)ws + w.pull_cnt_offset);
    a->pull_ls = (int32_t*)((char*)ws + w.pull_ls_offset);
    a->pull_n = (int32_t*)((char*)ws + w.pull_n_offset);
    a->pull_ent = (PullEnt*)((char*)ws + w.pull_ent_offset);
}

static int id_bits_of(int E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b;
}

// The notify launch of a block-pull dispatch: every block sorted, and
// expert_offsets scanned from tokens_per_expert.  With `tiles`, every
// dispatch tile is counted too (the push path's table, which the quantising
// scatter reads after a separate notify phase), tile 0 writing the offsets.
static hipError_t launch_pull_notify(const DispatchArgs& a, bool tiles, hipStream_t stream) {
    NotifyArgs n;
    memset(&n, 0, sizeof n);
    n.d = a;
    n.id_bits = id_bits_of(a.E);
    n.sort_wgs = a.pull.nblk;
    n.count_wgs = tiles ? a.plan.tiles : 0;
    n.count_offsets = tiles ? 1 : 0;
    n.reduce = tiles ? 0 : 2;
    return launch_notify(n, stream);
}

// `tiles`: the phase may be followed by the quantising scatter (a separate
// notify call), which reads the per-tile counts.
static hipError_t launch_notify_phase(const DispatchArgs& a, bool tiles, hipStream_t stream) {
    return a.pull.use ? launch_pull_notify(a, tiles, stream) : launch_dispatch_notify(a, stream);
}

static hipError_t launch_scatter_phase(const DispatchArgs& a, hipStream_t stream) {
    return a.pull.use ? launch_scatter_pull(a, stream) : launch_dispatch_scatter(a, stream);
}

// Checks shared by the dispatch calls; fills the launch arguments.  Pointers
// a phase does not use may be passed as NULL-equivalents by the caller of that
// phase only through the phase-specific wrappers below.
// `ws_shape` (when not null) is the shape the workspace was sized and laid
// out for, if it differs from the dispatched one (the group rows).
static int dispatch_args(const moedisp_shape* s, const void* x, const float* x_scales, const int32_t* topk_idx,
                         const float* topk_weights, const int32_t* tokens_per_expert, void* recv_x,
                         float* recv_scales, int32_t* recv_src_idx, float* recv_weights, const int32_t* expert_offsets,
                         int32_t* slot_to_row, void* ws, size_t ws_bytes, bool scatter, DispatchArgs* a,
                         const moedisp_shape* ws_shape = nullptr, bool allow_pull = true) {
    int st = check_shape(s);
    if (st) return st;
    const bool fp8 = s->x_dtype == MOEDISP_FP8_E4M3;
    if (!tokens_per_expert || !expert_offsets) return MOEDISP_ERR_INVALID_ARG;
    if (s->num_tokens > 0 && !topk_idx) return MOEDISP_ERR_INVALID_ARG;
    if (scatter && s->num_tokens > 0 &&
        (!x || !topk_weights || !recv_x || !recv_src_idx || !recv_weights || !slot_to_row))
        return MOEDISP_ERR_INVALID_ARG;
    if (scatter && s->num_tokens > 0 && fp8 && (!x_scales || !recv_scales)) return MOEDISP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(recv_x, 16)) return MOEDISP_ERR_MISALIGNED;
    if (!aligned(x_scales, 4) || !aligned(recv_scales, 4) || !aligned(topk_idx, 4) || !aligned(topk_weights, 4) ||
        !aligned(tokens_per_expert, 4) || !aligned(recv_src_idx, 4) || !aligned(recv_weights, 4) ||
        !aligned(expert_offsets, 4) || !aligned(slot_to_row, 4))
        return MOEDISP_ERR_MISALIGNED;
    if (!ws_shape) ws_shape = s;
    if ((st = check_ws(ws_shape, ws, ws_bytes))) return st;
    const WsPlan w = plan_workspace(*ws_shape);
    a->T = s->num_tokens;
    a->k = s->topk;
    a->E = s->num_experts;
    a->row16 = (int)(row_bytes(*s) / 16);
    a->out16 = a->row16;
    a->scale_words = fp8 ? scales_per_row(*s) : 0;
    a->q_block_lanes = 0;
    a->q_scales_per_row = 0;
    a->recv_qscales = nullptr;
    a->bitmap = nullptr;
    a->src_k = s->topk;
    a->experts_per_group = s->num_experts / s->num_groups;
    a->recv_topk_idx = nullptr;
    a->recv_topk_weights = nullptr;
    a->capacity = s->num_tokens * s->topk;
    a->plan = plan_dispatch(*s);
    a->x = (const v4u*)x;
    a->x_scales = fp8 ? x_scales : nullptr;
    a->topk_idx = topk_idx;
    a->topk_weights = topk_weights;
    a->tokens_per_expert = tokens_per_expert;
    a->recv_x = (v4u*)recv_x;
    a->recv_scales = fp8 ? recv_scales : nullptr;
    a->recv_src_idx = recv_src_idx;
    a->recv_weights = recv_weights;
    a->expert_offsets = const_cast<int32_t*>(expert_offsets);
    a->slot_to_row = slot_to_row;
    a->hdr = (WsHeader*)ws;
    a->tile_counts = (int32_t*)((char*)ws + w.counts_offset);
    set_pull(a, *s, w, ws, allow_pull && ws_shape == s);
    return MOEDISP_OK;
}

int ep_dispatch_notify(const moedisp_shape* s, const int32_t* topk_idx, const int32_t* tokens_per_expert,
                       int32_t* expert_offsets, void* ws, size_t ws_bytes, void* stream) {
    DispatchArgs a;
    memset(&a, 0, sizeof a);
    const int st = dispatch_args(s, nullptr, nullptr, topk_idx, nullptr, tokens_per_expert, nullptr, nullptr, nullptr,
                                 nullptr, expert_offsets, nullptr, ws, ws_bytes, false, &a);
    if (st) return st;
    return hip_status(launch_notify_phase(a, true, (hipStream_t)stream));
}

int ep_get_dispatch_layout_notify(const moedisp_shape* s, const int32_t* topk_idx, int32_t* tokens_per_expert,
                                  int32_t* tokens_per_group, uint32_t* is_token_in_group, int32_t* expert_offsets,
                                  void* ws, size_t ws_bytes, void* stream) {
    LayoutArgs a;
    int st = layout_args(s, topk_idx, tokens_per_expert, tokens_per_group, is_token_in_group, ws, ws_bytes, &a);
    if (st) return st;
    if (!expert_offsets) return MOEDISP_ERR_INVALID_ARG;
    if (!aligned(expert_offsets, 4)) return MOEDISP_ERR_MISALIGNED;
    // the dispatch's tiles must lie inside the layout workgroups, and their
    // counts fit in LDS; otherwise the two calls, in order
    const DispatchPlan P = plan_dispatch(*s);
    const LayoutNotifyPlan lnp = plan_layout_notify(*s);
    const int shift = lnp.tile_shift;
    const bool fused = lnp.fused != 0;
    const WsPlan w = plan_workspace(*s);
    if (plan_pull(*s).use) {
        // block-pull: the layout's partial counts (with the dispatch tiles'
        // counts where they lie inside its workgroups) and the block sort in
        // one launch, then the reduce of the partials (and the remaining
        // tiles' counts)
        DispatchArgs d;
        if ((st = dispatch_args(s, nullptr, nullptr, topk_idx, nullptr, tokens_per_expert, nullptr, nullptr, nullptr,
                                nullptr, expert_offsets, nullptr, ws, ws_bytes, false, &d)))
            return st;
        LayoutSortArgs ls;
        memset(&ls, 0, sizeof ls);
        ls.lay = a;
        if (fused) {
            ls.lay.tile_counts = (int32_t*)((char*)ws + w.counts_offset);
            ls.lay.tile_shift = shift;
            ls.lay.tiles = P.tiles;
            ls.lay.tile_stride = P.tile_stride;
        }
        ls.d = d;
        ls.id_bits = id_bits_of(a.E);
        ls.sort_wgs = d.pull.nblk;
        LayoutArgs r = a;
        r.expert_offsets = expert_offsets;
        NotifyArgs n;
        memset(&n, 0, sizeof n);
        n.d = d;
        n.lay = r;
        n.id_bits = ls.id_bits;
        n.count_wgs = P.tiles;
        n.count_offsets = 0;
        n.reduce = 1;
        if (!grid_fits((long long)a.blocks + ls.sort_wgs, kLayoutThreads) ||
            (!fused && !grid_fits((long long)n.count_wgs + 1, kNotifyThreads)))
            return MOEDISP_ERR_UNSUPPORTED;
        if ((st = hip_status(launch_layout_sort(ls, (hipStream_t)stream)))) return st;
        if (fused) return hip_status(launch_layout_reduce(r, (hipStream_t)stream));
        return hip_status(launch_notify(n, (hipStream_t)stream));
    }
    if (!fused) {
        if ((st = hip_status(launch_layout(a, (hipStream_t)stream)))) return st;
        return ep_dispatch_notify(s, topk_idx, tokens_per_expert, expert_offsets, ws, ws_bytes, stream);
    }
    a.tile_counts = (int32_t*)((char*)ws + w.counts_offset);
    a.tile_shift = shift;
    a.tiles = P.tiles;
    a.tile_stride = P.tile_stride;
    a.expert_offsets = expert_offsets;
    return hip_status(launch_layout(a, (hipStream_t)stream));
}

int ep_dispatch_scatter(const moedisp_shape* s, const void* x, const float* x_scales, const int32_t* topk_idx,
                        const float* topk_weights, const int32_t* tokens_per_expert, void* recv_x, float* recv_scales,
                        int32_t* recv_src_idx, float* recv_weights, const int32_t* expert_offsets,
                        int32_t* slot_to_row, void* ws, size_t ws_bytes, void* stream) {
    DispatchArgs a;
    memset(&a, 0, sizeof a);
    const int st = dispatch_args(s, x, x_scales, topk_idx, topk_weights, tokens_per_expert, recv_x, recv_scales,
                                 recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws, ws_bytes, true, &a);
    if (st) return st;
    return hip_status(launch_scatter_phase(a, (hipStream_t)stream));
}

int ep_dispatch(const moedisp_shape* s, const void* x, const float* x_scales, const int32_t* topk_idx,
                const float* topk_weights, const int32_t* tokens_per_expert, void* recv_x, float* recv_scales,
                int32_t* recv_src_idx, float* recv_weights, int32_t* expert_offsets, int32_t* slot_to_row,
                void* ws, size_t ws_bytes, void* stream) {
    DispatchArgs a;
    memset(&a, 0, sizeof a);
    const int st = dispatch_args(s, x, x_scales, topk_idx, topk_weights, tokens_per_expert, recv_x, recv_scales,
                                 recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws, ws_bytes, true, &a);
    if (st) return st;
    if (a.pull.use ? !grid_fits(a.pull.blocks, a.pull.threads) : !grid_fits(a.plan.blocks, a.plan.threads))
        return MOEDISP_ERR_UNSUPPORTED;  // before either launch
    const hipError_t e = launch_notify_phase(a, false, (hipStream_t)stream);
    if (e != hipSuccess) return MOEDISP_ERR_HIP;
    return hip_status(launch_scatter_phase(a, (hipStream_t)stream));
}

int ep_dispatch_noalloc(const moedisp_shape* s, const void* x, const float* x_scales, const int32_t* topk_idx,
                        const float* topk_weights, const int32_t* tokens_per_expert, void* recv_x,
                        float* recv_scales, int32_t* recv_src_idx, float* recv_weights, int32_t* expert_offsets,
                        int32_t* slot_to_row, int32_t* status, void* stream) {
    if (!status) return MOEDISP_ERR_INVALID_ARG;
    if (!aligned(status, 4)) return MOEDISP_ERR_MISALIGNED;
    // every host check first, against a stand-in workspace address (aligned,
    // never dereferenced) of the array's size: a shape whose workspace
    // exceeds the array is WORKSPACE_TOO_SMALL before any HIP call
    DispatchArgs a;
    memset(&a, 0, sizeof a);
    int st = dispatch_args(s, x, x_scales, topk_idx, topk_weights, tokens_per_expert, recv_x, recv_scales,
                           recv_src_idx, recv_weights, expert_offsets, slot_to_row, (void*)(uintptr_t)256,
                           kScratchBytes, true, &a);
    if (st) return st;
    if (a.pull.use ? !grid_fits(a.pull.blocks, a.pull.threads) : !grid_fits(a.plan.blocks, a.plan.threads))
        return MOEDISP_ERR_UNSUPPORTED;
    void* ws = nullptr;
    if ((st = scratch_of_current_device(&ws))) return st;
    memset(&a, 0, sizeof a);
    if ((st = dispatch_args(s, x, x_scales, topk_idx, topk_weights, tokens_per_expert, recv_x, recv_scales,
                            recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws, kScratchBytes, true, &a)))
        return st;
    // the kernels or their status bits into the header's first word, its
    // only use: here that word is the caller's, cleared first (by a kernel,
    // so that the call can be captured in a graph)
    static_assert(offsetof(WsHeader, status) == 0, "status is the header's first word");
    a.hdr = reinterpret_cast<WsHeader*>(status);
    hipError_t e = launch_set_word(reinterpret_cast<uint32_t*>(status), 0u, (hipStream_t)stream);
    if (e != hipSuccess) return MOEDISP_ERR_HIP;
    e = launch_notify_phase(a, false, (hipStream_t)stream);
    if (e != hipSuccess) return MOEDISP_ERR_HIP;
    return hip_status(launch_scatter_phase(a, (hipStream_t)stream));
}

// Checks of the quantising dispatch calls; fills the launch arguments.
static int quant_args(const moedisp_shape* s, int32_t quant_block, int32_t scale_fmt, const void* x,
                      const int32_t* topk_idx, const float* topk_weights, const int32_t* tokens_per_expert,
                      void* recv_x, void* recv_scales, int32_t* recv_src_idx, float* recv_weights,
                      const int32_t* expert_offsets, int32_t* slot_to_row, void* ws, size_t ws_bytes,
                      DispatchArgs* a) {
    int st = check_shape(s);
    if (st) return st;
    if (s->x_dtype != MOEDISP_BF16) return MOEDISP_ERR_UNSUPPORTED;
    if (scale_fmt != MOEDISP_SCALE_FP32 && scale_fmt != MOEDISP_SCALE_UE8M0) return MOEDISP_ERR_UNSUPPORTED;
    if (quant_block < 32 || quant_block > 1024 || (quant_block & (quant_block - 1)) != 0)
        return MOEDISP_ERR_UNSUPPORTED;
    if (s->hidden % quant_block != 0) return MOEDISP_ERR_INVALID_ARG;
    if (!tokens_per_expert || !expert_offsets) return MOEDISP_ERR_INVALID_ARG;
    if (s->num_tokens > 0 && (!topk_idx || !x || !topk_weights || !recv_x || !recv_scales || !recv_src_idx ||
                              !recv_weights || !slot_to_row))
        return MOEDISP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(recv_x, 16)) return MOEDISP_ERR_MISALIGNED;
    if ((scale_fmt == MOEDISP_SCALE_FP32 && !aligned(recv_scales, 4)) || !aligned(topk_idx, 4) ||
        !aligned(topk_weights, 4) || !aligned(tokens_per_expert, 4) || !aligned(recv_src_idx, 4) ||
        !aligned(recv_weights, 4) || !aligned(expert_offsets, 4) || !aligned(slot_to_row, 4))
        return MOEDISP_ERR_MISALIGNED;
    if ((st = check_ws(s, ws, ws_bytes))) return st;
    const WsPlan w = plan_workspace(*s);
    a->T = s->num_tokens;
    a->k = s->topk;
    a->E = s->num_experts;
    a->row16 = (int)((size_t)s->hidden * 2 / 16);
    a->out16 = s->hidden / 16;
    a->scale_words = 0;
    a->q_block_lanes = quant_block / 16;
    a->q_scales_per_row = s->hidden / quant_block;
    a->capacity = s->num_tokens * s->topk;
    a->plan = plan_dispatch_quant(*s);
    a->x = (const v4u*)x;
    a->x_scales = nullptr;
    a->topk_idx = topk_idx;
    a->topk_weights = topk_weights;
    a->tokens_per_expert = tokens_per_expert;
    a->recv_x = (v4u*)recv_x;
    a->recv_scales = nullptr;
    a->recv_src_idx = recv_src_idx;
    a->recv_weights = recv_weights;
    a->expert_offsets = const_cast<int32_t*>(expert_offsets);
    a->slot_to_row = slot_to_row;
    a->recv_qscales = recv_scales;
    a->bitmap = nullptr;
    a->src_k = s->topk;
    a->experts_per_group = s->num_experts / s->num_groups;
    a->recv_topk_idx = nullptr;
    a->recv_topk_weights = nullptr;
    a->hdr = (WsHeader*)ws;
    a->tile_counts = (int32_t*)((char*)ws + w.counts_offset);
    return MOEDISP_OK;
}

int ep_dispatch_scatter_quant(const moedisp_shape* s, int32_t quant_block, int32_t scale_fmt, const void* x,
                              const int32_t* topk_idx, const float* topk_weights,
                              const int32_t* tokens_per_expert, void* recv_x, void* recv_scales,
                              int32_t* recv_src_idx, float* recv_weights, const int32_t* expert_offsets,
                              int32_t* slot_to_row, void* ws, size_t ws_bytes, void* stream) {
    DispatchArgs a;
    memset(&a, 0, sizeof a);
    const int st = quant_args(s, quant_block, scale_fmt, x, topk_idx, topk_weights, tokens_per_expert, recv_x,
                              recv_scales, recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws, ws_bytes, &a);
    if (st) return st;
    return hip_status(launch_dispatch_scatter_quant(a, scale_fmt, (hipStream_t)stream));
}

int ep_dispatch_quant(const moedisp_shape* s, int32_t quant_block, int32_t scale_fmt, const void* x,
                      const int32_t* topk_idx, const float* topk_weights, const int32_t* tokens_per_expert,
                      void* recv_x, void* recv_scales, int32_t* recv_src_idx, float* recv_weights,
                      int32_t* expert_offsets, int32_t* slot_to_row, void* ws, size_t ws_bytes, void* stream) {
    DispatchArgs a;
    memset(&a, 0, sizeof a);
    const int st = quant_args(s, quant_block, scale_fmt, x, topk_idx, topk_weights, tokens_per_expert, recv_x,
                              recv_scales, recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws, ws_bytes, &a);
    if (st) return st;
    // the count kernel's tile plan is the shape's, shared with the copy path
    if (!grid_fits(a.plan.blocks, a.plan.threads)) return MOEDISP_ERR_UNSUPPORTED;  // before either launch
    if (launch_dispatch_notify(a, (hipStream_t)stream) != hipSuccess) return MOEDISP_ERR_HIP;
    return hip_status(launch_dispatch_scatter_quant(a, scale_fmt, (hipStream_t)stream));
}

}  // extern "C"

// Padded-layout arguments: C >= 0, B >= 0, B + C <= S, E * S < 2^31.
static int check_padded(const moedisp_shape* s, long long C, long long S, long long B) {
    if (C < 0 || B < 0 || S < 1 || B + C > S) return MOEDISP_ERR_INVALID_ARG;
    if ((long long)s->num_experts * S > 0x7FFFFFFFll) return MOEDISP_ERR_UNSUPPORTED;
    return MOEDISP_OK;
}

// ep_combine over receive buffers of `capacity` rows.
static int flat_combine(const moedisp_shape* s, int capacity, const void* expert_out, const int32_t* recv_src_idx,
                        const float* recv_weights, const int32_t* slot_to_row, void* out, int32_t out_dtype,
                        void* ws, size_t ws_bytes, void* stream) {
    int st = check_shape(s);
    if (st) return st;
    if (out_dtype != MOEDISP_BF16 && out_dtype != MOEDISP_FP32) return MOEDISP_ERR_UNSUPPORTED;
    if ((size_t)s->hidden * 2 % 16 != 0) return MOEDISP_ERR_UNSUPPORTED;
    if (s->num_tokens > 0 && (!expert_out || !recv_weights || !slot_to_row || !out)) return MOEDISP_ERR_INVALID_ARG;
    if (!aligned(expert_out, 16) || !aligned(out, 16)) return MOEDISP_ERR_MISALIGNED;
    if (!aligned(recv_src_idx, 4) || !aligned(recv_weights, 4) || !aligned(slot_to_row, 4))
        return MOEDISP_ERR_MISALIGNED;
    if ((st = check_ws(s, ws, ws_bytes))) return st;
    if (s->num_tokens == 0) return MOEDISP_OK;
    const CombinePlan p = plan_combine(*s, s->topk);
    CombineArgs a;
    a.T = s->num_tokens;
    a.k = s->topk;
    a.row16 = (int)((size_t)s->hidden * 2 / 16);
    a.capacity = capacity;
    a.col_splits = p.col_splits;
    a.threads = p.threads;
    a.units_per_lane = p.units_per_lane;
    a.expert_out = (const v4u*)expert_out;
    a.recv_src_idx = recv_src_idx;
    a.recv_weights = recv_weights;
    a.slot_to_row = slot_to_row;
    a.row_limit = nullptr;
    a.out = out;
    a.hdr = (WsHeader*)ws;
    return hip_status(launch_combine(a, out_dtype == MOEDISP_FP32, (hipStream_t)stream));
}

extern "C" {

int ep_combine(const moedisp_shape* s, const void* expert_out, const int32_t* recv_src_idx,
               const float* recv_weights, const int32_t* slot_to_row, void* out, int32_t out_dtype, void* ws,
               size_t ws_bytes, void* stream) {
    const int st = check_shape(s);
    if (st) return st;
    return flat_combine(s, s->num_tokens * s->topk, expert_out, recv_src_idx, recv_weights, slot_to_row, out,
                        out_dtype, ws, ws_bytes, stream);
}

int ep_combine_padded(const moedisp_shape* s, int32_t expert_stride, const void* expert_out,
                      const int32_t* recv_src_idx, const float* recv_weights, const int32_t* slot_to_row,
                      void* out, int32_t out_dtype, void* ws, size_t ws_bytes, void* stream) {
    int st = check_shape(s);
    if (st) return st;
    if ((st = check_padded(s, 0, expert_stride, 0))) return st;
    return flat_combine(s, s->num_experts * expert_stride, expert_out, recv_src_idx, recv_weights, slot_to_row,
                        out, out_dtype, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Small-batch path: layout + dispatch in one launch

}  // extern "C"

// The small path's checks and launch; pad_s > 0 for the padded layout (no
// expert_offsets).
static int small_call(const moedisp_shape* s, int pad_c, int pad_s, int pad_b, const void* x,
                      const float* x_scales, const int32_t* topk_idx, const float* topk_weights,
                      int32_t* tokens_per_expert, int32_t* tokens_per_group, uint32_t* is_token_in_group,
                      void* recv_x, float* recv_scales, int32_t* recv_src_idx, float* recv_weights,
                      int32_t* expert_offsets, int32_t* slot_to_row, void* ws, size_t ws_bytes, void* stream) {
    int st = check_shape(s);
    if (st) return st;
    const bool fp8 = s->x_dtype == MOEDISP_FP8_E4M3;
    if (!plan_small(*s).supported) return MOEDISP_ERR_UNSUPPORTED;
    if (!tokens_per_expert || !tokens_per_group || (pad_s == 0 && !expert_offsets)) return MOEDISP_ERR_INVALID_ARG;
    if (s->num_tokens > 0 && (!x || !topk_idx || !topk_weights || !is_token_in_group || !recv_x || !recv_src_idx ||
                              !recv_weights || !slot_to_row))
        return MOEDISP_ERR_INVALID_ARG;
    if (s->num_tokens > 0 && fp8 && (!x_scales || !recv_scales)) return MOEDISP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(recv_x, 16)) return MOEDISP_ERR_MISALIGNED;
    if (!aligned(x_scales, 4) || !aligned(recv_scales, 4) || !aligned(topk_idx, 4) || !aligned(topk_weights, 4) ||
        !aligned(tokens_per_expert, 4) || !aligned(tokens_per_group, 4) || !aligned(is_token_in_group, 4) ||
        !aligned(recv_src_idx, 4) || !aligned(recv_weights, 4) || !aligned(expert_offsets, 4) ||
        !aligned(slot_to_row, 4))
        return MOEDISP_ERR_MISALIGNED;
    if ((st = check_ws(s, ws, ws_bytes))) return st;
    const SmallPlan sp = plan_small(*s);
    FusedArgs a;
    a.T = s->num_tokens;
    a.k = s->topk;
    a.E = s->num_experts;
    a.G = s->num_groups;
    a.experts_per_group = s->num_experts / s->num_groups;
    group_index_constants(a.experts_per_group, &a.pg_shift, &a.pg_magic);
    a.row16 = (int)(row_bytes(*s) / 16);
    a.scale_words = fp8 ? scales_per_row(*s) : 0;
    a.capacity = pad_s > 0 ? s->num_experts * pad_s : s->num_tokens * s->topk;
    a.split_units = sp.split_units;
    a.col_splits = sp.col_splits;
    a.threads = sp.threads;
    a.pad_c = pad_c;
    a.pad_s = pad_s;
    a.pad_b = pad_b;
    a.x = (const v4u*)x;
    a.x_scales = fp8 ? x_scales : nullptr;
    a.topk_idx = topk_idx;
    a.topk_weights = topk_weights;
    a.tokens_per_expert = tokens_per_expert;
    a.tokens_per_group = tokens_per_group;
    a.is_token_in_group = is_token_in_group;
    a.recv_x = (v4u*)recv_x;
    a.recv_scales = fp8 ? recv_scales : nullptr;
    a.recv_src_idx = recv_src_idx;
    a.recv_weights = recv_weights;
    a.expert_offsets = pad_s > 0 ? nullptr : expert_offsets;
    a.slot_to_row = slot_to_row;
    a.hdr = (WsHeader*)ws;
    return hip_status(launch_dispatch_fused(a, (hipStream_t)stream));
}

extern "C" {

int ep_layout_dispatch_small(const moedisp_shape* s, const void* x, const float* x_scales, const int32_t* topk_idx,
                             const float* topk_weights, int32_t* tokens_per_expert, int32_t* tokens_per_group,
                             uint32_t* is_token_in_group, void* recv_x, float* recv_scales, int32_t* recv_src_idx,
                             float* recv_weights, int32_t* expert_offsets, int32_t* slot_to_row, void* ws,
                             size_t ws_bytes, void* stream) {
    return small_call(s, 0, 0, 0, x, x_scales, topk_idx, topk_weights, tokens_per_expert, tokens_per_group,
                      is_token_in_group, recv_x, recv_scales, recv_src_idx, recv_weights, expert_offsets,
                      slot_to_row, ws, ws_bytes, stream);
}

int ep_layout_dispatch_small_padded(const moedisp_shape* s, int32_t expert_capacity, int32_t expert_stride,
                                    int32_t row_base, const void* x, const float* x_scales,
                                    const int32_t* topk_idx, const float* topk_weights,
                                    int32_t* tokens_per_expert, int32_t* tokens_per_group,
                                    uint32_t* is_token_in_group, void* recv_x, float* recv_scales,
                                    int32_t* recv_src_idx, float* recv_weights, int32_t* slot_to_row, void* ws,
                                    size_t ws_bytes, void* stream) {
    int st = check_shape(s);
    if (st) return st;
    if ((st = check_padded(s, expert_capacity, expert_stride, row_base))) return st;
    return small_call(s, expert_capacity, expert_stride, row_base, x, x_scales, topk_idx, topk_weights,
                      tokens_per_expert, tokens_per_group, is_token_in_group, recv_x, recv_scales, recv_src_idx,
                      recv_weights, nullptr, slot_to_row, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Group-deduplicated (high-throughput) path

int ep_dispatch_groups(const moedisp_shape* s, const void* x, const float* x_scales, const int32_t* topk_idx,
                       const float* topk_weights, const uint32_t* is_token_in_group, const int32_t* tokens_per_group,
                       void* recv_x, float* recv_scales, int32_t* recv_src_idx, int32_t* recv_topk_idx,
                       float* recv_topk_weights, int32_t* group_offsets, int32_t* token_group_row, void* ws,
                       size_t ws_bytes, void* stream) {
    int st = check_shape(s);
    if (st) return st;
    const bool fp8 = s->x_dtype == MOEDISP_FP8_E4M3;
    if (!tokens_per_group || !group_offsets) return MOEDISP_ERR_INVALID_ARG;
    if (s->num_tokens > 0 && (!x || !topk_idx || !topk_weights || !is_token_in_group || !recv_x ||
                              !recv_src_idx || !recv_topk_idx || !recv_topk_weights || !token_group_row))
        return MOEDISP_ERR_INVALID_ARG;
    if (s->num_tokens > 0 && fp8 && (!x_scales || !recv_scales)) return MOEDISP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(recv_x, 16)) return MOEDISP_ERR_MISALIGNED;
    if (!aligned(x_scales, 4) || !aligned(recv_scales, 4) || !aligned(topk_idx, 4) || !aligned(topk_weights, 4) ||
        !aligned(is_token_in_group, 4) || !aligned(tokens_per_group, 4) || !aligned(recv_src_idx, 4) ||
        !aligned(recv_topk_idx, 4) || !aligned(recv_topk_weights, 4) || !aligned(group_offsets, 4) ||
        !aligned(token_group_row, 4))
        return MOEDISP_ERR_MISALIGNED;
    if ((st = check_ws(s, ws, ws_bytes))) return st;
    const WsPlan w = plan_workspace(*s);
    DispatchArgs a;
    memset(&a, 0, sizeof a);
    a.T = s->num_tokens;
    a.k = s->num_groups;
    a.E = s->num_groups;
    a.row16 = (int)(row_bytes(*s) / 16);
    a.out16 = a.row16;
    a.scale_words = fp8 ? scales_per_row(*s) : 0;
    a.q_block_lanes = 0;
    a.q_scales_per_row = 0;
    a.capacity = group_rows_shape(*s).num_tokens;
    a.plan = plan_dispatch_groups(*s);
    a.x = (const v4u*)x;
    a.x_scales = fp8 ? x_scales : nullptr;
    a.topk_idx = topk_idx;
    a.topk_weights = topk_weights;
    a.tokens_per_expert = tokens_per_group;
    a.recv_x = (v4u*)recv_x;
    a.recv_scales = fp8 ? recv_scales : nullptr;
    a.recv_src_idx = recv_src_idx;
    a.recv_weights = nullptr;
    a.expert_offsets = group_offsets;
    a.slot_to_row = token_group_row;
    a.recv_qscales = nullptr;
    a.bitmap = is_token_in_group;
    a.src_k = s->topk;
    a.experts_per_group = s->num_experts / s->num_groups;
    a.recv_topk_idx = recv_topk_idx;
    a.recv_topk_weights = recv_topk_weights;
    a.hdr = (WsHeader*)ws;
    a.tile_counts = (int32_t*)((char*)ws + w.counts_offset);
    if (!grid_fits(a.plan.blocks, a.plan.threads)) return MOEDISP_ERR_UNSUPPORTED;  // before either launch
    if (launch_dispatch_notify(a, (hipStream_t)stream) != hipSuccess) return MOEDISP_ERR_HIP;
    return hip_status(launch_dispatch_scatter(a, (hipStream_t)stream));
}

int ep_group_permute(const moedisp_shape* s, const void* group_x, const float* group_scales,
                     const int32_t* recv_topk_idx, const float* recv_topk_weights, const int32_t* tokens_per_expert,
                     void* recv_x, float* recv_scales, int32_t* recv_src_idx, float* recv_weights,
                     int32_t* expert_offsets, int32_t* slot_to_row, void* ws, size_t ws_bytes, void* stream) {
    int st = check_shape(s);
    if (st) return st;
    const moedisp_shape rs = group_rows_shape(*s);
    DispatchArgs a;
    memset(&a, 0, sizeof a);
    // the workspace of the token shape also holds the group rows' tile counts
    st = dispatch_args(&rs, group_x, group_scales, recv_topk_idx, recv_topk_weights, tokens_per_expert, recv_x,
                       recv_scales, recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws, ws_bytes, true, &a, s);
    if (st) return st;
    a.capacity = s->num_tokens * s->topk;  // the receive buffers hold T*k rows
    const PullPlan qp = plan_pull_permute(*s);
    if (qp.use) {
        // block-pull over the group rows: block sorts (compact lists) with
        // the offsets scan, then the copy
        const WsPlan w = plan_workspace(*s);
        a.pull = qp;
        a.pull_cnt = (int32_t*)((char*)ws + w.perm_cnt_offset);
        a.pull_ls = (int32_t*)((char*)ws + w.perm_ls_offset);
        a.pull_n = (int32_t*)((char*)ws + w.perm_n_offset);
        a.pull_ent = (PullEnt*)((char*)ws + w.perm_ent_offset);
        if (!grid_fits(qp.blocks, qp.threads)) return MOEDISP_ERR_UNSUPPORTED;
        if (launch_pull_notify(a, false, (hipStream_t)stream) != hipSuccess) return MOEDISP_ERR_HIP;
        return hip_status(launch_scatter_pull(a, (hipStream_t)stream));
    }
    a.plan = plan_group_permute(*s);       // same tiles as plan_dispatch(rs), more rows per workgroup
    if (!grid_fits(a.plan.blocks, a.plan.threads)) return MOEDISP_ERR_UNSUPPORTED;  // before either launch
    if (launch_dispatch_notify(a, (hipStream_t)stream) != hipSuccess) return MOEDISP_ERR_HIP;
    return hip_status(launch_dispatch_scatter(a, (hipStream_t)stream));
}

// The combine kernel over `rows` output rows of `k` slots each.
static int combine_call(const moedisp_shape* s, int rows, int k, int loads_per_row, int capacity, const void* in,
                        const int32_t* src_check, const float* weights, const int32_t* slot_to_row,
                        const int32_t* row_limit, void* out, int32_t out_dtype, void* ws, size_t ws_bytes,
                        void* stream) {
    int st = check_shape(s);
    if (st) return st;
    if (out_dtype != MOEDISP_BF16 && out_dtype != MOEDISP_FP32) return MOEDISP_ERR_UNSUPPORTED;
    if ((size_t)s->hidden * 2 % 16 != 0) return MOEDISP_ERR_UNSUPPORTED;
    if (rows > 0 && (!in || !slot_to_row || !out)) return MOEDISP_ERR_INVALID_ARG;
    if (!aligned(in, 16) || !aligned(out, 16)) return MOEDISP_ERR_MISALIGNED;
    if (!aligned(src_check, 4) || !aligned(weights, 4) || !aligned(slot_to_row, 4) || !aligned(row_limit, 4))
        return MOEDISP_ERR_MISALIGNED;
    if ((st = check_ws(s, ws, ws_bytes))) return st;
    if (rows == 0) return MOEDISP_OK;
    moedisp_shape cs = *s;
    cs.num_tokens = rows;
    cs.topk = k;
    const CombinePlan p = plan_combine(cs, loads_per_row);
    CombineArgs a;
    a.T = rows;
    a.k = k;
    a.row16 = (int)((size_t)s->hidden * 2 / 16);
    a.capacity = capacity;
    a.col_splits = p.col_splits;
    a.threads = p.threads;
    a.units_per_lane = p.units_per_lane;
    a.expert_out = (const v4u*)in;
    a.recv_src_idx = src_check;
    a.recv_weights = weights;
    a.slot_to_row = slot_to_row;
    a.row_limit = row_limit;
    a.out = out;
    a.hdr = (WsHeader*)ws;
    return hip_status(launch_combine(a, out_dtype == MOEDISP_FP32, (hipStream_t)stream));
}

int ep_group_reduce(const moedisp_shape* s, const void* expert_out, const int32_t* recv_src_idx,
                    const float* recv_weights, const int32_t* slot_to_row, const int32_t* group_offsets,
                    void* group_out, int32_t out_dtype, void* ws, size_t ws_bytes, void* stream) {
    if (!s) return MOEDISP_ERR_INVALID_ARG;
    if (s->num_tokens > 0 && (!recv_weights || !group_offsets)) return MOEDISP_ERR_INVALID_ARG;
    const int rows = check_shape(s) == MOEDISP_OK ? group_rows_shape(*s).num_tokens : 0;
    // a group row routes about k / min(G, k) of its k slots (the shape is
    // checked by combine_call)
    const int m = s->num_groups < s->topk ? s->num_groups : s->topk;
    const int per_row = m > 0 ? (s->topk + m - 1) / m : 1;
    return combine_call(s, rows, s->topk, per_row, s->num_tokens * s->topk, expert_out, recv_src_idx, recv_weights,
                        slot_to_row, group_offsets ? group_offsets + s->num_groups : nullptr, group_out, out_dtype,
                        ws, ws_bytes, stream);
}

int ep_combine_groups(const moedisp_shape* s, const void* group_rows, const int32_t* recv_src_idx,
                      const int32_t* token_group_row, void* out, int32_t out_dtype, void* ws, size_t ws_bytes,
                      void* stream) {
    if (!s) return MOEDISP_ERR_INVALID_ARG;
    const int cap = check_shape(s) == MOEDISP_OK ? group_rows_shape(*s).num_tokens : 0;
    return combine_call(s, s->num_tokens, s->num_groups, s->num_groups, cap, group_rows, recv_src_idx, nullptr,
                        token_group_row, nullptr, out, out_dtype, ws, ws_bytes, stream);
}

int ep_check_status(void* ws, size_t ws_bytes, void* stream, int32_t* host_status) {
    if (!ws || !host_status || ws_bytes < sizeof(WsHeader)) return MOEDISP_ERR_INVALID_ARG;
    if (!aligned(ws, 256)) return MOEDISP_ERR_MISALIGNED;
    hipStream_t st = (hipStream_t)stream;
    uint32_t v = 0;
    if (hipMemcpyAsync(&v, &((WsHeader*)ws)->status, sizeof v, hipMemcpyDeviceToHost, st) != hipSuccess)
        return MOEDISP_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return MOEDISP_ERR_HIP;
    *host_status = (int32_t)v;
    if (v) return hip_status(launch_set_word(&((WsHeader*)ws)->status, 0u, st));
    return MOEDISP_OK;
}

const char* ep_status_string(int status) {
    switch (status) {
        case MOEDISP_OK: return "ok";
        case MOEDISP_ERR_INVALID_ARG: return "invalid argument";
        case MOEDISP_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case MOEDISP_ERR_MISALIGNED: return "misaligned pointer";
        case MOEDISP_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MOEDISP_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

// Upper bounds of the kernels' static LDS (their __shared__ declarations).
constexpr int64_t kStaticLdsLayout = 16, kStaticLdsReduce = kMaxExperts * 4 + kReduceThreads / 16, kStaticLdsCount = 48,
                  kStaticLdsNotify = 144, kStaticLdsFused = 2816;

static moedisp_launch_info launch_info(long long blocks, long long threads, size_t lds, int64_t static_lds) {
    moedisp_launch_info l;
    l.blocks = blocks;
    l.threads = threads;
    l.lds_bytes = (int64_t)lds;
    l.static_lds_bytes = static_lds;
    return l;
}

static moedisp_launch_info push_count(const DispatchPlan& p, int E) {
    return launch_info(p.tiles, kThreads, (size_t)E * sizeof(int32_t), kStaticLdsCount);
}

static moedisp_launch_info push_scatter(const DispatchPlan& p, int k) {
    return launch_info(p.blocks, p.threads, (size_t)p.tile_tokens * k * sizeof(int32_t), (int64_t)sizeof(ScatterSmem));
}

int ep_plan_query(const moedisp_shape* s, moedisp_plan_info* info, size_t info_bytes) {
    if (!info || info_bytes != sizeof(moedisp_plan_info)) return MOEDISP_ERR_INVALID_ARG;
    memset(info, 0, sizeof *info);
    info->struct_bytes = (int64_t)sizeof(moedisp_plan_info);
    const int st = check_shape(s);
    if (st) return st;
    const int T = s->num_tokens, E = s->num_experts, G = s->num_groups, k = s->topk;
    const WsPlan w = plan_workspace(*s);
    // layout
    const int tpb = layout_tokens_per_block(*s);
    info->layout_tokens_per_block = tpb;
    info->layout = launch_info(w.layout_blocks, kLayoutThreads, layout_lds_bytes(E, G, k, tpb, 0), kStaticLdsLayout);
    info->layout_reduce = launch_info(1, kReduceThreads, 0, kStaticLdsReduce);
    // flat dispatch
    const DispatchPlan P = plan_dispatch(*s);
    info->tile_tokens = P.tile_tokens;
    info->tiles = P.tiles;
    info->tile_stride = P.tile_stride;
    info->block_tokens = P.block_tokens;
    info->block_slots = (int64_t)P.block_tokens * k;
    info->col_splits = P.col_splits;
    info->split_units = P.split_units;
    info->units_per_lane = P.units_per_lane;
    info->count = push_count(P, E);
    info->scatter = push_scatter(P, k);
    const PullPlan pp = plan_pull(*s);
    const LayoutNotifyPlan lnp = plan_layout_notify(*s);
    info->layout_notify_fused = lnp.fused;
    size_t lay_lds = layout_lds_bytes(E, G, k, tpb, lnp.fused ? (tpb >> lnp.tile_shift) : 0);
    long long lay_blocks = w.layout_blocks;
    if (pp.use) {
        info->pull = 1;
        info->pull_tb = pp.tb;
        info->pull_nblk = pp.nblk;
        info->pull_cap_b = pp.cap_b;
        info->pull_cnt_stride = pp.cnt_stride;
        info->pull_rows_per_wg = pp.rpw;
        info->pull_units = pp.units;
        const size_t sort = sort_lds_words(pp.tb, pp.cap_b, E) * sizeof(int32_t);
        // ep_dispatch's notify launch: the sorts and the offsets scan
        info->pull_notify = launch_info((long long)pp.nblk + 1, kNotifyThreads, sort > (size_t)E * 4 ? sort : (size_t)E * 4,
                                        kStaticLdsNotify);
        info->pull_copy = launch_info(pp.blocks, pp.threads, 0, 0);
        if (sort > lay_lds) lay_lds = sort;
        lay_blocks += pp.nblk;
    }
    info->layout_notify = launch_info(lay_blocks, kLayoutThreads, lay_lds, kStaticLdsLayout);
    // quantising scatter (bf16 rows of whole 32-channel blocks, the smallest
    // block ep_dispatch_quant takes)
    if (s->x_dtype == MOEDISP_BF16 && s->hidden % 32 == 0) {
        const DispatchPlan Q = plan_dispatch_quant(*s);
        info->quant_block_slots = (int64_t)Q.block_tokens * k;
        info->scatter_quant = push_scatter(Q, k);
    }
    // group path
    const moedisp_shape rs = group_rows_shape(*s);
    info->group_rows = rs.num_tokens;
    const DispatchPlan GP = plan_dispatch_groups(*s);
    info->groups_tile_stride = GP.tile_stride;
    info->groups_tiles = GP.tiles;
    info->groups_block_slots = (int64_t)GP.block_tokens * G;
    info->groups_count = push_count(GP, G);
    info->groups_scatter = push_scatter(GP, G);
    const PullPlan qp = plan_pull_permute(*s);
    if (qp.use) {
        info->permute_pull = 1;
        info->permute_pull_tb = qp.tb;
        info->permute_pull_nblk = qp.nblk;
        info->permute_pull_cap_b = qp.cap_b;
        info->permute_pull_cnt_stride = qp.cnt_stride;
        info->permute_pull_units = qp.units;
        info->permute_pull_wgs_per_xcd = qp.wq;
        const size_t sort = sort_lds_words(qp.tb, qp.cap_b, E) * sizeof(int32_t);
        info->permute_pull_notify = launch_info((long long)qp.nblk + 1, kNotifyThreads,
                                                sort > (size_t)E * 4 ? sort : (size_t)E * 4, kStaticLdsNotify);
        info->permute_pull_copy = launch_info(qp.blocks, qp.threads, 0, 0);
    } else {
        const DispatchPlan RP = plan_group_permute(*s);
        info->permute_tile_stride = RP.tile_stride;
        info->permute_tiles = RP.tiles;
        info->permute_block_slots = (int64_t)RP.block_tokens * k;
        info->permute_count = push_count(RP, E);
        info->permute_scatter = push_scatter(RP, k);
    }
    // combines (no LDS)
    if (T > 0) {
        const CombinePlan C = plan_combine(*s, k);
        info->combine_col_splits = C.col_splits;
        info->combine_units_per_lane = C.units_per_lane;
        info->combine = launch_info(C.blocks, C.threads, 0, 0);
        const int m = G < k ? G : k;
        moedisp_shape cs = *s;
        cs.num_tokens = rs.num_tokens;
        const CombinePlan RC = plan_combine(cs, (k + m - 1) / m);
        info->group_reduce = launch_info(RC.blocks, RC.threads, 0, 0);
        cs = *s;
        cs.topk = G;
        const CombinePlan GC = plan_combine(cs, G);
        info->combine_groups = launch_info(GC.blocks, GC.threads, 0, 0);
    }
    // small path
    const SmallPlan sp = plan_small(*s);
    if (sp.supported) {
        info->small = 1;
        info->small_fused = launch_info(sp.blocks, sp.threads, sp.lds_bytes, kStaticLdsFused);
    }
    // workspace
    info->ws_total = (int64_t)w.total;
    info->ws_partial_offset = (int64_t)w.partial_offset;
    info->ws_partial_bytes = (int64_t)w.layout_blocks * (E + G) * (int64_t)sizeof(int32_t);
    info->ws_counts_offset = (int64_t)w.counts_offset;
    info->ws_counts_bytes = (int64_t)(w.pull_cnt_offset - w.counts_offset);
    info->ws_counts_needed_flat = (int64_t)P.tile_stride * E * 4;
    info->ws_counts_needed_groups = (int64_t)GP.tile_stride * G * 4;
    info->ws_counts_needed_rows = (int64_t)plan_dispatch(rs).tile_stride * E * 4;
    info->ws_pull_cnt_offset = (int64_t)w.pull_cnt_offset;
    info->ws_pull_ls_offset = (int64_t)w.pull_ls_offset;
    info->ws_pull_n_offset = (int64_t)w.pull_n_offset;
    info->ws_pull_ent_offset = (int64_t)w.pull_ent_offset;
    info->ws_pull_end = pp.use ? (int64_t)(w.pull_ent_offset + (size_t)pp.nblk * pp.cap_b * sizeof(PullEnt))
                               : (int64_t)w.pull_ent_offset;
    info->ws_permute_pull_cnt_offset = (int64_t)w.perm_cnt_offset;
    info->ws_permute_pull_ls_offset = (int64_t)w.perm_ls_offset;
    info->ws_permute_pull_n_offset = (int64_t)w.perm_n_offset;
    info->ws_permute_pull_ent_offset = (int64_t)w.perm_ent_offset;
    info->ws_permute_pull_end = qp.use ? (int64_t)(w.perm_ent_offset + (size_t)qp.nblk * qp.cap_b * sizeof(PullEnt))
                                       : (int64_t)w.perm_ent_offset;
    info->max_block_slots = kMaxBlockSlots;
    info->max_tile_slots = kMaxTileSlots;
    info->max_threads = kMaxDispatchThreads;
    info->pull_max_block_slots = kPullMaxBlockSlots;
    info->pull_max_blocks = kPullMaxBlocks;
    return MOEDISP_OK;
}

int ep_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if ((!dst || !src) && bytes) return MOEDISP_ERR_INVALID_ARG;
    if (bytes % 16 != 0) return MOEDISP_ERR_UNSUPPORTED;
    if (!aligned(dst, 16) || !aligned(src, 16)) return MOEDISP_ERR_MISALIGNED;
    return hip_status(launch_probe_copy((v4u*)dst, (const v4u*)src, bytes / 16, (hipStream_t)stream));
}

int ep_probe_read(const void* src, size_t bytes, void* sink, void* stream) {
    if ((!src && bytes) || !sink) return MOEDISP_ERR_INVALID_ARG;
    if (bytes % 16 != 0) return MOEDISP_ERR_UNSUPPORTED;
    if (!aligned(src, 16) || !aligned(sink, 16)) return MOEDISP_ERR_MISALIGNED;
    return hip_status(launch_probe_read((const v4u*)src, bytes / 16, (v4u*)sink, (hipStream_t)stream));
}

int ep_probe_fill(void* dst, size_t bytes, int32_t shuffled, void* stream) {
    if (!dst && bytes) return MOEDISP_ERR_INVALID_ARG;
    if (bytes % 4096 != 0 || (shuffled != 0 && shuffled != 1)) return MOEDISP_ERR_UNSUPPORTED;
    if (!aligned(dst, 16)) return MOEDISP_ERR_MISALIGNED;
    const size_t chunks = bytes / 4096;
    size_t mult = 1;
    if (shuffled && chunks > 1) {
        // a prime near chunks * golden ratio that does not divide chunks:
        // consecutive workgroups land far apart, and the map is a bijection
        static const size_t primes[] = {1000003, 999983, 999979, 1299709, 15485863, 32452843};
        for (size_t p : primes)
            if (chunks % p != 0) {
                mult = p;
                break;
            }
    }
    return hip_status(launch_probe_fill((v4u*)dst, chunks, mult, (hipStream_t)stream));
}

}  // extern "C"
