// kda_api.cpp -- C entry points of libkda_mi355x.so: argument validation,
// launch planning from host-visible metadata, and the hand-off to the gfx950
// kernels.  Pure C++: every HIP runtime call lives in kda_kernels.hip.
//
// Rules taken from the pages: one kernel launch per call and no fallback to
// another implementation ("flashinfer.kda_decode", backend="cake" section);
// the schedule is chosen from host-visible sizes only and device tensors are
// never read on the host ("Serving-native packed Kimi K3 decode"; the
// fused_kda_decode Parameters on state_indices_mode); strict tensor and alias
// validation ("feat(cake_kda): add serving-native packed decode backend",
// walkthrough of the CUDA binding).
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/kda.h"
#include "kda_internal.h"

using namespace kda_detail;

namespace {

thread_local char g_err[512];

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok()
{
    g_err[0] = 0;
    return KDA_OK;
}

// Extents are computed in 128-bit arithmetic from validated (non-negative)
// sizes and strides, so no product can wrap; a buffer that would span more
// than 2^48 bytes (or past the end of the address space) is an error.
typedef unsigned __int128 u128;
constexpr u128 MAX_BYTES = (u128)1 << 48;

// Byte range [lo, hi) of a buffer; empty when lo == hi.
struct Range {
    uintptr_t lo, hi;
    const char *name;
    bool too_large;
};

Range span(const void *p, u128 bytes, const char *name)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    if (bytes > MAX_BYTES || (u128)lo + bytes > (u128)UINTPTR_MAX) return Range{lo, lo, name, true};
    return Range{lo, lo + (uintptr_t)bytes, name, false};
}

bool overlap(const Range &a, const Range &b)
{
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// Each written range must not overlap any other range (written or read).
int check_alias(const Range *w, int nw, const Range *r, int nr)
{
    for (int i = 0; i < nw + nr; ++i) {
        const Range &x = i < nw ? w[i] : r[i - nw];
        if (x.too_large) return fail(KDA_ERR_SHAPE, "%s would span more than 2^48 bytes", x.name);
    }
    for (int i = 0; i < nw; ++i) {
        for (int j = i + 1; j < nw; ++j)
            if (overlap(w[i], w[j]))
                return fail(KDA_ERR_ALIAS, "%s overlaps %s", w[i].name, w[j].name);
        for (int j = 0; j < nr; ++j)
            if (overlap(w[i], r[j]))
                return fail(KDA_ERR_ALIAS, "%s overlaps %s", w[i].name, r[j].name);
    }
    return KDA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned2(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr int64_t HEAD_ELEMS = (int64_t)KD * KD;
constexpr int64_t MAX_INDEX = 0x7fffffffLL;

int elem_size(int32_t dtype) { return dtype == KDA_DTYPE_F32 ? 4 : 2; }

// Extent in elements of a row-strided [rows, width] tensor (stride >= width >= 0).
u128 rows_extent(int64_t rows, int64_t stride, int64_t width)
{
    return rows <= 0 ? 0 : (u128)(uint64_t)(rows - 1) * (uint64_t)stride + (uint64_t)width;
}

// Largest row / slot stride accepted, in elements (checked before any product).
constexpr int64_t MAX_STRIDE = (int64_t)1 << 44;

int check_gate(int32_t mode)
{
    if (mode == KDA_GATE_SOFTPLUS) return KDA_OK;
    if (mode == KDA_GATE_LOWER_BOUND)
        return fail(KDA_ERR_UNSUPPORTED,
                    "the bounded (lower_bound) gate is not defined by the method's pages; "
                    "only the softplus gate is implemented");
    return fail(KDA_ERR_UNSUPPORTED, "unknown gate_mode %d", (int)mode);
}

int check_pool(const void *state, int32_t dtype, int64_t num_slots, int64_t slot_stride, int32_t H)
{
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16)
        return fail(KDA_ERR_DTYPE, "state_dtype %d is neither F32 nor BF16", (int)dtype);
    if (num_slots < 1 || num_slots > MAX_INDEX)
        return fail(KDA_ERR_SHAPE, "num_slots %lld out of range", (long long)num_slots);
    if (slot_stride < (int64_t)H * HEAD_ELEMS || slot_stride > MAX_STRIDE)
        return fail(KDA_ERR_STRIDE, "slot_stride %lld must be in [H*128*128, 2^44]", (long long)slot_stride);
    if (!aligned16(state) || ((slot_stride * elem_size(dtype)) & 15) != 0)
        return fail(KDA_ERR_ALIGN, "state base and slot stride must be 16-byte aligned");
    return KDA_OK;
}

u128 pool_bytes(int32_t dtype, int64_t num_slots, int64_t slot_stride, int32_t H)
{
    return ((u128)(uint64_t)(num_slots - 1) * (uint64_t)slot_stride + (u128)(uint64_t)H * HEAD_ELEMS) *
           (u128)elem_size(dtype);
}

// Value rows per workgroup.  A (row, head) item is split into vsplit
// workgroups of 128/vsplit value rows (16*G with G = 8/vsplit rows per DPP
// row).  Measured on MI355X (cold-cache sweeps of H=32 fp32 and H=12 bf16,
// B=1..512): 32 rows per workgroup (vsplit 4, two 16-byte accesses per lane
// and value row group, eight waves per SIMD) is best or within 3% of best
// almost everywhere; bf16 pools with 512..1535 items are 4-6% faster at 64
// rows per workgroup.
// The token loop (T >= 2 per sequence) is bound by per-token arithmetic and
// latency rather than by the single pass over the state: splitting a head
// over workgroups repeats the token staging in every split, so it pays only
// while the grid is small.  Measured on MI355X (read-only batched T=4 calls,
// H=12 and 32, fp32 and bf16 pools): 4 splits below ~96 items, 2 up to ~1024,
// none above.
int choose_vsplit(int64_t items, bool bf16, bool token_loop, bool f32_checkpoints, bool update)
{
    // A token loop that writes fp32 checkpoints is bound by those writes, and
    // smaller state tiles stream them better: 32 rows measured 3.5% faster
    // than whole heads on the ragged H=16 N=64 workload (57.5 against
    // 59.6 us; 2 splits 58.4, 8 splits 62.5), while bf16 checkpoints (36.6
    // against 40.7 us) and calls without checkpoints keep the rule below.
    if (token_loop && f32_checkpoints) return 4;
    // Updating token loops over an fp32 pool write back twice the bytes of a
    // bf16 one and stream them best in 32-row tiles up to ~380 items (batched
    // T=4, H=32: 7.81 against 8.15 us at 128 items, 10.68 against 10.99 at
    // 256; 2 splits win from 512); read-only and bf16 calls keep the rule
    // below (read-only ragged fp32: 9.75 us with 2 splits against 9.99 with 4
    // at 256 items).
    if (token_loop && update && !bf16 && items < 384) return 4;
    if (token_loop) return items < 96 ? 4 : (items < 1024 ? 2 : 1);
    // T=1.  fp32 pools (H=12 and 32, B=1..512, graph replays over cold slot
    // sets): 16 value rows per workgroup (vsplit 8) below ~100 items (lower
    // latency: more CUs per head) and from ~320 items on (2.5-7% faster at
    // B>=128: smaller tiles stream better at the same 8 waves per SIMD);
    // 32 rows in between, where vsplit 8 measured 4-8% slower.  bf16 pools:
    // vsplit 8 only for a handful of items; 64 rows from 240 to 1535 items
    // (against 32 rows, H=12 and 32: 9-13% faster at 252-256 and 384 items,
    // 4-6% at 504-768, even at 288, 3.5% slower only at H=32 B=14; 7%
    // slower at 192 items).
    if (bf16) return items < 64 ? 8 : (items >= 240 && items < 1536 ? 2 : 4);
    // fp32 at 224-287 items: 64 rows (H=32 B=8: 7.23 against 7.64 us for 32
    // rows and 8.11 for 16; H=12 B=20: 7.60 against 7.89), two workgroups
    // per CU with the whole grid resident.
    if (items >= 224 && items < 288) return 2;
    return (items < 112 || items >= 320) ? 8 : 4;
}

void fill_plan(kda_launch_plan *plan, const Launch &l, int64_t items)
{
    if (!plan) return;
    plan->struct_size = sizeof(kda_launch_plan);
    plan->kernel = l.family;
    plan->grid_x = l.grid;
    plan->block = l.block;
    plan->rows_per_block = l.rows_per_block;
    plan->vsplit = l.vsplit;
    plan->items = items;
}

// ------------------------------------------------------------ recurrent ----

int dtype_ok(int32_t d) { return d == KDA_DTYPE_F32 || d == KDA_DTYPE_BF16; }

int prepare_recurrent(const kda_recurrent_args *a, RecParams *p, Launch *l)
{
    if (!a) return fail(KDA_ERR_NULLPTR, "args is NULL");
    if (a->struct_size != sizeof(kda_recurrent_args))
        return fail(KDA_ERR_ABI, "struct_size %u != %zu", a->struct_size, sizeof(kda_recurrent_args));
    if (a->K != KD || a->V != KD)
        return fail(KDA_ERR_UNSUPPORTED, "K=%d V=%d: only K=V=128", a->K, a->V);
    if (a->H < 1 || a->HV < 1) return fail(KDA_ERR_SHAPE, "H=%d HV=%d must be >= 1", a->H, a->HV);
    if (a->HV % a->H != 0)
        return fail(KDA_ERR_UNSUPPORTED, "HV=%d is not a multiple of H=%d", a->HV, a->H);
    if (a->n_seqs < 1) return fail(KDA_ERR_SHAPE, "n_seqs=%d must be >= 1", a->n_seqs);
    if (a->flags & ~KDA_FLAG_NO_STATE_UPDATE) return fail(KDA_ERR_UNSUPPORTED, "unknown flags 0x%x", a->flags);
    if (a->tokens_per_seq < 0) return fail(KDA_ERR_SHAPE, "tokens_per_seq=%d < 0", a->tokens_per_seq);
    const bool ragged = a->cu_seqlens != nullptr;
    const int64_t tps = a->tokens_per_seq > 1 ? a->tokens_per_seq : 1;
    if (!ragged && (int64_t)a->n_tokens != (int64_t)a->n_seqs * tps)
        return fail(KDA_ERR_SHAPE, "n_tokens=%d != n_seqs=%d * tokens_per_seq=%lld", a->n_tokens, a->n_seqs,
                    (long long)tps);
    if (a->n_tokens < 0) return fail(KDA_ERR_SHAPE, "n_tokens=%d < 0", a->n_tokens);
    const bool precomputed = a->gate_mode == KDA_GATE_PRECOMPUTED;
    int rc = precomputed ? KDA_OK : check_gate(a->gate_mode);
    if (rc) return rc;
    if (!dtype_ok(a->g_dtype) || !dtype_ok(a->beta_dtype))
        return fail(KDA_ERR_DTYPE, "g_dtype %d / beta_dtype %d must be F32 or BF16", a->g_dtype, a->beta_dtype);
    if (!a->state || !a->state_indices || (!precomputed && (!a->A_log || !a->dt_bias)))
        return fail(KDA_ERR_NULLPTR, "a required pointer is NULL");
    if (a->n_tokens > 0 && (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->out))
        return fail(KDA_ERR_NULLPTR, "a required per-token pointer is NULL");
    const int64_t HQ = (int64_t)a->H * KD;
    const int64_t HVC = (int64_t)a->HV * KD;
    if (a->q_stride < HQ || a->k_stride < HQ)
        return fail(KDA_ERR_STRIDE, "q/k token strides must be >= H*128");
    if (a->v_stride < HVC || a->g_stride < HVC)
        return fail(KDA_ERR_STRIDE, "v/g token strides must be >= HV*128");
    if (a->beta_stride < a->HV) return fail(KDA_ERR_STRIDE, "beta_stride must be >= HV");
    const int g_es = a->g_dtype == KDA_DTYPE_F32 ? 4 : 2;
    const int b_es = a->beta_dtype == KDA_DTYPE_F32 ? 4 : 2;
    auto aligned_to = [](const void *ptr, int n) { return (reinterpret_cast<uintptr_t>(ptr) & (uintptr_t)(n - 1)) == 0; };
    if (!aligned2(a->q) || !aligned2(a->k) || !aligned2(a->v) || !aligned_to(a->g, g_es) ||
        !aligned_to(a->beta, b_es) || !aligned4(a->A_log) || !aligned4(a->dt_bias) ||
        !aligned4(a->state_indices) || (ragged && !aligned4(a->cu_seqlens)))
        return fail(KDA_ERR_ALIGN, "inputs must be aligned to their element size");
    if (!aligned16(a->out)) return fail(KDA_ERR_ALIGN, "out must be 16-byte aligned");
    if (!(a->l2_eps >= 0.0f) || !isfinite(a->scale))
        return fail(KDA_ERR_SHAPE, "l2_eps must be >= 0 and scale finite");
    rc = check_pool(a->state, a->state_dtype, a->num_slots, a->slot_stride, a->HV);
    if (rc) return rc;
    if (a->checkpoints) {
        if (a->ckpt_dtype != a->state_dtype)
            return fail(KDA_ERR_UNSUPPORTED, "checkpoints must use the state dtype");
        if (!aligned16(a->checkpoints)) return fail(KDA_ERR_ALIGN, "checkpoints must be 16-byte aligned");
    }
    const bool update = !(a->flags & KDA_FLAG_NO_STATE_UPDATE);
    const bool caches = a->correction_cache || a->kg_cache;
    if (caches) {
        if (a->cache_t_max < 1) return fail(KDA_ERR_SHAPE, "cache_t_max must be >= 1 with a verify cache");
        if (a->kg_cache && !dtype_ok(a->kg_dtype)) return fail(KDA_ERR_DTYPE, "kg_dtype %d", a->kg_dtype);
        if (!aligned16(a->correction_cache) || !aligned4(a->kg_cache))
            return fail(KDA_ERR_ALIGN, "correction_cache must be 16-byte and kg_cache 4-byte aligned");
    }
    const u128 cache_rows = caches ? (u128)(uint64_t)a->num_slots * (uint64_t)a->HV * (uint64_t)a->cache_t_max : 0;
    const int kg_es = a->kg_dtype == KDA_DTYPE_F32 ? 4 : 2;
    const int64_t T = a->n_tokens;
    const int es = elem_size(a->state_dtype);
    const Range state_r = span(a->state, pool_bytes(a->state_dtype, a->num_slots, a->slot_stride, a->HV), "state");
    Range w[5] = {span(a->out, (u128)T * HVC * 2, "out"),
                  span(a->checkpoints, a->checkpoints ? (u128)T * a->HV * HEAD_ELEMS * es : 0, "checkpoints"),
                  update ? state_r : Range{0, 0, ""},
                  span(a->correction_cache, a->correction_cache ? cache_rows * KD * 4 : 0, "correction_cache"),
                  span(a->kg_cache, a->kg_cache ? cache_rows * 2 * KD * kg_es : 0, "kg_cache")};
    Range r[10] = {span(a->q, rows_extent(T, a->q_stride, HQ) * 2, "q"),
                   span(a->k, rows_extent(T, a->k_stride, HQ) * 2, "k"),
                   span(a->v, rows_extent(T, a->v_stride, HVC) * 2, "v"),
                   span(a->g, rows_extent(T, a->g_stride, HVC) * g_es, "g"),
                   span(a->beta, rows_extent(T, a->beta_stride, a->HV) * b_es, "beta"),
                   span(a->A_log, a->A_log ? (u128)a->HV * 4 : 0, "A_log"),
                   span(a->dt_bias, a->dt_bias ? (u128)HVC * 4 : 0, "dt_bias"),
                   span(a->state_indices, (u128)a->n_seqs * 4, "state_indices"),
                   span(a->cu_seqlens, ragged ? ((u128)(uint64_t)a->n_seqs + 1) * 4 : 0, "cu_seqlens"),
                   update ? Range{0, 0, ""} : state_r};
    rc = check_alias(w, 5, r, 10);
    if (rc) return rc;

    const int64_t items = (int64_t)a->n_seqs * a->HV;
    const bool token_loop = ragged || tps > 1;
    // Read-only calls without checkpoints whose sequences have at most
    // VERIFY_WY_MAX_T tokens (batched: T >= 2; ragged: the length the caller
    // declares in tokens_per_seq): the tokens' reads of the initial state
    // become one matrix product per head, on the WY verify kernel.
    const int64_t bound = ragged ? a->tokens_per_seq : tps;
    // (that kernel addresses a sequence's token rows by 32-bit byte offsets
    // from its first row: every input's last row, at its widest lane, lies
    // within 2^31 bytes of the first)
    auto rows_fit = [&](int64_t stride, int64_t span, int64_t es) {
        return (u128)(uint64_t)(bound - 1) * (uint64_t)stride * (uint64_t)es + (u128)(uint64_t)span * (uint64_t)es <
               ((u128)1 << 31);
    };
    const bool wy = !update && !a->checkpoints && bound >= (ragged ? 1 : 2) && bound <= VERIFY_WY_MAX_T &&
                    rows_fit(a->q_stride, HQ, 2) && rows_fit(a->k_stride, HQ, 2) && rows_fit(a->v_stride, HVC, 2) &&
                    rows_fit(a->g_stride, HVC, g_es) && rows_fit(a->beta_stride, a->HV, b_es);
    const int vsplit = wy ? 1 : choose_vsplit(items, a->state_dtype == KDA_DTYPE_BF16, token_loop,
                                                 a->checkpoints != nullptr && a->state_dtype == KDA_DTYPE_F32, update);
    if (items * vsplit > 0x7ffffff0LL) return fail(KDA_ERR_SHAPE, "too many work items");
    l->family = wy ? KERNEL_VERIFY_WY : token_loop ? KERNEL_RECURRENT_VARLEN : KERNEL_RECURRENT_T1;
    l->vsplit = vsplit;
    l->rows_per_block = KD / vsplit;
    l->grid = (int32_t)((items * vsplit + 7) & ~7LL);  // padded to whole XCD rounds
    l->block = 256;
    l->bf16_state = a->state_dtype == KDA_DTYPE_BF16;

    p->q = static_cast<const uint16_t *>(a->q);
    p->k = static_cast<const uint16_t *>(a->k);
    p->v = static_cast<const uint16_t *>(a->v);
    p->g = a->g;
    p->beta = a->beta;
    p->q_stride = a->q_stride;
    p->k_stride = a->k_stride;
    p->v_stride = a->v_stride;
    p->g_stride = a->g_stride;
    p->beta_stride = a->beta_stride;
    p->A_log = a->A_log;
    p->dt_bias = a->dt_bias;
    p->scale = a->scale;
    p->l2_eps = a->l2_eps;
    p->state = a->state;
    p->num_slots = a->num_slots;
    p->slot_stride = a->slot_stride;
    p->state_indices = a->state_indices;
    p->cu_seqlens = a->cu_seqlens;
    p->ckpt = a->checkpoints;
    p->out = static_cast<uint16_t *>(a->out);
    p->n_seqs = a->n_seqs;
    p->n_tokens = a->n_tokens;
    p->H = a->H;
    p->HV = a->HV;
    p->group = a->HV / a->H;
    p->tps = (int32_t)(wy ? bound : tps);
    p->g_f32 = a->g_dtype == KDA_DTYPE_F32;
    p->beta_f32 = a->beta_dtype == KDA_DTYPE_F32;
    p->precomputed = precomputed;
    p->update_state = update;
    p->vsplit = vsplit;
    p->n_work = (int32_t)(items * vsplit);
    p->corr = static_cast<float *>(a->correction_cache);
    p->kg = a->kg_cache;
    p->kg_f32 = a->kg_dtype == KDA_DTYPE_F32;
    p->t_max = caches ? a->cache_t_max : 0;
    return ok();
}

int packed_to_recurrent(const kda_packed_args *a, kda_recurrent_args *r)
{
    if (!a) return fail(KDA_ERR_NULLPTR, "args is NULL");
    if (a->struct_size != sizeof(kda_packed_args))
        return fail(KDA_ERR_ABI, "struct_size %u != %zu", a->struct_size, sizeof(kda_packed_args));
    if (a->H < 1) return fail(KDA_ERR_SHAPE, "H=%d must be >= 1", a->H);
    if (a->B < 1) return fail(KDA_ERR_SHAPE, "B=%d must be >= 1", a->B);
    const int64_t HC = (int64_t)a->H * KD;
    if (a->qkv_stride < 3 * HC) return fail(KDA_ERR_STRIDE, "qkv_stride must be >= 3*H*128");
    if (a->gate_stride < HC) return fail(KDA_ERR_STRIDE, "gate_stride must be >= H*128");
    if (a->beta_stride < a->H) return fail(KDA_ERR_STRIDE, "beta_stride must be >= H");
    if (!a->mixed_qkv) return fail(KDA_ERR_NULLPTR, "mixed_qkv is NULL");
    memset(r, 0, sizeof *r);
    r->struct_size = sizeof *r;
    r->g_dtype = KDA_DTYPE_BF16;
    r->beta_dtype = KDA_DTYPE_BF16;
    r->tokens_per_seq = 1;
    r->n_seqs = a->B;
    r->n_tokens = a->B;
    r->H = r->HV = a->H;
    r->K = r->V = KD;
    const uint16_t *qkv = static_cast<const uint16_t *>(a->mixed_qkv);
    r->q = qkv;
    r->k = qkv + HC;
    r->v = qkv + 2 * HC;
    r->q_stride = r->k_stride = r->v_stride = a->qkv_stride;
    r->g = a->raw_gate;
    r->g_stride = a->gate_stride;
    r->beta = a->raw_beta;
    r->beta_stride = a->beta_stride;
    r->A_log = a->A_log;
    r->dt_bias = a->dt_bias;
    r->scale = 1.0f / sqrtf((float)KD);
    r->l2_eps = 1e-6f;
    r->gate_mode = a->gate_mode;
    r->lower_bound = a->lower_bound;
    r->state = a->state;
    r->state_dtype = a->state_dtype;
    r->ckpt_dtype = a->state_dtype;
    r->num_slots = a->num_slots;
    r->slot_stride = a->slot_stride;
    r->state_indices = a->state_indices;
    r->out = a->out;
    return KDA_OK;
}

// ---------------------------------------------------------------- fused ----

int prepare_fused(const kda_fused_args *a, FusedParams *p, Launch *l)
{
    if (!a) return fail(KDA_ERR_NULLPTR, "args is NULL");
    if (a->struct_size != sizeof(kda_fused_args))
        return fail(KDA_ERR_ABI, "struct_size %u != %zu", a->struct_size, sizeof(kda_fused_args));
    if (a->H < 1) return fail(KDA_ERR_SHAPE, "H=%d must be >= 1", a->H);
    if (a->rows < 1) return fail(KDA_ERR_SHAPE, "rows=%d must be >= 1", a->rows);
    int rc = check_gate(a->gate_mode);
    if (rc) return rc;
    if (!a->x || !a->weight || !a->conv_state || !a->raw_gate || !a->raw_beta || !a->A_log ||
        !a->dt_bias || !a->state_indices || !a->state || !a->output_gate || !a->norm_weight || !a->out)
        return fail(KDA_ERR_NULLPTR, "a required pointer is NULL");
    const int64_t HC = (int64_t)a->H * KD;
    const int64_t C3 = 3 * HC;
    if (a->x_stride < C3) return fail(KDA_ERR_STRIDE, "x_stride must be >= 3*H*128");
    if (a->conv_slot_stride < 3 * C3) return fail(KDA_ERR_STRIDE, "conv_slot_stride must be >= 3*3*H*128");
    if (a->gate_stride < HC || a->ogate_stride < HC)
        return fail(KDA_ERR_STRIDE, "raw_gate/output_gate row strides must be >= H*128");
    if (a->beta_stride < a->H) return fail(KDA_ERR_STRIDE, "beta_stride must be >= H");
    if (!(a->norm_eps >= 0.0f)) return fail(KDA_ERR_SHAPE, "norm_eps must be >= 0");
    if (!aligned2(a->x) || !aligned2(a->conv_state) || !aligned2(a->raw_gate) || !aligned2(a->raw_beta) ||
        !aligned2(a->output_gate) || !aligned4(a->weight) || !aligned4(a->A_log) ||
        !aligned4(a->dt_bias) || !aligned4(a->norm_weight) || !aligned4(a->state_indices))
        return fail(KDA_ERR_ALIGN, "inputs must be aligned to their element size");
    if (!aligned16(a->out)) return fail(KDA_ERR_ALIGN, "out must be 16-byte aligned");
    rc = check_pool(a->state, a->state_dtype, a->num_slots, a->slot_stride, a->H);
    if (rc) return rc;
    const int64_t R = a->rows;
    Range w[3] = {span(a->out, (u128)R * HC * 2, "out"),
                  span(a->state, pool_bytes(a->state_dtype, a->num_slots, a->slot_stride, a->H), "state"),
                  span(a->conv_state, rows_extent(a->num_slots, a->conv_slot_stride, 3 * C3) * 2,
                       "conv_state")};
    Range r[10] = {span(a->x, rows_extent(R, a->x_stride, C3) * 2, "x"),
                   span(a->weight, (u128)12 * HC * 4, "weight"),
                   span(a->raw_gate, rows_extent(R, a->gate_stride, HC) * 2, "raw_gate"),
                   span(a->raw_beta, rows_extent(R, a->beta_stride, a->H) * 2, "raw_beta"),
                   span(a->A_log, (u128)a->H * 4, "A_log"),
                   span(a->dt_bias, (u128)HC * 4, "dt_bias"),
                   span(a->state_indices, (u128)R * 4, "state_indices"),
                   span(a->output_gate, rows_extent(R, a->ogate_stride, HC) * 2, "output_gate"),
                   span(a->norm_weight, (u128)KD * 4, "norm_weight"),
                   Range{0, 0, ""}};
    rc = check_alias(w, 3, r, 9);
    if (rc) return rc;
    const int64_t items = R * a->H;
    if (items > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "too many work items");
    l->family = KERNEL_FUSED;
    l->vsplit = 1;
    l->rows_per_block = KD;
    l->grid = (int32_t)items;
    l->block = 256;
    l->bf16_state = a->state_dtype == KDA_DTYPE_BF16;

    p->x = static_cast<const uint16_t *>(a->x);
    p->x_stride = a->x_stride;
    p->weight = a->weight;
    p->conv_state = static_cast<uint16_t *>(a->conv_state);
    p->conv_slot_stride = a->conv_slot_stride;
    p->graw = static_cast<const uint16_t *>(a->raw_gate);
    p->g_stride = a->gate_stride;
    p->braw = static_cast<const uint16_t *>(a->raw_beta);
    p->beta_stride = a->beta_stride;
    p->A_log = a->A_log;
    p->dt_bias = a->dt_bias;
    p->state_indices = a->state_indices;
    p->state = a->state;
    p->num_slots = a->num_slots;
    p->slot_stride = a->slot_stride;
    p->ogate = static_cast<const uint16_t *>(a->output_gate);
    p->ogate_stride = a->ogate_stride;
    p->norm_weight = a->norm_weight;
    p->norm_eps = a->norm_eps;
    p->scale = 1.0f / sqrtf((float)KD);
    p->l2_eps = 1e-6f;
    p->out = static_cast<uint16_t *>(a->out);
    p->rows = a->rows;
    p->H = a->H;
    return ok();
}

// --------------------------------------------------------- packed fused ----

struct PfGeometry {
    int vs, block;
};

// Workgroups per (sequence, head) and threads per workgroup of the packed
// fused decode.  Unsplit (measured on MI355X, H=12 and 24, T=5, fp32 and
// bf16 pools): 512 threads (4 value rows per lane) are 5-10% faster up to
// ~1000 items, 256 (8 rows per lane) are on par above; 1024 threads are
// never faster (the per-token work of a head is then bound by its CU's VALU
// issue, and each extra lane repeats the token's norm reductions).  Split
// (graph replays, H=12 and 24, T=5, N=1..32): bf16 pools are fastest with 4
// parts below 64 items (N=1: 9.7 against 11.8 us unsplit) and 2 parts below
// 128 (N=8: 12.3 against 12.8); fp32 pools, whose parts move twice the
// bytes, with 4 parts below 32 items (N=1: 9.7 against 10.4 with 2 and 11.1
// unsplit), 2 parts below 80 (N=3..6: 3-7% faster than 4 parts) and none
// from 96 (N=8: 12.4 against 12.9 with 2 parts).  From 32 sequences on the
// CUs are busy and splitting only adds the exchange (+3 to +16 us).
PfGeometry packed_fused_geometry(int64_t items, bool can_split, bool bf16)
{
    PfGeometry g{1, items < 1024 ? 512 : 256};
    if (can_split) {
        const int64_t four = bf16 ? 64 : 32, two = bf16 ? 128 : 80;
        if (items < four) g = PfGeometry{4, 512};
        else if (items < two) g = PfGeometry{2, 512};
    }
    if (g.vs > 1) g.block = 512;  // the split kernels are built for 512 threads
    return g;
}

// assume_scratch: plan as if split scratch were given (for sizing it); the
// call's own split pointers must then be NULL.
int prepare_packed_fused(const kda_packed_fused_args *a, PackedFusedParams *p, Launch *l,
                         bool assume_scratch = false)
{
    if (!a) return fail(KDA_ERR_NULLPTR, "args is NULL");
    if (a->struct_size != sizeof(kda_packed_fused_args))
        return fail(KDA_ERR_ABI, "struct_size %u != %zu", a->struct_size, sizeof(kda_packed_fused_args));
    if (a->H < 1) return fail(KDA_ERR_SHAPE, "H=%d must be >= 1", a->H);
    if (a->n_seqs < 1) return fail(KDA_ERR_SHAPE, "n_seqs=%d must be >= 1", a->n_seqs);
    if (a->n_rows < 0) return fail(KDA_ERR_SHAPE, "n_rows=%d < 0", a->n_rows);
    if (a->max_tokens < 1) return fail(KDA_ERR_SHAPE, "max_tokens=%d must be >= 1", a->max_tokens);
    int rc = check_gate(a->gate_mode);
    if (rc) return rc;
    if (!a->weight || !a->conv_state || !a->A_log || !a->dt_bias || !a->state_indices ||
        !a->query_start_loc || !a->num_accepted_tokens || !a->state || !a->norm_weight)
        return fail(KDA_ERR_NULLPTR, "a required pointer is NULL");
    if (a->n_rows > 0 && (!a->x || !a->raw_gate || !a->raw_beta || !a->output_gate || !a->out))
        return fail(KDA_ERR_NULLPTR, "a required per-row pointer is NULL");
    const int64_t HC = (int64_t)a->H * KD;
    const int64_t C3 = 3 * HC;
    if (a->x_stride < C3) return fail(KDA_ERR_STRIDE, "x_stride must be >= 3*H*128");
    if (a->conv_slot_stride < 3 * C3) return fail(KDA_ERR_STRIDE, "conv_slot_stride must be >= 3*3*H*128");
    if (a->gate_stride < HC || a->ogate_stride < HC)
        return fail(KDA_ERR_STRIDE, "raw_gate/output_gate row strides must be >= H*128");
    if (a->beta_stride < a->H) return fail(KDA_ERR_STRIDE, "beta_stride must be >= H");
    if (a->indices_stride < a->max_tokens) return fail(KDA_ERR_STRIDE, "indices_stride must be >= max_tokens");
    if (!(a->norm_eps >= 0.0f)) return fail(KDA_ERR_SHAPE, "norm_eps must be >= 0");
    if (!aligned2(a->x) || !aligned2(a->conv_state) || !aligned2(a->raw_gate) || !aligned2(a->raw_beta) ||
        !aligned2(a->output_gate) || !aligned4(a->weight) || !aligned4(a->A_log) || !aligned4(a->dt_bias) ||
        !aligned4(a->norm_weight) || !aligned4(a->state_indices) || !aligned4(a->query_start_loc) ||
        !aligned4(a->num_accepted_tokens))
        return fail(KDA_ERR_ALIGN, "inputs must be aligned to their element size");
    if (!aligned16(a->out)) return fail(KDA_ERR_ALIGN, "out must be 16-byte aligned");
    if (!a->split_counters != !a->split_partials)
        return fail(KDA_ERR_NULLPTR, "split_counters and split_partials are given together or not at all");
    const bool can_split = a->split_counters != nullptr || assume_scratch;
    if (can_split && (!aligned4(a->split_counters) || !aligned16(a->split_partials)))
        return fail(KDA_ERR_ALIGN, "split_counters must be 4-byte and split_partials 16-byte aligned");
    rc = check_pool(a->state, a->state_dtype, a->num_slots, a->slot_stride, a->H);
    if (rc) return rc;
    const int64_t R = a->n_rows;
    const int64_t N = a->n_seqs;
    Range w[5] = {span(a->out, (u128)R * HC * 2, "out"),
                  span(a->state, pool_bytes(a->state_dtype, a->num_slots, a->slot_stride, a->H), "state"),
                  span(a->conv_state, rows_extent(a->num_slots, a->conv_slot_stride, 3 * C3) * 2,
                       "conv_state"),
                  span(a->split_counters, a->split_counters ? (u128)N * a->H * 4 : 0, "split_counters"),
                  span(a->split_partials, a->split_partials ? (u128)R * HC * 4 : 0, "split_partials")};
    Range r[12] = {span(a->x, rows_extent(R, a->x_stride, C3) * 2, "x"),
                   span(a->weight, (u128)12 * HC * 4, "weight"),
                   span(a->raw_gate, rows_extent(R, a->gate_stride, HC) * 2, "raw_gate"),
                   span(a->raw_beta, rows_extent(R, a->beta_stride, a->H) * 2, "raw_beta"),
                   span(a->A_log, (u128)a->H * 4, "A_log"),
                   span(a->dt_bias, (u128)HC * 4, "dt_bias"),
                   span(a->state_indices, rows_extent(N, a->indices_stride, a->max_tokens) * 4, "state_indices"),
                   span(a->query_start_loc, (u128)(N + 1) * 4, "query_start_loc"),
                   span(a->num_accepted_tokens, (u128)N * 4, "num_accepted_tokens"),
                   span(a->output_gate, rows_extent(R, a->ogate_stride, HC) * 2, "output_gate"),
                   span(a->norm_weight, (u128)KD * 4, "norm_weight"),
                   Range{0, 0, ""}};
    rc = check_alias(w, 5, r, 11);
    if (rc) return rc;
    const int64_t items = N * a->H;
    const PfGeometry geo = packed_fused_geometry(items, can_split, a->state_dtype == KDA_DTYPE_BF16);
    if (items * geo.vs > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "too many work items");
    l->family = KERNEL_PACKED_FUSED;
    l->vsplit = geo.vs;
    l->rows_per_block = KD / geo.vs;
    l->grid = (int32_t)(items * geo.vs);
    l->block = geo.block;
    l->bf16_state = a->state_dtype == KDA_DTYPE_BF16;

    p->x = static_cast<const uint16_t *>(a->x);
    p->x_stride = a->x_stride;
    p->weight = a->weight;
    p->conv_state = static_cast<uint16_t *>(a->conv_state);
    p->conv_slot_stride = a->conv_slot_stride;
    p->graw = static_cast<const uint16_t *>(a->raw_gate);
    p->g_stride = a->gate_stride;
    p->braw = static_cast<const uint16_t *>(a->raw_beta);
    p->beta_stride = a->beta_stride;
    p->A_log = a->A_log;
    p->dt_bias = a->dt_bias;
    p->state_indices = a->state_indices;
    p->indices_stride = a->indices_stride;
    p->qsl = a->query_start_loc;
    p->accepted = a->num_accepted_tokens;
    p->state = a->state;
    p->num_slots = a->num_slots;
    p->slot_stride = a->slot_stride;
    p->ogate = static_cast<const uint16_t *>(a->output_gate);
    p->ogate_stride = a->ogate_stride;
    p->norm_weight = a->norm_weight;
    p->norm_eps = a->norm_eps;
    p->scale = 1.0f / sqrtf((float)KD);
    p->l2_eps = 1e-6f;
    p->out = static_cast<uint16_t *>(a->out);
    p->counters = a->split_counters;
    p->partials = a->split_partials;
    p->n_rows = a->n_rows;
    p->n_seqs = a->n_seqs;
    p->H = a->H;
    p->max_tokens = a->max_tokens;
    return ok();
}

int check_current_device()
{
    int dev = -1;
    int r = current_device_is_gfx950(&dev);
    if (r < 0) return fail(KDA_ERR_DEVICE, "HIP error while querying the device: %s", last_hip_error());
    if (r == 0) return fail(KDA_ERR_DEVICE, "device %d is not a gfx950 (MI355X)", dev);
    return KDA_OK;
}

int launched(int rc)
{
    if (rc) return fail(KDA_ERR_LAUNCH, "kernel launch failed: %s", last_hip_error());
    return ok();
}

}  // namespace

extern "C" {

KDA_API int kda_recurrent_plan(const kda_recurrent_args *args, kda_launch_plan *plan)
{
    RecParams p;
    Launch l;
    int rc = prepare_recurrent(args, &p, &l);
    if (rc) return rc;
    fill_plan(plan, l, (int64_t)args->n_seqs * args->HV);
    return KDA_OK;
}

KDA_API int kda_recurrent(const kda_recurrent_args *args, void *stream)
{
    RecParams p;
    Launch l;
    int rc = prepare_recurrent(args, &p, &l);
    if (rc) return rc;
    if (args->n_tokens == 0) return ok();  // every sequence is empty: nothing to do
    rc = check_current_device();
    if (rc) return rc;
    return launched(launch_recurrent(p, l, stream));
}

KDA_API int kda_packed_plan(const kda_packed_args *args, kda_launch_plan *plan)
{
    kda_recurrent_args r;
    int rc = packed_to_recurrent(args, &r);
    if (rc) return rc;
    return kda_recurrent_plan(&r, plan);
}

KDA_API int kda_packed_decode(const kda_packed_args *args, void *stream)
{
    kda_recurrent_args r;
    int rc = packed_to_recurrent(args, &r);
    if (rc) return rc;
    return kda_recurrent(&r, stream);
}

KDA_API int kda_fused_plan(const kda_fused_args *args, kda_launch_plan *plan)
{
    FusedParams p;
    Launch l;
    int rc = prepare_fused(args, &p, &l);
    if (rc) return rc;
    fill_plan(plan, l, (int64_t)args->rows * args->H);
    return KDA_OK;
}

KDA_API int kda_fused_decode(const kda_fused_args *args, void *stream)
{
    FusedParams p;
    Launch l;
    int rc = prepare_fused(args, &p, &l);
    if (rc) return rc;
    rc = check_current_device();
    if (rc) return rc;
    return launched(launch_fused(p, l, stream));
}

KDA_API int kda_packed_fused_plan(const kda_packed_fused_args *args, kda_launch_plan *plan)
{
    PackedFusedParams p;
    Launch l;
    int rc = prepare_packed_fused(args, &p, &l);
    if (rc) return rc;
    fill_plan(plan, l, (int64_t)args->n_seqs * args->H);
    return KDA_OK;
}

KDA_API int kda_packed_fused_workspace(const kda_packed_fused_args *args, int64_t *counter_bytes,
                                      int64_t *partial_bytes)
{
    if (!counter_bytes || !partial_bytes) return fail(KDA_ERR_NULLPTR, "counter_bytes / partial_bytes is NULL");
    *counter_bytes = *partial_bytes = 0;
    if (args && (args->split_counters || args->split_partials))
        return fail(KDA_ERR_UNSUPPORTED, "split_counters and split_partials must be NULL when sizing them");
    PackedFusedParams p;
    Launch l;
    int rc = prepare_packed_fused(args, &p, &l, true);
    if (rc) return rc;
    if (l.vsplit > 1) {
        *counter_bytes = (int64_t)args->n_seqs * args->H * 4;
        *partial_bytes = (int64_t)args->n_rows * args->H * KD * 4;
    }
    return KDA_OK;
}

KDA_API int kda_packed_fused_decode(const kda_packed_fused_args *args, void *stream)
{
    PackedFusedParams p;
    Launch l;
    int rc = prepare_packed_fused(args, &p, &l);
    if (rc) return rc;
    rc = check_current_device();
    if (rc) return rc;
    return launched(launch_packed_fused(p, l, stream));
}

KDA_API int kda_packed_fused_decode_noalloc(const kda_packed_fused_args *args, void *stream)
{
    if (!args) return fail(KDA_ERR_NULLPTR, "args is NULL");
    if (args->struct_size != sizeof(kda_packed_fused_args))
        return fail(KDA_ERR_ABI, "struct_size %u != %zu", args->struct_size, sizeof(kda_packed_fused_args));
    if (args->split_counters || args->split_partials)
        return fail(KDA_ERR_UNSUPPORTED,
                    "kda_packed_fused_decode_noalloc uses the library's own split scratch: "
                    "split_counters and split_partials must be NULL");
    int rc = check_current_device();
    if (rc) return rc;
    void *scratch = nullptr;
    if (noalloc_scratch(&scratch))
        return fail(KDA_ERR_LAUNCH, "cannot locate the library's scratch array: %s", last_hip_error());
    kda_packed_fused_args a = *args;
    a.split_counters = static_cast<int32_t *>(scratch);
    a.split_partials = reinterpret_cast<float *>(static_cast<char *>(scratch) + NOALLOC_COUNTER_BYTES);
    PackedFusedParams p;
    Launch l;
    rc = prepare_packed_fused(&a, &p, &l);
    if (rc) return rc;
    if (l.vsplit > 1) {
        const int64_t cb = (int64_t)a.n_seqs * a.H * 4;
        const int64_t pb = (int64_t)a.n_rows * a.H * KD * 4;
        if (cb > NOALLOC_COUNTER_BYTES || pb > NOALLOC_PARTIAL_BYTES)
            return fail(KDA_ERR_SHAPE,
                        "this call splits its heads and needs %lld bytes of counters and %lld of outputs; "
                        "the allocation-free entry point holds %lld and %lld (n_rows*H <= %lld)",
                        (long long)cb, (long long)pb, (long long)NOALLOC_COUNTER_BYTES,
                        (long long)NOALLOC_PARTIAL_BYTES, (long long)(NOALLOC_PARTIAL_BYTES / (KD * 4)));
    }
    return launched(launch_packed_fused(p, l, stream));
}

KDA_API const char *kda_status_string(int status)
{
    switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULLPTR: return "null pointer";
    case KDA_ERR_SHAPE: return "invalid shape";
    case KDA_ERR_DTYPE: return "invalid dtype";
    case KDA_ERR_STRIDE: return "invalid stride";
    case KDA_ERR_ALIGN: return "misaligned pointer or stride";
    case KDA_ERR_ALIAS: return "aliasing buffers";
    case KDA_ERR_UNSUPPORTED: return "unsupported mode";
    case KDA_ERR_DEVICE: return "unsupported device";
    case KDA_ERR_LAUNCH: return "kernel launch failed";
    case KDA_ERR_ABI: return "ABI struct size mismatch";
    default: return "unknown status";
    }
}

KDA_API const char *kda_last_error(void) { return g_err; }

KDA_API int kda_version(void) { return KDA_ABI_VERSION; }

KDA_API int kda_check_device(int device)
{
    int r = device_is_gfx950(device);
    if (r < 0) return fail(KDA_ERR_DEVICE, "HIP error while querying device %d: %s", device, last_hip_error());
    if (r == 0) return fail(KDA_ERR_DEVICE, "device %d is not a gfx950 (MI355X)", device);
    return ok();
}

}  // extern "C"
