/*
 * kda_oracle.c -- plain fp64 CPU reference of the KDA decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check
 * and the benchmark's cpu_baseline leg may load this library.  It shares
 * no code, header, table or helper with the HIP path and must never be
 * used to produce a product result.
 *
 * Everything is evaluated in double precision with straightforward loops,
 * in the order the method states it; there is no blocking, fusion or
 * reordering.  bf16 inputs are widened exactly; results are rounded to the
 * storage format (bf16 round-to-nearest-even, or fp32 round-to-nearest)
 * only when they are written back, and are also returned unrounded.
 *
 * Sources (the flashinfer KDA decode pages):
 *  - "flashinfer.kda_decode" API page: recurrent_kda / packed_kda_decode /
 *    fused_kda_decode function table; the backend="cake" section (Kimi-Linear
 *    equal-head schedules evaluate -exp(A_log) * softplus(g + dt_bias) and a
 *    beta sigmoid in-kernel); the "Serving-native packed Kimi K3 decode"
 *    section (fused Q/K extraction and L2 normalisation, -1 inactive rows
 *    emit zeros without touching state).
 *  - "flashinfer.kda_decode.fused_kda_decode" page, Parameters: conv weight
 *    [3, 4, H*128], conv_state [num_slots, 3*H*128, 3] with strides
 *    [slot_stride, 1, 3*H*128], non-positive indices are null, the state is
 *    evaluated in fp32 and a bf16 state is rounded when written back,
 *    gated RMSNorm with output_gate logits and norm_weight[128].
 *  - "feat(cake_kda): add serving-native packed decode backend", Exact
 *    contract: scale 1/sqrt(128), L2 epsilon 1e-6.
 *  - "feat(kda): add fused speculative decode kernel" (#4809), Description and
 *    walkthrough: packed ragged T>=2 decode with per-token state checkpoints.
 *
 * The recurrence is Kimi Delta Attention (a gated delta rule with one decay
 * per key channel).  With S the K x V state of one (sequence, head):
 *     S <- diag(exp(g)) S;   u = v - S^T k;   S <- S + beta k u^T;
 *     o = scale * S^T q
 * with q, k L2-normalised.  Readings where the pages are silent:
 *  - the pool stores S transposed: pool[slot][h][v][k] = S[k][v]
 *    (the pages speak of value rows / value-row splits of the state);
 *  - L2 norm is x / sqrt(sum x^2 + eps);
 *  - the readout uses the updated state;
 *  - conv: history [c0, c1, c2, x] (oldest first) against taps 0..3, no
 *    bias, SiLU after; the cache afterwards holds [c1, c2, x];
 *  - gated RMSNorm: y = o / sqrt(mean(o^2) + eps) * w * sigmoid(gate) on the
 *    unrounded o;
 *  - a null row (index < 0, or <= 0 for the fused call, or >= num_slots)
 *    yields +0 outputs and writes no state, cache or checkpoint.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KD 128 /* K = V = 128 */

enum { KDAO_F32 = 0, KDAO_BF16 = 1, KDAO_F64 = 2 };

/* ---- bf16 storage format ------------------------------------------------ */

static double bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Nearest bf16 (8 significant bits, fp32 exponent range) to x, ties to
 * even, computed directly from the double (no intermediate fp32 rounding). */
uint16_t kdao_bf16_from_f64(double x)
{
    double r;
    if (isnan(x)) return 0x7FC0;
    if (x == 0.0 || isinf(x)) {
        r = x;
    } else {
        double ax = fabs(x);
        if (ax < 0x1p-126) {
            /* subnormal range: quantum 2^-133 */
            r = nearbyint(x * 0x1p133) * 0x1p-133;
        } else {
            int e;
            double m = frexp(x, &e);          /* x = m * 2^e, 0.5 <= |m| < 1 */
            double q = nearbyint(m * 256.0);  /* 8 significant bits, RNE */
            r = ldexp(q, e - 8);
        }
        /* 0x1.FEp127 is the largest bf16; anything rounding above it is inf */
        if (fabs(r) > 0x1.FEp127) r = copysign(INFINITY, x);
    }
    float f = (float)r; /* exact: r is representable in bf16 */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static double load_elem(const void *p, int dt, size_t i)
{
    switch (dt) {
    case KDAO_F32: return (double)((const float *)p)[i];
    case KDAO_BF16: return bf16_to_f64(((const uint16_t *)p)[i]);
    default: return ((const double *)p)[i];
    }
}

static void store_elem(void *p, int dt, size_t i, double x)
{
    switch (dt) {
    case KDAO_F32: ((float *)p)[i] = (float)x; break; /* round to nearest */
    case KDAO_BF16: ((uint16_t *)p)[i] = kdao_bf16_from_f64(x); break;
    default: ((double *)p)[i] = x; break;
    }
}

/* ---- scalar functions ---------------------------------------------------- */

static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* x / sqrt(sum x^2 + eps) over one 128-vector */
static void l2_normalise(const double *x, double eps, double *out)
{
    double ss = 0.0;
    for (int i = 0; i < KD; ++i) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss + eps);
    for (int i = 0; i < KD; ++i) out[i] = x[i] * inv;
}

/* Gate transform of the Kimi-Linear KDA layer:
 *   g_k = -exp(A_log[h]) * softplus(raw_k + dt_bias[h*128 + k]),  decay = exp(g) */
static void gate_decay(const double *raw, double A_log_h, const float *dt_bias_h,
                       double *decay)
{
    double a = exp(A_log_h);
    for (int i = 0; i < KD; ++i) {
        double g = -a * softplus(raw[i] + (double)dt_bias_h[i]);
        decay[i] = exp(g);
    }
}

/* One token of the recurrence on S[k][v] (math orientation, K x V).
 * qh, kh are the L2-normalised vectors; o receives scale * S'^T q; corr (may
 * be NULL) receives the delta-rule correction beta * u, the vector the
 * update adds along k: S' = D S + k corr^T. */
static void kda_token(double S[KD][KD], const double *qh, const double *kh,
                      const double *v, const double *decay, double beta,
                      double scale, double *o, double *corr)
{
    /* S <- diag(exp g) S : row k of S scaled by decay[k] */
    for (int k = 0; k < KD; ++k)
        for (int j = 0; j < KD; ++j) S[k][j] *= decay[k];
    /* u = v - S^T k */
    double u[KD];
    for (int j = 0; j < KD; ++j) {
        double acc = 0.0;
        for (int k = 0; k < KD; ++k) acc += S[k][j] * kh[k];
        u[j] = v[j] - acc;
    }
    /* S <- S + beta k u^T */
    for (int k = 0; k < KD; ++k)
        for (int j = 0; j < KD; ++j) S[k][j] += beta * kh[k] * u[j];
    if (corr)
        for (int j = 0; j < KD; ++j) corr[j] = beta * u[j];
    /* o = scale * S^T q */
    for (int j = 0; j < KD; ++j) {
        double acc = 0.0;
        for (int k = 0; k < KD; ++k) acc += S[k][j] * qh[k];
        o[j] = scale * acc;
    }
}

/* pool[slot][h][v][k] holds S[k][v] */
static void gather_state(const void *pool, int dt, size_t head_base, double S[KD][KD])
{
    for (int v = 0; v < KD; ++v)
        for (int k = 0; k < KD; ++k)
            S[k][v] = load_elem(pool, dt, head_base + (size_t)v * KD + k);
}

static void scatter_state(void *pool, int dt, size_t head_base, double S[KD][KD])
{
    for (int v = 0; v < KD; ++v)
        for (int k = 0; k < KD; ++k)
            store_elem(pool, dt, head_base + (size_t)v * KD + k, S[k][v]);
}

static void widen_bf16(const uint16_t *src, double *dst, int n)
{
    for (int i = 0; i < n; ++i) dst[i] = bf16_to_f64(src[i]);
}

/*
 * Recurrent KDA: T=1 (cu_seqlens == NULL and tokens_per_seq <= 1, one token
 * per sequence), uniform batches of tokens_per_seq tokens per sequence, or
 * packed ragged T>=0 per sequence (cu_seqlens [n_seqs+1]); tokens are
 * processed in order with the state carried between them.
 *
 * Heads: H q/k heads and HV value heads, HV a multiple of H; value head hv
 * reads q/k head hv / (HV/H) (grouped value heads).  The state, v, the gate,
 * beta, A_log and dt_bias are per value head.
 *
 * gate_mode 0 (in-kernel gate): g is the raw gate, decay = exp(-exp(A_log) *
 * softplus(g + dt_bias)) and beta holds logits, beta = sigmoid(logit).
 * gate_mode 1 (precomputed): g is the log-decay (decay = exp(g)) and beta is
 * beta itself; A_log and dt_bias are not read.
 * update_state 0: the pool is read only (speculative verify); outputs and
 * checkpoints are produced as usual.
 * Verify caches (slot-indexed, position j = t - t0 inside the sequence, only
 * for j < t_max, live sequences only):
 *   corr [num_slots][HV][t_max][128]: the delta-rule correction beta * u of
 *   the token, so that S_t = D_t S_{t-1} + k_hat_t corr_t^T;
 *   kg   [num_slots][HV][t_max][256]: the raw key of the value head's q/k
 *   head (before L2 normalisation) and the raw gate as given (the log-decay
 *   in precomputed mode).
 *
 * Layouts (all contiguous, host memory):
 *   q, k: bf16 [n_tokens][H][128];  v: bf16 [n_tokens][HV][128]
 *   g: [n_tokens][HV][128] and beta: [n_tokens][HV], each bf16 or fp32
 *   (g_f32, beta_f32);  A_log fp32 [HV];  dt_bias fp32 [HV*128]
 *   state: [num_slots][HV][128 v][128 k] of state_dtype
 *   out64 (may be NULL) double [n_tokens][HV][128];  out_bf16 (may be NULL)
 *   ckpt (may be NULL): [n_tokens][HV][128 v][128 k] of ckpt_dtype, the state
 *   after each token;  ckpt64 (may be NULL) the same in double.
 * Returns 0, or -1 on inconsistent metadata.
 */
static double load_in(const void *p, int is_f32, size_t i)
{
    return is_f32 ? (double)((const float *)p)[i] : bf16_to_f64(((const uint16_t *)p)[i]);
}

int kdao_recurrent3(int64_t n_tokens, int64_t n_seqs, int64_t H, int64_t HV,
                    const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const void *g, int g_f32, const void *beta, int beta_f32, int gate_mode,
                    const float *A_log, const float *dt_bias,
                    double scale, double l2_eps,
                    const int32_t *cu_seqlens, int64_t tokens_per_seq,
                    const int32_t *state_indices, int64_t num_slots, int state_dtype,
                    void *state, int update_state,
                    double *out64, uint16_t *out_bf16,
                    int ckpt_dtype, void *ckpt, double *ckpt64,
                    int64_t t_max, double *corr, double *kg)
{
    if (n_tokens < 0 || n_seqs < 0 || H <= 0 || HV <= 0 || HV % H != 0) return -1;
    const int64_t tps = tokens_per_seq > 1 ? tokens_per_seq : 1;
    if (!cu_seqlens && n_tokens != n_seqs * tps) return -1;
    if (cu_seqlens) {
        if (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] != n_tokens) return -1;
        for (int64_t i = 0; i < n_seqs; ++i)
            if (cu_seqlens[i + 1] < cu_seqlens[i]) return -1;
    }
    const int64_t group = HV / H;
    double (*S)[KD] = malloc(sizeof(double) * KD * KD);
    if (!S) return -2;
    double qv[KD], kv[KD], vv[KD], gv[KD], qh[KD], kh[KD], dec[KD], o[KD];

    const size_t head_elems = (size_t)KD * KD;
    for (int64_t i = 0; i < n_seqs; ++i) {
        int64_t t0 = cu_seqlens ? cu_seqlens[i] : i * tps;
        int64_t t1 = cu_seqlens ? cu_seqlens[i + 1] : (i + 1) * tps;
        int32_t idx = state_indices[i];
        int null_row = idx < 0 || (int64_t)idx >= num_slots;
        for (int64_t hv = 0; hv < HV; ++hv) {
            const int64_t hk = hv / group;
            if (null_row) {
                for (int64_t t = t0; t < t1; ++t)
                    for (int j = 0; j < KD; ++j) {
                        size_t oi = ((size_t)t * HV + hv) * KD + j;
                        if (out64) out64[oi] = 0.0;
                        if (out_bf16) out_bf16[oi] = 0;
                    }
                continue;
            }
            if (t1 == t0) continue; /* empty sequence: nothing read or written */
            size_t head_base = ((size_t)idx * HV + hv) * head_elems;
            gather_state(state, state_dtype, head_base, S);
            for (int64_t t = t0; t < t1; ++t) {
                size_t vq = ((size_t)t * H + hk) * KD;   /* q/k head of this value head */
                size_t vh = ((size_t)t * HV + hv) * KD;  /* value-head vectors */
                widen_bf16(q + vq, qv, KD);
                widen_bf16(k + vq, kv, KD);
                widen_bf16(v + vh, vv, KD);
                for (int j = 0; j < KD; ++j) gv[j] = load_in(g, g_f32, vh + j);
                double bin = load_in(beta, beta_f32, (size_t)t * HV + hv);
                double b;
                if (gate_mode == 0) {
                    b = sigmoid(bin);
                    gate_decay(gv, (double)A_log[hv], dt_bias + hv * KD, dec);
                } else {
                    b = bin;
                    for (int j = 0; j < KD; ++j) dec[j] = exp(gv[j]);
                }
                l2_normalise(qv, l2_eps, qh);
                l2_normalise(kv, l2_eps, kh);
                double c[KD];
                kda_token(S, qh, kh, vv, dec, b, scale, o, c);
                const int64_t pos = t - t0; /* token position inside the sequence */
                if (pos < t_max) {
                    size_t cs = (((size_t)idx * HV + hv) * t_max + pos);
                    if (corr)
                        for (int j = 0; j < KD; ++j) corr[cs * KD + j] = c[j];
                    if (kg)
                        for (int j = 0; j < KD; ++j) {
                            kg[cs * 2 * KD + j] = kv[j];      /* raw key of the q/k head */
                            kg[cs * 2 * KD + KD + j] = gv[j]; /* raw gate (or log-decay) */
                        }
                }
                for (int j = 0; j < KD; ++j) {
                    if (out64) out64[vh + j] = o[j];
                    if (out_bf16) out_bf16[vh + j] = kdao_bf16_from_f64(o[j]);
                }
                size_t cb = ((size_t)t * HV + hv) * head_elems;
                if (ckpt) scatter_state(ckpt, ckpt_dtype, cb, S);
                if (ckpt64) scatter_state(ckpt64, KDAO_F64, cb, S);
            }
            if (update_state) scatter_state(state, state_dtype, head_base, S);
        }
    }
    free(S);
    return 0;
}

/* kdao_recurrent3 without the verify caches. */
int kdao_recurrent2(int64_t n_tokens, int64_t n_seqs, int64_t H, int64_t HV,
                    const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const void *g, int g_f32, const void *beta, int beta_f32, int gate_mode,
                    const float *A_log, const float *dt_bias,
                    double scale, double l2_eps,
                    const int32_t *cu_seqlens, int64_t tokens_per_seq,
                    const int32_t *state_indices, int64_t num_slots, int state_dtype,
                    void *state, int update_state,
                    double *out64, uint16_t *out_bf16,
                    int ckpt_dtype, void *ckpt, double *ckpt64)
{
    return kdao_recurrent3(n_tokens, n_seqs, H, HV, q, k, v, g, g_f32, beta, beta_f32, gate_mode,
                           A_log, dt_bias, scale, l2_eps, cu_seqlens, tokens_per_seq,
                           state_indices, num_slots, state_dtype, state, update_state, out64,
                           out_bf16, ckpt_dtype, ckpt, ckpt64, 0, NULL, NULL);
}

/* The equal-head, in-kernel-gate, state-updating form of kdao_recurrent2. */
int kdao_recurrent(int64_t n_tokens, int64_t n_seqs, int64_t H,
                   const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   const uint16_t *graw, const uint16_t *braw,
                   const float *A_log, const float *dt_bias,
                   double scale, double l2_eps,
                   const int32_t *cu_seqlens, const int32_t *state_indices,
                   int64_t num_slots, int state_dtype, void *state,
                   double *out64, uint16_t *out_bf16,
                   int ckpt_dtype, void *ckpt, double *ckpt64)
{
    return kdao_recurrent2(n_tokens, n_seqs, H, H, q, k, v, graw, 0, braw, 0, 0, A_log, dt_bias,
                           scale, l2_eps, cu_seqlens, 1, state_indices, num_slots, state_dtype,
                           state, 1, out64, out_bf16, ckpt_dtype, ckpt, ckpt64);
}

/*
 * Fused decode: width-4 depthwise causal conv + SiLU over the packed
 * q|k|v projection, one KDA token, gated RMSNorm.
 *
 *   x bf16 [rows][3*H*128];  weight fp32 [3][4][H*128]
 *   conv_state bf16, slot s, position p, channel c at
 *       conv_state[s*conv_slot_stride + p*3*H*128 + c]   (updated in place)
 *   graw bf16 [rows][H][128];  braw bf16 [rows][H]
 *   state [num_slots][H][128 v][128 k] of state_dtype (updated in place)
 *   ogate bf16 [rows][H][128];  norm_weight fp32 [128]
 *   out64 / out_bf16: [rows][H][128] (either may be NULL)
 *   o_pre64 (may be NULL): [rows][H][128] the recurrence output before norm
 *   act64 (may be NULL): [rows][3*H*128] the post-SiLU conv activations
 */
int kdao_fused(int64_t rows, int64_t H, const uint16_t *x, const float *weight,
               int64_t num_slots, uint16_t *conv_state, int64_t conv_slot_stride,
               const uint16_t *graw, const uint16_t *braw,
               const float *A_log, const float *dt_bias,
               const int32_t *state_indices, int state_dtype, void *state,
               const uint16_t *ogate, const float *norm_weight, double norm_eps,
               double scale, double l2_eps,
               double *out64, uint16_t *out_bf16, double *o_pre64, double *act64)
{
    if (rows < 0 || H <= 0) return -1;
    const int64_t HC = H * KD;     /* channels per q/k/v group */
    const int64_t C3 = 3 * HC;     /* channels of the packed projection */
    if (conv_slot_stride < 3 * C3) return -1;
    double (*S)[KD] = malloc(sizeof(double) * KD * KD);
    double *act = malloc(sizeof(double) * (size_t)C3);
    if (!S || !act) { free(S); free(act); return -2; }
    double qh[KD], kh[KD], gv[KD], dec[KD], o[KD];
    const size_t head_elems = (size_t)KD * KD;

    for (int64_t b = 0; b < rows; ++b) {
        int32_t idx = state_indices[b];
        int null_row = idx <= 0 || (int64_t)idx >= num_slots;
        if (null_row) {
            for (int64_t i = 0; i < HC; ++i) {
                size_t oi = (size_t)b * HC + i;
                if (out64) out64[oi] = 0.0;
                if (out_bf16) out_bf16[oi] = 0;
                if (o_pre64) o_pre64[oi] = 0.0;
            }
            if (act64)
                for (int64_t c = 0; c < C3; ++c) act64[(size_t)b * C3 + c] = 0.0;
            continue;
        }
        /* depthwise causal conv, width 4, then SiLU; shift the cache */
        uint16_t *cs = conv_state + (size_t)idx * conv_slot_stride;
        for (int64_t c = 0; c < C3; ++c) {
            int64_t grp = c / HC, cc = c % HC;
            double hist[4];
            hist[0] = bf16_to_f64(cs[0 * C3 + c]);
            hist[1] = bf16_to_f64(cs[1 * C3 + c]);
            hist[2] = bf16_to_f64(cs[2 * C3 + c]);
            hist[3] = bf16_to_f64(x[(size_t)b * C3 + c]);
            double y = 0.0;
            for (int j = 0; j < 4; ++j)
                y += (double)weight[(grp * 4 + j) * HC + cc] * hist[j];
            act[c] = y * sigmoid(y);
            cs[0 * C3 + c] = cs[1 * C3 + c];
            cs[1 * C3 + c] = cs[2 * C3 + c];
            cs[2 * C3 + c] = x[(size_t)b * C3 + c];
        }
        if (act64)
            for (int64_t c = 0; c < C3; ++c) act64[(size_t)b * C3 + c] = act[c];
        for (int64_t h = 0; h < H; ++h) {
            const double *qa = act + 0 * HC + h * KD;
            const double *ka = act + 1 * HC + h * KD;
            const double *va = act + 2 * HC + h * KD;
            size_t vec = ((size_t)b * H + h) * KD;
            widen_bf16(graw + vec, gv, KD);
            double beta = sigmoid(bf16_to_f64(braw[(size_t)b * H + h]));
            l2_normalise(qa, l2_eps, qh);
            l2_normalise(ka, l2_eps, kh);
            gate_decay(gv, (double)A_log[h], dt_bias + h * KD, dec);
            size_t head_base = ((size_t)idx * H + h) * head_elems;
            gather_state(state, state_dtype, head_base, S);
            kda_token(S, qh, kh, va, dec, beta, scale, o, NULL);
            scatter_state(state, state_dtype, head_base, S);
            /* gated RMSNorm over the 128 values of this head */
            double ms = 0.0;
            for (int j = 0; j < KD; ++j) ms += o[j] * o[j];
            ms /= (double)KD;
            double inv = 1.0 / sqrt(ms + norm_eps);
            for (int j = 0; j < KD; ++j) {
                double y = o[j] * inv * (double)norm_weight[j] *
                           sigmoid(bf16_to_f64(ogate[vec + j]));
                if (out64) out64[vec + j] = y;
                if (out_bf16) out_bf16[vec + j] = kdao_bf16_from_f64(y);
                if (o_pre64) o_pre64[vec + j] = o[j];
            }
        }
    }
    free(S);
    free(act);
    return 0;
}

/*
 * Packed fused decode with T >= 1 tokens per sequence ("feat(kda): add fused
 * speculative decode kernel": packed ragged rows from query_start_loc,
 * caches updated from accepted-token metadata, per-token conv and state
 * checkpoints, empty and padding rows; the bf16-pool follow-up: the
 * recurrence stays unrounded across the token loop and each checkpoint is
 * rounded when stored).
 *
 * Readings (the pages give the signature and these behaviours, not the
 * index arithmetic):
 *  - sequence i owns packed rows [qsl[i], qsl[i+1]) (clipped to the rows);
 *  - state_indices is [n_seqs][max_tokens]: column j names the slot that
 *    receives the conv window and the state after token j; the sequence
 *    starts from the slot of column a-1, a = num_accepted[i] (the last
 *    accepted checkpoint of the previous step);
 *  - a start slot that is <= 0, >= num_slots, or a outside 1..max_tokens
 *    makes the sequence null: its rows give +0 and nothing is written;
 *  - a checkpoint column <= 0 or >= num_slots (or a token j >= max_tokens)
 *    is padding: that token writes no cache, the loop goes on;
 *  - rows that belong to no sequence give +0.
 * conv_state is position-major [slots][3][3*H*128] (the fused call's
 * layout); ckpt64 (optional) receives the unrounded state after each token,
 * pool layout [row][h][v][k].
 */
int kdao_packed_fused(int64_t n_rows, int64_t n_seqs, int64_t H, int64_t max_tokens,
                      const uint16_t *x, const float *weight,
                      int64_t num_slots, uint16_t *conv_state, int64_t conv_slot_stride,
                      const uint16_t *graw, const uint16_t *braw,
                      const float *A_log, const float *dt_bias,
                      const int32_t *state_indices, const int32_t *query_start_loc,
                      const int32_t *num_accepted, int state_dtype, void *state,
                      const uint16_t *ogate, const float *norm_weight, double norm_eps,
                      double scale, double l2_eps,
                      double *out64, uint16_t *out_bf16, double *o_pre64, double *act64,
                      double *ckpt64)
{
    if (n_rows < 0 || n_seqs < 0 || H <= 0 || max_tokens < 1) return -1;
    const int64_t HC = H * KD;
    const int64_t C3 = 3 * HC;
    if (conv_slot_stride < 3 * C3) return -1;
    const size_t head_elems = (size_t)KD * KD;

    /* every row starts as +0; live sequences overwrite theirs */
    for (size_t i = 0; i < (size_t)n_rows * HC; ++i) {
        if (out64) out64[i] = 0.0;
        if (out_bf16) out_bf16[i] = 0;
        if (o_pre64) o_pre64[i] = 0.0;
    }
    if (act64) memset(act64, 0, sizeof(double) * (size_t)n_rows * C3);
    if (ckpt64) memset(ckpt64, 0, sizeof(double) * (size_t)n_rows * H * head_elems);

    double (*S)[KD][KD] = malloc(sizeof(double) * (size_t)H * head_elems);
    uint16_t *win = malloc(sizeof(uint16_t) * 3 * (size_t)C3);  /* [3][C3], oldest first */
    double *act = malloc(sizeof(double) * (size_t)C3);
    if (!S || !win || !act) { free(S); free(win); free(act); return -2; }
    double qh[KD], kh[KD], gv[KD], dec[KD], o[KD];

    for (int64_t i = 0; i < n_seqs; ++i) {
        int64_t t0 = query_start_loc[i], t1 = query_start_loc[i + 1];
        t0 = t0 < 0 ? 0 : (t0 > n_rows ? n_rows : t0);
        t1 = t1 < t0 ? t0 : (t1 > n_rows ? n_rows : t1);
        const int32_t *cols = state_indices + (size_t)i * max_tokens;
        int32_t a = num_accepted[i];
        int32_t src = (a >= 1 && a <= max_tokens) ? cols[a - 1] : -1;
        if (src <= 0 || (int64_t)src >= num_slots || t1 <= t0) continue;

        /* the accepted checkpoint: conv window and every head's state */
        memcpy(win, conv_state + (size_t)src * conv_slot_stride, sizeof(uint16_t) * 3 * (size_t)C3);
        for (int64_t h = 0; h < H; ++h)
            gather_state(state, state_dtype, ((size_t)src * H + h) * head_elems, S[h]);

        for (int64_t r = t0; r < t1; ++r) {
            const int64_t j = r - t0;  /* token position inside the sequence */
            /* conv over [window, x_r], SiLU; the window advances by x_r */
            for (int64_t c = 0; c < C3; ++c) {
                int64_t grp = c / HC, cc = c % HC;
                double hist[4] = {bf16_to_f64(win[c]), bf16_to_f64(win[C3 + c]),
                                  bf16_to_f64(win[2 * C3 + c]), bf16_to_f64(x[(size_t)r * C3 + c])};
                double y = 0.0;
                for (int t = 0; t < 4; ++t) y += (double)weight[(grp * 4 + t) * HC + cc] * hist[t];
                act[c] = y * sigmoid(y);
                win[c] = win[C3 + c];
                win[C3 + c] = win[2 * C3 + c];
                win[2 * C3 + c] = x[(size_t)r * C3 + c];
            }
            if (act64) memcpy(act64 + (size_t)r * C3, act, sizeof(double) * (size_t)C3);
            for (int64_t h = 0; h < H; ++h) {
                size_t vec = ((size_t)r * H + h) * KD;
                widen_bf16(graw + vec, gv, KD);
                double beta = sigmoid(bf16_to_f64(braw[(size_t)r * H + h]));
                l2_normalise(act + h * KD, l2_eps, qh);
                l2_normalise(act + HC + h * KD, l2_eps, kh);
                gate_decay(gv, (double)A_log[h], dt_bias + h * KD, dec);
                kda_token(S[h], qh, kh, act + 2 * HC + h * KD, dec, beta, scale, o, NULL);
                double ms = 0.0;
                for (int v = 0; v < KD; ++v) ms += o[v] * o[v];
                double inv = 1.0 / sqrt(ms / (double)KD + norm_eps);
                for (int v = 0; v < KD; ++v) {
                    double y = o[v] * inv * (double)norm_weight[v] * sigmoid(bf16_to_f64(ogate[vec + v]));
                    if (out64) out64[vec + v] = y;
                    if (out_bf16) out_bf16[vec + v] = kdao_bf16_from_f64(y);
                    if (o_pre64) o_pre64[vec + v] = o[v];
                }
                if (ckpt64) {
                    double *ck = ckpt64 + ((size_t)r * H + h) * head_elems;
                    for (int v = 0; v < KD; ++v)
                        for (int k = 0; k < KD; ++k) ck[(size_t)v * KD + k] = S[h][k][v];
                }
            }
            /* checkpoint of token j: window and state (rounded on store) */
            int32_t dst = j < max_tokens ? cols[j] : -1;
            if (dst > 0 && (int64_t)dst < num_slots) {
                memcpy(conv_state + (size_t)dst * conv_slot_stride, win, sizeof(uint16_t) * 3 * (size_t)C3);
                for (int64_t h = 0; h < H; ++h)
                    scatter_state(state, state_dtype, ((size_t)dst * H + h) * head_elems, S[h]);
            }
        }
    }
    free(S);
    free(win);
    free(act);
    return 0;
}

/* Element-wise kdao_bf16_from_f64 over an array (test helper). */
void kdao_bf16_from_f64_n(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = kdao_bf16_from_f64(x[i]);
}
