/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA decode library, libkda_mi355x.so.
 *
 * KDA (Kimi Delta Attention) decode: per (sequence, head) a 128 x 128 state
 * S (K x V) is updated by a gated delta rule with one decay per key channel,
 *     S <- diag(exp g) S;  u = v - S^T k;  S <- S + beta k u^T;  o = scale S^T q,
 * with q and k L2-normalised in the kernel, g = -exp(A_log[h]) *
 * softplus(raw_g + dt_bias) and beta = sigmoid(raw_beta).  Pages followed:
 * "flashinfer.kda_decode" (function table; backend="cake" section for the
 * in-kernel gate; "Serving-native packed Kimi K3 decode"), the
 * "flashinfer.kda_decode.fused_kda_decode" Parameters list, and the PRs
 * "feat(cake_kda): add serving-native packed decode backend" (Exact
 * contract) and "feat(kda): add fused speculative decode kernel" (#4809,
 * packed ragged T>=2 decode with per-token state checkpoints).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers in the argument structs are DEVICE pointers owned by the
 *    caller, unless stated otherwise.  The library allocates nothing, never
 *    synchronises and never reads device memory on the host, so every call
 *    can be captured into a HIP graph.  Each successful call enqueues exactly
 *    one kernel on `stream` (a hipStream_t; NULL = the null stream), except a
 *    ragged recurrent call with n_tokens == 0, which enqueues nothing.
 *  - State pools have logical shape [num_slots, H, 128, 128] and store the
 *    state transposed: element (slot, h, v, k) = S[k][v], at
 *        state + slot*slot_stride + (h*128 + v)*128 + k     (elements).
 *    The inner [H, 128, 128] block of each slot is contiguous; slot_stride
 *    (in elements) is any value >= H*128*128 that keeps the 16-byte
 *    alignment.  State dtype is fp32 or bf16; the recurrence runs in fp32 and
 *    a bf16 state is rounded to nearest-even when written back
 *    ("fused_kda_decode" Parameters: state).
 *  - state_indices is a contiguous int32 array, one per row / sequence (the
 *    packed fused call takes a table of checkpoint columns per sequence,
 *    described with its arguments).
 *    Null rows produce +0 outputs and leave every cache untouched
 *    ("Serving-native packed Kimi K3 decode": -1 is inactive padding;
 *    "fused_kda_decode" Parameters: non-positive indices are null, slot 0 is
 *    reserved).  Indices >= num_slots also take the null path (no memory
 *    access).  Active slots must be unique within one call (caller contract).
 *  - bf16 data are IEEE-754 binary32 upper halves (uint16 bit patterns).
 *  - Strides are in elements.  Errors are decided from the host-visible
 *    arguments only; a failed call launches nothing and returns a negative
 *    kda_status; kda_last_error() then gives a message (thread-local).
 *    There is no fallback path.
 */
#ifndef KDA_MI355X_H
#define KDA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_API __attribute__((visibility("default")))
#define KDA_ABI_VERSION 6
#define KDA_HEAD_DIM 128

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULLPTR = -1,     /* a required pointer is NULL */
    KDA_ERR_SHAPE = -2,       /* sizes out of range or inconsistent */
    KDA_ERR_DTYPE = -3,       /* unknown dtype code */
    KDA_ERR_STRIDE = -4,      /* a stride is too small */
    KDA_ERR_ALIGN = -5,       /* a base or stride breaks 16-byte alignment */
    KDA_ERR_ALIAS = -6,       /* an output overlaps an input or another output */
    KDA_ERR_UNSUPPORTED = -7, /* a mode the library does not implement */
    KDA_ERR_DEVICE = -8,      /* the current device is not gfx950 */
    KDA_ERR_LAUNCH = -9,      /* the HIP launch failed */
    KDA_ERR_ABI = -10         /* struct_size does not match this library */
} kda_status;

typedef enum kda_dtype { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1 } kda_dtype;

/* Gate transform.  SOFTPLUS: g = -exp(A_log[h]) * softplus(raw + dt_bias)
 * and beta = sigmoid(logit) (the Kimi-Linear in-kernel gate, lower_bound=None
 * on the pages).  PRECOMPUTED (recurrent_kda only; use_gate_in_kernel=False
 * on the flashinfer.kda_decode page): g is the log-decay itself (decay =
 * exp(g)) and beta is beta itself; A_log and dt_bias are not read.
 * LOWER_BOUND: the bounded Kimi K3 gate; the pages name it but do not define
 * it, so every call asking for it returns KDA_ERR_UNSUPPORTED. */
typedef enum kda_gate_mode {
    KDA_GATE_SOFTPLUS = 0,
    KDA_GATE_LOWER_BOUND = 1,
    KDA_GATE_PRECOMPUTED = 2
} kda_gate_mode;

/* kda_recurrent_args.flags */
#define KDA_FLAG_NO_STATE_UPDATE 1u /* read-only pool (speculative verify) */

/* Launch geometry chosen from host metadata only (for inspection/tests). */
typedef struct kda_launch_plan {
    uint32_t struct_size;
    int32_t kernel;          /* internal kernel family id */
    int32_t grid_x;          /* workgroups */
    int32_t block;           /* threads per workgroup */
    int32_t rows_per_block;  /* value rows of one (row, head) per workgroup */
    int32_t vsplit;          /* workgroups per (row, head) = 128 / rows_per_block */
    int64_t items;           /* (row or sequence) x head work items */
} kda_launch_plan;

/*
 * recurrent_kda ("flashinfer.kda_decode" function table: recurrent_kda with
 * one token per sequence (T=1) and packed speculative decode with T>=2;
 * "Frozen / speculative-verify mode": disable_state_update=True reads a
 * committed pool and never writes it back, for the batched [B, T, ...] form
 * and the packed cu_seqlens form).
 *
 *  n_seqs            sequences (rows), >= 1.
 *  n_tokens          tokens: n_seqs * max(1, tokens_per_seq) when cu_seqlens
 *                    is NULL; otherwise cu_seqlens[n_seqs], >= 0.
 *  H, HV             q/k heads and value heads; HV must be a multiple of H.
 *                    Value head hv reads q/k head hv / (HV / H); the state,
 *                    v, g, beta, A_log, dt_bias and the output are per value
 *                    head.
 *  K, V              must both be 128.
 *  q, k              bf16, token t head h at ptr + t*X_stride + h*128 (the
 *                    inner [H,128] is contiguous).
 *  v, g              v bf16, g in g_dtype; token t value head hv at
 *                    ptr + t*X_stride + hv*128 (inner [HV,128] contiguous).
 *                    g is the raw gate (SOFTPLUS) or the log-decay
 *                    (PRECOMPUTED).
 *  beta              in beta_dtype, token t value head hv at
 *                    beta + t*beta_stride + hv: logits (SOFTPLUS) or beta
 *                    itself (PRECOMPUTED).
 *  A_log, dt_bias    fp32 [HV] and fp32 [HV*128], contiguous (SOFTPLUS only;
 *                    may be NULL for PRECOMPUTED).
 *  scale             output scale (the pages use 1/sqrt(128)).
 *  l2_eps            q/k L2-norm epsilon (the pages use 1e-6), >= 0.
 *  gate_mode         kda_gate_mode (LOWER_BOUND is unsupported).
 *  lower_bound       ignored unless LOWER_BOUND.
 *  state             pool [num_slots, HV, 128, 128] as described above;
 *                    state_dtype its kda_dtype.
 *  num_slots         slots in the pool, >= 1; slot_stride in elements.
 *  state_indices     int32 [n_seqs]; idx < 0 or idx >= num_slots is null.
 *  cu_seqlens        NULL, or int32 [n_seqs+1], cu_seqlens[0] == 0,
 *                    non-decreasing (read on the device at every launch, so a
 *                    captured graph follows new lengths; n_tokens must match
 *                    its last entry).  Empty sequences touch nothing.
 *  checkpoints       NULL or [n_tokens, HV, 128, 128] contiguous in the
 *                    pool's [v][k] layout, dtype ckpt_dtype (= state_dtype):
 *                    the state after each token.  Null sequences write none.
 *  out               bf16 [n_tokens, HV, 128] contiguous.
 *  g_dtype, beta_dtype  kda_dtype of g and beta (bf16 or fp32).
 *  tokens_per_seq    without cu_seqlens: 0 or 1 is T=1, T > 1 is the uniform
 *                    batched form (sequence i owns tokens [i*T, (i+1)*T)).
 *                    With cu_seqlens: 0, or the length of the longest
 *                    sequence as declared by the caller (a caller contract).
 *                    A read-only call without checkpoints that declares at
 *                    most 16 takes the matrix-product form below; there, the
 *                    tokens of a sequence past the declared length (a broken
 *                    contract) give +0 outputs and record nothing.  Other
 *                    ragged calls ignore it.
 *  flags             KDA_FLAG_NO_STATE_UPDATE: the pool is only read.  The
 *                    outputs are those of the updating call; read-only calls
 *                    without checkpoints whose sequences have at most 16
 *                    tokens (batched T >= 2, or ragged with tokens_per_seq
 *                    declared) evaluate them in another order (one matrix
 *                    product per head, "Frozen / speculative-verify mode"),
 *                    equal up to rounding.
 *  correction_cache  NULL or fp32 [num_slots, HV, cache_t_max, 128], contiguous,
 *                    16-byte aligned ("Frozen / speculative-verify mode":
 *                    slot-indexed per-token delta-rule corrections): for token
 *                    j of a live sequence in slot s, [s, hv, j, :] receives
 *                    beta * u, the vector the update adds along k_hat
 *                    (S_j = D_j S_{j-1} + k_hat_j c_j^T).
 *  kg_cache          NULL or [num_slots, HV, cache_t_max, 256] of kg_dtype,
 *                    contiguous: [s, hv, j, 0:128] the raw key of the value
 *                    head's q/k head (before L2 normalisation), [.., 128:256]
 *                    the raw gate as given (the log-decay when PRECOMPUTED).
 *                    Positions j >= cache_t_max are not recorded; null and
 *                    empty sequences record nothing.
 *  kg_dtype          kda_dtype of kg_cache (fp32 keeps fp32 gates exactly).
 *  cache_t_max       tokens recorded per (slot, value head), >= 1 when a cache
 *                    is given.
 */
typedef struct kda_recurrent_args {
    uint32_t struct_size;
    int32_t n_seqs;
    int32_t n_tokens;
    int32_t H;
    int32_t HV;
    int32_t K;
    int32_t V;
    const void *q;
    const void *k;
    const void *v;
    const void *g;
    const void *beta;
    int64_t q_stride;
    int64_t k_stride;
    int64_t v_stride;
    int64_t g_stride;
    int64_t beta_stride;
    const float *A_log;
    const float *dt_bias;
    float scale;
    float l2_eps;
    int32_t gate_mode;
    float lower_bound;
    void *state;
    int32_t state_dtype;
    int32_t ckpt_dtype;
    int64_t num_slots;
    int64_t slot_stride;
    const int32_t *state_indices;
    const int32_t *cu_seqlens;
    void *checkpoints;
    void *out;
    int32_t g_dtype;
    int32_t beta_dtype;
    int32_t tokens_per_seq;
    uint32_t flags;
    void *correction_cache;
    void *kg_cache;
    int32_t kg_dtype;
    int32_t cache_t_max;
} kda_recurrent_args;

/*
 * packed_kda_decode ("Serving-native packed Kimi K3 decode" on the
 * flashinfer.kda_decode page; Exact contract of "feat(cake_kda): add
 * serving-native packed decode backend").  T=1.  Fixed scale 1/sqrt(128)
 * and L2 epsilon 1e-6.  The pages fix H=12 and a bf16 pool; this library
 * accepts any H >= 1 and an fp32 or bf16 pool.
 *
 *  B                 rows, >= 1.
 *  mixed_qkv         bf16 [B, 3*H*128] post-convolution projection: q at
 *                    [0, H*128), k at [H*128, 2*H*128), v at [2*H*128,
 *                    3*H*128); row stride qkv_stride >= 3*H*128.
 *  raw_gate          bf16 [B, H*128], row stride gate_stride.
 *  raw_beta          bf16 [B, H], row stride beta_stride.
 *  state_indices     int32 [B]; -1 (any negative) is an inactive row.
 *  out               bf16 [B, 1, H, 128] contiguous.
 */
typedef struct kda_packed_args {
    uint32_t struct_size;
    int32_t B;
    int32_t H;
    const void *mixed_qkv;
    int64_t qkv_stride;
    const void *raw_gate;
    int64_t gate_stride;
    const void *raw_beta;
    int64_t beta_stride;
    const float *A_log;
    const float *dt_bias;
    int32_t gate_mode;
    float lower_bound;
    void *state;
    int32_t state_dtype;
    int64_t num_slots;
    int64_t slot_stride;
    const int32_t *state_indices;
    void *out;
} kda_packed_args;

/*
 * fused_kda_decode ("flashinfer.kda_decode.fused_kda_decode": width-4
 * depthwise causal conv + SiLU, one KDA update, gated RMSNorm).
 *
 *  rows              decode rows, >= 1.
 *  x                 bf16 [rows, 3*H*128], channel-contiguous, row stride
 *                    x_stride.
 *  weight            fp32 [3, 4, H*128] contiguous: group (q|k|v), tap, channel.
 *                    Tap 3 multiplies the current x, taps 0..2 the cache.
 *  conv_state        bf16 cache [num_slots, 3*H*128, 3] with strides
 *                    [conv_slot_stride, 1, 3*H*128]: position p (0 = oldest)
 *                    of channel c at conv_state + slot*conv_slot_stride +
 *                    p*3*H*128 + c.  Shifted by one position for live rows.
 *  raw_gate          bf16 [rows, H*128] (row stride gate_stride).
 *  raw_beta          bf16 [rows, H] (row stride beta_stride).
 *  state_indices     int32 [rows]; live indices in [1, num_slots); idx <= 0
 *                    (and idx >= num_slots) are null.
 *  state             fp32 or bf16 pool, same num_slots as conv_state.
 *  output_gate       bf16 [rows, H*128] logits (row stride ogate_stride).
 *  norm_weight       fp32 [128].  norm_eps >= 0.
 *  out               bf16 [rows, H, 128] contiguous:
 *                    y = o / sqrt(mean(o^2) + eps) * w * sigmoid(gate).
 *  Scale 1/sqrt(128) and L2 epsilon 1e-6 as in the packed call.
 */
typedef struct kda_fused_args {
    uint32_t struct_size;
    int32_t rows;
    int32_t H;
    const void *x;
    int64_t x_stride;
    const float *weight;
    void *conv_state;
    int64_t conv_slot_stride;
    const void *raw_gate;
    int64_t gate_stride;
    const void *raw_beta;
    int64_t beta_stride;
    const float *A_log;
    const float *dt_bias;
    int32_t gate_mode;
    float lower_bound;
    const int32_t *state_indices;
    void *state;
    int32_t state_dtype;
    int64_t num_slots;
    int64_t slot_stride;
    const void *output_gate;
    int64_t ogate_stride;
    const float *norm_weight;
    float norm_eps;
    void *out;
} kda_fused_args;

/*
 * packed_fused_kda_decode ("feat(kda): add fused speculative decode kernel":
 * the fused conv + KDA + gated RMSNorm step over packed ragged rows with
 * T >= 1 tokens per sequence; caches updated from accepted-token metadata,
 * one conv and state checkpoint per token, empty and padding rows; its
 * bf16-pool follow-up: the recurrence stays fp32 across the tokens and each
 * checkpoint is rounded to bf16 when stored).
 *
 *  n_rows            packed token rows, >= 0.
 *  n_seqs            sequences, >= 1.
 *  max_tokens        columns of state_indices, >= 1.
 *  x, weight, conv_state, raw_gate, raw_beta, A_log, dt_bias, state,
 *  output_gate, norm_weight, norm_eps, out, gate_mode
 *                    as in kda_fused_args, per packed row (rows = n_rows).
 *  state_indices     int32 [n_seqs, max_tokens], row stride indices_stride
 *                    (>= max_tokens).  Column j of sequence i is the slot that
 *                    receives the conv window and the state after token j of
 *                    the sequence; a column <= 0 or >= num_slots (and any
 *                    token j >= max_tokens) writes no checkpoint.
 *  query_start_loc   int32 [n_seqs + 1], non-decreasing: sequence i owns rows
 *                    [qsl[i], qsl[i+1]) (clipped to [0, n_rows)).
 *  num_accepted_tokens
 *                    int32 [n_seqs]: sequence i starts from the conv window
 *                    and state of slot state_indices[i, a-1], a = this value.
 *                    A start slot <= 0 or >= num_slots, or a outside
 *                    1..max_tokens, makes the sequence null: its rows give +0
 *                    and it writes nothing.
 *  split_counters, split_partials
 *                    optional workspace, both or neither, owned by the caller.
 *                    With it, the work of one (sequence, head) may be spread
 *                    over several workgroups when there are too few pairs to
 *                    fill the device (kda_packed_fused_plan reports the split
 *                    as vsplit): int32 [n_seqs*H] arrival counters, which
 *                    must be zero when the call starts and are zero again
 *                    when it completes (zero-fill them once after
 *                    allocating), and fp32 [n_rows*H*128], 16-byte aligned,
 *                    for unnormalised outputs.  Calls that share them must
 *                    not overlap in time.  NULL: one workgroup per pair.  The
 *                    split changes only the summation order of the RMS norm
 *                    (outputs may move by one bf16 ulp); pools, conv caches
 *                    and everything else are identical bit for bit.
 *  Rows that belong to no sequence give +0.  All metadata is read on the
 *  device, so a captured graph may be replayed with new values.  Slots must
 *  not be shared between sequences of one call (they would race).
 */
typedef struct kda_packed_fused_args {
    uint32_t struct_size;
    int32_t n_rows;
    int32_t n_seqs;
    int32_t H;
    int32_t max_tokens;
    const void *x;
    int64_t x_stride;
    const float *weight;
    void *conv_state;
    int64_t conv_slot_stride;
    const void *raw_gate;
    int64_t gate_stride;
    const void *raw_beta;
    int64_t beta_stride;
    const float *A_log;
    const float *dt_bias;
    int32_t gate_mode;
    float lower_bound;
    const int32_t *state_indices;
    int64_t indices_stride;
    const int32_t *query_start_loc;
    const int32_t *num_accepted_tokens;
    void *state;
    int32_t state_dtype;
    int64_t num_slots;
    int64_t slot_stride;
    const void *output_gate;
    int64_t ogate_stride;
    const float *norm_weight;
    float norm_eps;
    void *out;
    int32_t *split_counters;
    float *split_partials;
} kda_packed_fused_args;

/* Validate and enqueue.  Return KDA_OK or a negative kda_status. */
KDA_API int kda_recurrent(const kda_recurrent_args *args, void *stream);
KDA_API int kda_packed_decode(const kda_packed_args *args, void *stream);
KDA_API int kda_fused_decode(const kda_fused_args *args, void *stream);
KDA_API int kda_packed_fused_decode(const kda_packed_fused_args *args, void *stream);

/*
 * Workspace a packed fused call would use (host only: no HIP call, no
 * device access).  With split_counters and split_partials NULL in `args`
 * (else KDA_ERR_UNSUPPORTED), validates the call as kda_packed_fused_decode
 * does and reports the bytes of split counters and of split outputs it
 * would use if given a workspace: both 0 when it would keep one workgroup
 * per (sequence, head) anyway, so a caller need not pass (or allocate) a
 * workspace for it.  On error both are 0.
 */
KDA_API int kda_packed_fused_workspace(const kda_packed_fused_args *args, int64_t *counter_bytes,
                                       int64_t *partial_bytes);

/*
 * Allocation-free packed fused decode, for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, results
 * and launch geometry as kda_packed_fused_decode, except that split_counters
 * and split_partials must be NULL (else KDA_ERR_UNSUPPORTED): when the call
 * splits its heads, their counters and unnormalised outputs live in a
 * scratch array the library holds on each device for the life of the process
 * (4 KiB of counters and 4 MiB of outputs per device).  A call that would
 * split and needs more (n_seqs*H > 1024 or n_rows*H > 8192) is rejected with
 * KDA_ERR_SHAPE before anything is launched; a call that does not split uses
 * no scratch.  The counters are zero when the library is loaded and every
 * call leaves them zero.  All calls on one device share that device's array:
 * calls that overlap in time on one device (two streams, or a graph replayed
 * beside an eager call) race on it and must not be made.  The call
 * allocates nothing and synchronises nothing; its first call on a device
 * looks up the device address of that device's copy of the array.
 */
KDA_API int kda_packed_fused_decode_noalloc(const kda_packed_fused_args *args, void *stream);

/* Validate only (no HIP call, no device access) and report the launch
 * geometry the matching entry point would use.  `plan` may be NULL. */
KDA_API int kda_recurrent_plan(const kda_recurrent_args *args, kda_launch_plan *plan);
KDA_API int kda_packed_plan(const kda_packed_args *args, kda_launch_plan *plan);
KDA_API int kda_fused_plan(const kda_fused_args *args, kda_launch_plan *plan);
KDA_API int kda_packed_fused_plan(const kda_packed_fused_args *args, kda_launch_plan *plan);

/*
 * Status, error detail, version and device checks.  In the backend="cake"
 * section of "flashinfer.kda_decode" each call checks its device and its
 * argument contract before it launches and fails, rather than running some
 * other implementation, when anything is outside that contract; these calls
 * report how such a check ended.
 */
/* Static text of a status code. */
KDA_API const char *kda_status_string(int status);
/* Detail of the last failure on the calling thread ("" if none). */
KDA_API const char *kda_last_error(void);
/* KDA_ABI_VERSION of the loaded library. */
KDA_API int kda_version(void);
/* KDA_OK if HIP device `device` is a gfx950 (the only architecture built),
 * else KDA_ERR_DEVICE; every entry point makes the same check on the current
 * device before it launches. */
KDA_API int kda_check_device(int device);

#ifdef __cplusplus
}
#endif

#endif /* KDA_MI355X_H */
