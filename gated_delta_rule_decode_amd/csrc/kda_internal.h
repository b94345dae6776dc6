// kda_internal.h -- parameter blocks passed from the host validator to the
// gfx950 kernels of libkda_mi355x.so (not part of the public ABI).
#pragma once
#include <stdint.h>

namespace kda_detail {

constexpr int KD = 128;  // K = V = 128

enum KernelFamily : int32_t {
    KERNEL_RECURRENT_T1 = 1,   // one token per sequence
    KERNEL_RECURRENT_VARLEN = 2,  // ragged token loop with the state held in registers
    KERNEL_FUSED = 3,          // conv + SiLU -> KDA -> gated RMSNorm
    KERNEL_PACKED_FUSED = 4,   // the fused step over packed ragged rows, T >= 1 per sequence
    KERNEL_VERIFY_WY = 5,      // read-only calls, <= VERIFY_WY_MAX_T tokens per sequence: one MFMA product per head
};

constexpr int VERIFY_WY_MAX_T = 16;   // tokens per sequence the WY verify kernel takes

// Recurrence over (sequence, value head, value slice) work items; serves
// recurrent_kda (T=1, uniform batches, ragged T>=0, grouped value heads,
// in-kernel or precomputed gate, state-updating or read-only) and
// packed_kda_decode.
struct RecParams {
    const uint16_t *q, *k, *v;   // bf16
    const void *g, *beta;        // bf16 or fp32 (g_f32, beta_f32)
    int64_t q_stride, k_stride, v_stride, g_stride, beta_stride;  // per token, elements
    const float *A_log, *dt_bias;  // in-kernel gate only
    float scale, l2_eps;
    void *state;                 // fp32 or bf16 pool, [slot][hv][v][k]
    int64_t num_slots, slot_stride;
    const int32_t *state_indices;
    const int32_t *cu_seqlens;   // nullptr: sequence i owns tokens [i*tps, (i+1)*tps)
    void *ckpt;                  // nullptr or [n_tokens][HV][128][128], state dtype
    uint16_t *out;               // bf16 [n_tokens][HV][128]
    int32_t n_seqs, n_tokens, H, HV;
    int32_t group;               // HV / H: value heads per q/k head
    int32_t tps;                 // tokens per sequence without cu_seqlens (>= 1); with cu_seqlens
                                 // in the WY verify kernel, the declared longest sequence
    int32_t g_f32, beta_f32;     // input dtypes of g and beta
    int32_t precomputed;         // 1: g is the log-decay and beta is beta itself
    int32_t update_state;        // 0: the pool is read only
    int32_t vsplit;              // workgroups per (sequence, value head)
    int32_t n_work;              // n_seqs * HV * vsplit (grid is padded to a multiple of 8)
    float *corr;                 // nullptr or fp32 [num_slots][HV][t_max][128]
    void *kg;                    // nullptr or [num_slots][HV][t_max][256], kg_f32 ? fp32 : bf16
    int32_t kg_f32;
    int32_t t_max;
};

struct FusedParams {
    const uint16_t *x;
    int64_t x_stride;
    const float *weight;         // [3][4][H*128]
    uint16_t *conv_state;
    int64_t conv_slot_stride;
    const uint16_t *graw;
    int64_t g_stride;
    const uint16_t *braw;
    int64_t beta_stride;
    const float *A_log, *dt_bias;
    const int32_t *state_indices;
    void *state;
    int64_t num_slots, slot_stride;
    const uint16_t *ogate;
    int64_t ogate_stride;
    const float *norm_weight;
    float norm_eps, scale, l2_eps;
    uint16_t *out;               // bf16 [rows][H][128]
    int32_t rows, H;
};

// Packed fused decode: one workgroup per (sequence, head), token loop with
// the state and the conv window in registers, one checkpoint per token.
struct PackedFusedParams {
    const uint16_t *x;
    int64_t x_stride;
    const float *weight;         // [3][4][H*128]
    uint16_t *conv_state;        // [slot][3][3*H*128], slot stride conv_slot_stride
    int64_t conv_slot_stride;
    const uint16_t *graw;
    int64_t g_stride;
    const uint16_t *braw;
    int64_t beta_stride;
    const float *A_log, *dt_bias;
    const int32_t *state_indices;  // [n_seqs][max_tokens], row stride indices_stride
    int64_t indices_stride;
    const int32_t *qsl;            // [n_seqs + 1]
    const int32_t *accepted;       // [n_seqs]
    void *state;
    int64_t num_slots, slot_stride;
    const uint16_t *ogate;
    int64_t ogate_stride;
    const float *norm_weight;
    float norm_eps, scale, l2_eps;
    uint16_t *out;               // bf16 [n_rows][H][128]
    int32_t *counters;           // [n_seqs][H] arrivals per head (split heads); zero between calls
    float *partials;             // fp32 [n_rows][H][128] unnormalised outputs (split heads)
    int32_t n_rows, n_seqs, H, max_tokens;
};

// Scratch of the allocation-free packed fused entry point, one array per
// device held by the library: arrival counters of split heads (int32), then
// their unnormalised outputs (fp32).
constexpr int64_t NOALLOC_COUNTER_BYTES = 4096;          // 1024 (sequence, head) pairs
constexpr int64_t NOALLOC_PARTIAL_BYTES = 4 << 20;       // 8192 (row, head) pairs of 128 values
constexpr int64_t NOALLOC_SCRATCH_BYTES = NOALLOC_COUNTER_BYTES + NOALLOC_PARTIAL_BYTES;

struct Launch {
    int32_t family;
    int32_t rows_per_block;  // 16 * G
    int32_t vsplit;
    int32_t grid;
    int32_t block;
    int32_t bf16_state;
};

// Implemented in kda_kernels.hip.  Return 0 or a negative kda_status.
int launch_recurrent(const RecParams &p, const Launch &l, void *stream);
int launch_fused(const FusedParams &p, const Launch &l, void *stream);
int launch_packed_fused(const PackedFusedParams &p, const Launch &l, void *stream);
// Device address of the current device's copy of the allocation-free
// scratch array (NOALLOC_SCRATCH_BYTES); 0 or a negative kda_status.
int noalloc_scratch(void **ptr);
int current_device_is_gfx950(int *device_out);  // 1 yes, 0 no, <0 HIP error
int device_is_gfx950(int device);
const char *last_hip_error();

}  // namespace kda_detail
