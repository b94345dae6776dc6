// kda_kernels.hip -- gfx950 (CDNA4) kernels of the KDA decode step.
//
// The step is matrix-vector work on a 128 x 128 state per (row, head): per
// value row it needs two 128-long dot products (k.S and q.S), a rank-1
// update and one output value, i.e. ~7 flop per state element against 8
// (fp32) or 4 (bf16) bytes of HBM read+write.  That is far below the
// MFMA/VALU ridge, so the kernels are built for HBM streaming, not matrix
// cores:
//
//  * A workgroup of 256 threads (4 wave64) owns one (row, head) and a slice
//    of VT = 16*G value rows.  Inside a wave the 16 lanes of one DPP row own
//    one value row at a time; lane m holds 8 key channels of it, so one
//    value row's dot products reduce with four DPP adds inside the DPP row
//    (quad_perm x2, row_half_mirror, row_mirror) and no LDS traffic.
//  * The state slice is loaded once with dwordx4 accesses into VGPRs
//    (64 VGPRs at G=8 fp32, 32 packed at bf16), updated in registers and
//    written back with dwordx4 stores.  For fp32 a lane owns key channels
//    {4m..4m+3} and {64+4m..64+4m+3}, so each load instruction of the 16
//    lanes covers 256 contiguous bytes of one value row; for bf16 a lane owns
//    {8m..8m+7} and one instruction covers a whole 256-byte value row.
//  * Per token, threads 0..255 stage q, k, v and the per-channel decay in
//    LDS (the gate transform is evaluated once per channel) and two waves
//    reduce the L2 norm sums of q and k into LDS partials; after one barrier
//    every lane reads its 8 channels.  The token loop (ragged, batched and
//    verify calls) stages CHUNK tokens at a time: one round of loads and one
//    barrier per chunk, then the chunk's tokens back to back.
//  * The fused kernels (conv + SiLU -> KDA -> gated RMSNorm) give each thread
//    its conv channels' windows in registers, reduce the norm sums in the
//    DPP rows and the RMS over the head's 128 outputs in LDS; the packed
//    fused kernel carries the state and the conv windows across a
//    sequence's tokens and, when few heads are live, splits a head over
//    2-4 workgroups that exchange unnormalised outputs through caller
//    scratch (the last to arrive normalises).
//  * Read-only calls with up to 16 tokens (speculative verify) are the
//    exception: every token's product with the state is a product with the
//    same initial state, so they run as one small matrix product per head on
//    the matrix cores plus a forward substitution per value row
//    (kda_verify_wy_kernel; the state is read as whole rows and reaches the
//    matrix-core layout through LDS).
//  * The slot base is one 64-bit pointer per workgroup; everything inside a
//    head is 32-bit offsets.
//  * Null rows (index below the call's first live index, or >= num_slots)
//    write zeros and touch no state.
//
// Pages: "flashinfer.kda_decode" (recurrent_kda T=1 and packed T>=2;
// Kimi-Linear in-kernel gate -exp(A_log)*softplus(g+dt_bias), beta sigmoid;
// packed Kimi K3 decode with -1 inactive rows), "flashinfer.kda_decode.
// fused_kda_decode" (Parameters), "feat(cake_kda): add serving-native packed
// decode backend" (Exact contract: scale 1/sqrt(128), L2 eps 1e-6) and
// "feat(kda): add fused speculative decode kernel" (per-token checkpoints).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "kda_internal.h"

namespace kda_detail {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- bf16 ----

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even), low half first: built as
// a two-element vector, which is one v_cvt_pk_bf16_f32 of both values (two
// scalar conversions joined by a shift and an or took four instructions).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Lanes of one wave hand data to each other through LDS: the release fence
// orders this lane's earlier LDS accesses before the barrier and the acquire
// fence its later ones after it, in the compiler's memory model (at wavefront
// scope neither emits an instruction; one wave's LDS accesses complete in
// order).  A bare wave barrier does not order memory accesses.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// s_waitcnt vmcnt(0): every vector memory access of this wave has completed
// (gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15 are "no wait" for the others).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Tokens staged per chunk by the token loops (measured on MI355X: the
// recurrent loop keeps the next chunk's inputs in registers through the
// current chunk, and two tokens per chunk keep it at 4 waves per SIMD; the
// packed fused loop has two barriers per chunk and prefers longer chunks).
constexpr int CHUNK = 2;
constexpr int PF_CHUNK = 8;

// ---------------------------------------------------------- reductions ----

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row.  Every lane of the row ends with the
// same bits (each step adds two equal-valued partners, and + commutes).
__device__ __forceinline__ float row_sum16(float x)
{
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);  // row_half_mirror
    x += dpp_mov<0x140>(x);  // row_mirror
    return x;
}

// Transpose-reduce over the 64 lanes of a wave: x[0..P) in every lane (P a
// power of two, 2 <= P <= 64) -> in lane l the wave total of value
// l >> (6 - log2 P).  Each halving step exchanges half the values with the
// partner lane at one distance (32 and 16: permlane swaps; 8, 4, 2, 1: DPP)
// and keeps the other half, so P sums cost about 2P operations instead of
// six each; distances left once one value remains reduce it in place.
template <int CTRL, int N>
__device__ __forceinline__ void halve_dpp(float *x, bool up)
{
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float a = x[i], b = x[i + N];
        const float send = up ? a : b, keep = up ? b : a;
        x[i] = keep + dpp_mov<CTRL>(send);
    }
}

__device__ __forceinline__ float swap32_sum(float a, float b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float swap16_sum(float a, float b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// one step at a DPP distance: halve N values, or reduce the last one in place
template <int CTRL, int N>
__device__ __forceinline__ void transpose_step(float *x, bool up)
{
    if constexpr (N >= 2) halve_dpp<CTRL, N / 2>(x, up);
    else x[0] += dpp_mov<CTRL>(x[0]);
}

template <int P>
__device__ __forceinline__ float wave_transpose_sum(float *x, int lane)
{
    static_assert(P >= 2 && P <= 64 && (P & (P - 1)) == 0, "P: a power of two in 2..64");
    constexpr int N1 = P / 2;                   // values left after distance 32
    constexpr int N2 = N1 >= 2 ? N1 / 2 : 1;    // ... 16
    constexpr int N3 = N2 >= 2 ? N2 / 2 : 1;    // ... 8
    constexpr int N4 = N3 >= 2 ? N3 / 2 : 1;    // ... 4
    constexpr int N5 = N4 >= 2 ? N4 / 2 : 1;    // ... 2
#pragma unroll
    for (int i = 0; i < N1; ++i) x[i] = swap32_sum(x[i], x[i + N1]);
    if constexpr (N1 >= 2) {
#pragma unroll
        for (int i = 0; i < N1 / 2; ++i) x[i] = swap16_sum(x[i], x[i + N1 / 2]);
    } else {
        x[0] = swap16_sum(x[0], x[0]);
    }
    transpose_step<0x140, N2>(x, lane & 8);  // row_mirror: lane m <-> 15 - m
    transpose_step<0x141, N3>(x, lane & 4);  // row_half_mirror: m <-> 7 - m
    transpose_step<0x4E, N4>(x, lane & 2);   // quad_perm [2,3,0,1]
    transpose_step<0xB1, N5>(x, lane & 1);   // quad_perm [1,0,3,2]
    return x[0];
}

__device__ __forceinline__ void row_sum16x2(float &a, float &b)
{
    a += dpp_mov<0xB1>(a); b += dpp_mov<0xB1>(b);
    a += dpp_mov<0x4E>(a); b += dpp_mov<0x4E>(b);
    a += dpp_mov<0x141>(a); b += dpp_mov<0x141>(b);
    a += dpp_mov<0x140>(a); b += dpp_mov<0x140>(b);
}

__device__ __forceinline__ void row_sum16x3(float &a, float &b, float &c)
{
    a += dpp_mov<0xB1>(a); b += dpp_mov<0xB1>(b); c += dpp_mov<0xB1>(c);
    a += dpp_mov<0x4E>(a); b += dpp_mov<0x4E>(b); c += dpp_mov<0x4E>(c);
    a += dpp_mov<0x141>(a); b += dpp_mov<0x141>(b); c += dpp_mov<0x141>(c);
    a += dpp_mov<0x140>(a); b += dpp_mov<0x140>(b); c += dpp_mov<0x140>(c);
}

// ---------------------------------------------------------- scalar math ----

// softplus(x) = max(x, 0) + log(1 + e^-|x|) with the hardware exp2 and log2:
// the log's argument lies in (1, 2], so none of the library log's handling
// of denormal, infinite or negative inputs is needed (14 instructions of
// it per call); the absolute error stays near 1e-7, and for e^-|x| below
// 2^-24 the log term is lost, an absolute error under 6e-8.
__device__ __forceinline__ float softplus_f(float x)
{
    return fmaxf(x, 0.0f) + __builtin_amdgcn_logf(1.0f + __expf(-fabsf(x))) * 0.69314718f;
}
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

__device__ __forceinline__ float lane_value(float x, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// Sums over the 64 lanes of a wave (three at once); the results are
// wave-uniform.
__device__ __forceinline__ void wave_sum3(float &a, float &b, float &c)
{
    row_sum16x3(a, b, c);
    a = (lane_value(a, 0) + lane_value(a, 16)) + (lane_value(a, 32) + lane_value(a, 48));
    b = (lane_value(b, 0) + lane_value(b, 16)) + (lane_value(b, 32) + lane_value(b, 48));
    c = (lane_value(c, 0) + lane_value(c, 16)) + (lane_value(c, 32) + lane_value(c, 48));
}

// --------------------------------------------------------- state tiles ----
//
// A lane's share of one value row: 8 fp32 values (key channels kc(0..7)).
// StateIO<bf16> maps a lane to channels 8m..8m+7 (one 16-byte access of a
// 256-byte bf16 row); StateIO<fp32> maps it to 4m..4m+3 and 64+4m..64+4m+3
// (two 16-byte accesses, each instruction covering 256 contiguous bytes).

template <bool BF16> struct StateIO;

// Loads and stores address one head tile from its (workgroup-uniform) base
// with 32-bit byte offsets, so the 64-bit slot address is formed once.
// Cache policy of state traffic, measured on MI355X:
// pool loads and pool stores (in place, or checkpoints into pool slots)
// nontemporal — plain ones cost 8-9% at T=1; stores into the contiguous
// checkpoint buffer of the token loop plain — 13% faster than nontemporal
// on the ragged H=16 workload.
constexpr bool ST_NT = true;   // pool stores
constexpr bool CK_NT = false;  // stores into the contiguous checkpoint buffer

template <typename V>
__device__ __forceinline__ V ld_nt(const char *base, uint32_t off)
{
    return __builtin_nontemporal_load(reinterpret_cast<const V *>(base + off));
}
template <typename V, bool NT>
__device__ __forceinline__ void st_as(char *base, uint32_t off, V v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<V *>(base + off));
    else *reinterpret_cast<V *>(base + off) = v;
}

template <> struct StateIO<false> {
    static constexpr uint32_t ROW_BYTES = KD * 4;
    struct Raw { f32x4 a, b; };
    static __device__ __forceinline__ int chan(int m, int e) { return e < 4 ? 4 * m + e : 64 + 4 * m + (e - 4); }
    // byte offset of the lane's first access in value row `row`
    static __device__ __forceinline__ uint32_t off(int row, int m) { return (uint32_t)row * ROW_BYTES + 16u * m; }
    static __device__ __forceinline__ Raw load(const char *head, uint32_t o)
    {
        Raw r;
        r.a = ld_nt<f32x4>(head, o);
        r.b = ld_nt<f32x4>(head, o + 256u);
        return r;
    }
    static __device__ __forceinline__ void unpack(const Raw &r, float s[8])
    {
        s[0] = r.a.x; s[1] = r.a.y; s[2] = r.a.z; s[3] = r.a.w;
        s[4] = r.b.x; s[5] = r.b.y; s[6] = r.b.z; s[7] = r.b.w;
    }
    static __device__ __forceinline__ Raw pack(const float s[8])
    {
        Raw r;
        r.a = f32x4{s[0], s[1], s[2], s[3]};
        r.b = f32x4{s[4], s[5], s[6], s[7]};
        return r;
    }
    template <bool NT = ST_NT>
    static __device__ __forceinline__ void store(char *head, uint32_t o, const Raw &r)
    {
        st_as<f32x4, NT>(head, o, r.a);
        st_as<f32x4, NT>(head, o + 256u, r.b);
    }
    static __device__ __forceinline__ void store_ckpt(char *head, uint32_t o, const Raw &r)
    {
        store<CK_NT>(head, o, r);
    }
};

template <> struct StateIO<true> {
    static constexpr uint32_t ROW_BYTES = KD * 2;
    struct Raw { u32x4 w; };
    static __device__ __forceinline__ int chan(int m, int e) { return 8 * m + e; }
    static __device__ __forceinline__ uint32_t off(int row, int m) { return (uint32_t)row * ROW_BYTES + 16u * m; }
    static __device__ __forceinline__ Raw load(const char *head, uint32_t o)
    {
        Raw r;
        r.w = ld_nt<u32x4>(head, o);
        return r;
    }
    static __device__ __forceinline__ void unpack(const Raw &r, float s[8])
    {
        s[0] = bf16_lo(r.w.x); s[1] = bf16_hi(r.w.x);
        s[2] = bf16_lo(r.w.y); s[3] = bf16_hi(r.w.y);
        s[4] = bf16_lo(r.w.z); s[5] = bf16_hi(r.w.z);
        s[6] = bf16_lo(r.w.w); s[7] = bf16_hi(r.w.w);
    }
    static __device__ __forceinline__ Raw pack(const float s[8])
    {
        Raw r;
        r.w = u32x4{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]),
                    pack_bf16x2(s[4], s[5]), pack_bf16x2(s[6], s[7])};
        return r;
    }
    template <bool NT = ST_NT>
    static __device__ __forceinline__ void store(char *head, uint32_t o, const Raw &r)
    {
        st_as<u32x4, NT>(head, o, r.w);
    }
    static __device__ __forceinline__ void store_ckpt(char *head, uint32_t o, const Raw &r)
    {
        store<CK_NT>(head, o, r);
    }
};

// Store G consecutive bf16 outputs (G in {1,2,4,8}) from one lane.
template <int G>
__device__ __forceinline__ void store_out_bf16(uint16_t *dst, const float *o)
{
    if constexpr (G == 8) {
        *reinterpret_cast<u32x4 *>(dst) =
            u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                  pack_bf16x2(o[6], o[7])};
    } else if constexpr (G == 4) {
        *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    } else if constexpr (G == 2) {
        *reinterpret_cast<uint32_t *>(dst) = pack_bf16x2(o[0], o[1]);
    } else {
        *dst = (uint16_t)(pack_bf16x2(o[0], 0.0f) & 0xffffu);
    }
}

template <int G>
__device__ __forceinline__ void store_zero_bf16(uint16_t *dst)
{
    float z[G];
#pragma unroll
    for (int i = 0; i < G; ++i) z[i] = 0.0f;
    store_out_bf16<G>(dst, z);
}

// Per-lane operands of one token: q, k (not normalised) and the decay at
// the lane's 8 key channels, plus the per-token scalars: beta,
// rk = 1/sqrt(|k|^2 + eps), rqs = scale/sqrt(|q|^2 + eps) and
// qk = scale * q_hat.k_hat.  The L2 normalisation is folded into these
// scalars instead of being applied to every channel.
struct TokenOps {
    float q[8], k[8], d[8];
    float beta, rk, rqs, qk;
};

// Channel values from LDS; the three norm sums either come from the
// staging waves (norms != nullptr: partials of waves 2 and 3) or are reduced
// here over the DPP row.
template <bool BF16>
__device__ __forceinline__ void read_token_ops(TokenOps &t, const float *sq, const float *sk,
                                               const float *sd, const float *norms, int m, float scale,
                                               float eps, float beta)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int c = StateIO<BF16>::chan(m, e);
        t.q[e] = sq[c];
        t.k[e] = sk[c];
        t.d[e] = sd[c];
    }
    float ss_q, ss_k, s_qk;
    if (norms) {
        ss_q = norms[0] + norms[4];
        ss_k = norms[1] + norms[5];
        s_qk = norms[2] + norms[6];
    } else {
        ss_q = 0.f, ss_k = 0.f, s_qk = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ss_q = fmaf(t.q[e], t.q[e], ss_q);
            ss_k = fmaf(t.k[e], t.k[e], ss_k);
            s_qk = fmaf(t.q[e], t.k[e], s_qk);
        }
        row_sum16x3(ss_q, ss_k, s_qk);
    }
    t.rqs = rsqrtf(ss_q + eps) * scale;
    t.rk = rsqrtf(ss_k + eps);
    t.qk = s_qk * t.rqs * t.rk;
    t.beta = beta;
}

// One token on one value row held as 8 fp32 values per lane:
//   s <- d*s;  a = k_hat.s;  c = scale*q_hat.s;  u = v - a;
//   s <- s + beta*u*k_hat;  o = c + beta*u*scale*(q_hat.k_hat)  (= scale*q_hat.s_new)
__device__ __forceinline__ float row_update(float s[8], const TokenOps &t, float v, float &bu_out)
{
    float pa = 0.f, pc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        s[e] *= t.d[e];
        pa = fmaf(t.k[e], s[e], pa);
        pc = fmaf(t.q[e], s[e], pc);
    }
    row_sum16x2(pa, pc);
    const float bu = t.beta * (v - pa * t.rk);
    const float bk = bu * t.rk;
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = fmaf(bk, t.k[e], s[e]);
    bu_out = bu;
    return fmaf(bu, t.qk, pc * t.rqs);
}

__device__ __forceinline__ float row_update(float s[8], const TokenOps &t, float v)
{
    float bu;
    return row_update(s, t, v, bu);
}

// Store G consecutive fp32 values (G in {1,2,4,8}) from one lane.
template <int G>
__device__ __forceinline__ void store_f32(float *dst, const float *x)
{
    if constexpr (G == 8) {
        reinterpret_cast<f32x4 *>(dst)[0] = f32x4{x[0], x[1], x[2], x[3]};
        reinterpret_cast<f32x4 *>(dst)[1] = f32x4{x[4], x[5], x[6], x[7]};
    } else if constexpr (G == 4) {
        *reinterpret_cast<f32x4 *>(dst) = f32x4{x[0], x[1], x[2], x[3]};
    } else if constexpr (G == 2) {
        *reinterpret_cast<float2 *>(dst) = float2{x[0], x[1]};
    } else {
        *dst = x[0];
    }
}

// One token's channel inputs, held in registers between their load and the
// LDS stage.  Every thread loads channel tid & 127 of q, k, v and the raw
// gate (no divergent branch around the loads, so the compiler does not wait
// on them before the state loads are issued); threads 0..127 then stage q,
// k and the decay, threads 128..255 stage v.  A gate or beta that may be
// fp32 or bf16 is fetched as two 16-bit halves whose addresses (not values)
// depend on the format, and is assembled only when staged: a select on the
// loaded values would make the compiler wait for the loads right away.
struct StageIn {
    uint32_t q, k, v;  // bf16 bits
    uint32_t g_lo, g_hi;  // fp32: the two halves; bf16: the value (g_hi unused)
};

// Two 16-bit halves of an fp32 or bf16 element at byte address `at`.
__device__ __forceinline__ void load_halves(const char *at, bool is_f32, uint32_t &lo, uint32_t &hi)
{
    lo = *reinterpret_cast<const uint16_t *>(at);
    hi = *reinterpret_cast<const uint16_t *>(at + (is_f32 ? 2 : 0));
}

__device__ __forceinline__ float halves_value(uint32_t lo, uint32_t hi, bool is_f32)
{
    return is_f32 ? __uint_as_float((hi << 16) | lo) : bf16_bits_to_f32(lo);
}

__device__ __forceinline__ StageIn load_stage(int tid, const uint16_t *q, const uint16_t *k,
                                              const uint16_t *v, const char *g, bool g_f32)
{
    const int c = tid & (KD - 1);
    StageIn s;
    s.q = q[c];
    s.k = k[c];
    s.v = v[c];
    load_halves(g + c * (g_f32 ? 4 : 2), g_f32, s.g_lo, s.g_hi);
    return s;
}

// Gate transform once per channel, decay = exp(-exp(A_log) * softplus(g +
// dt_bias), by threads 0..127; threads 128..255 stage v and reduce the three
// norm sums (|q|^2, |k|^2, q.k) over their wave, writing one partial per
// wave to norms[4 * (wave - 2) + {0, 1, 2}].
// With a precomputed gate, g already is the log-decay: decay = exp(g).
__device__ __forceinline__ void write_stage(int tid, const StageIn &s, float a_h, float dt, bool g_f32,
                                            bool precomputed, float *sq, float *sk, float *sd,
                                            float *sv, float *norms)
{
    const float q = bf16_bits_to_f32(s.q);
    const float k = bf16_bits_to_f32(s.k);
    if (tid < KD) {
        sq[tid] = q;
        sk[tid] = k;
        const float g = halves_value(s.g_lo, s.g_hi, g_f32);
        sd[tid] = precomputed ? __expf(g) : __expf(-a_h * softplus_f(g + dt));
    } else {
        sv[tid - KD] = bf16_bits_to_f32(s.v);
        float pq = q * q, pk = k * k, pqk = q * k;
        wave_sum3(pq, pk, pqk);
        if ((tid & 63) == 0) {
            float *n = norms + 4 * ((tid >> 6) - 2);
            n[0] = pq;
            n[1] = pk;
            n[2] = pqk;
        }
    }
}

// Verify cache row of one token: [raw key (128) | raw gate (128)], from the
// staging registers of threads 0..127 (channel tid), as fp32 or bf16.
__device__ __forceinline__ void store_kg(void *kg, bool kg_f32, int64_t row, int tid, const StageIn &s,
                                         bool g_f32)
{
    const int64_t at = row * (2 * KD) + tid;
    if (kg_f32) {
        float *d = static_cast<float *>(kg) + at;
        d[0] = bf16_bits_to_f32(s.k);
        d[KD] = halves_value(s.g_lo, s.g_hi, g_f32);
    } else {
        uint16_t *d = static_cast<uint16_t *>(kg) + at;
        d[0] = (uint16_t)s.k;
        d[KD] = g_f32 ? (uint16_t)(pack_bf16x2(halves_value(s.g_lo, s.g_hi, true), 0.0f) & 0xffffu)
                      : (uint16_t)s.g_lo;
    }
}

// ------------------------------------------------------- recurrent kernel ----

template <int G, bool BF16, bool VARLEN>
__global__ void __launch_bounds__(256) kda_recurrent_kernel(const RecParams p)
{
    using IO = StateIO<BF16>;
    constexpr int VT = 16 * G;  // value rows per workgroup

    // T=1: one token stage.  Token loop: a chunk of CHUNK tokens is staged at
    // once (one round of loads and one barrier per chunk).
    constexpr int NB = VARLEN ? CHUNK : 1;
    __shared__ float s_q[NB][KD], s_k[NB][KD], s_d[NB][KD], s_v[NB][KD];
    __shared__ float s_norm[NB][8];
    __shared__ float s_beta[NB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int m = lane & 15;   // position inside the DPP row
    const int qd = lane >> 4;  // DPP row inside the wave

    // Workgroups are handed to the 8 XCDs round-robin by block id; number
    // them so that each XCD walks one contiguous range of work and the
    // vsplit slices of one (sequence, head), which read the same q/k/v/g,
    // share an XCD and its L2.  The grid is padded to a multiple of 8.
    const int work = (int)(blockIdx.x & 7u) * (int)(gridDim.x >> 3) + (int)(blockIdx.x >> 3);
    if (work >= p.n_work) return;
    const int vs = work % p.vsplit;
    const int item = work / p.vsplit;
    const int seq = item / p.HV;
    const int hv = item - seq * p.HV;  // value head: state, v, gate, beta, output
    const int hq = hv / p.group;       // q/k head read by this value head
    const int r_base = vs * VT + wave * (4 * G) + qd * G;  // this lane's first value row

    int t0, t1;
    if constexpr (VARLEN) {
        if (p.cu_seqlens) {
            t0 = max(p.cu_seqlens[seq], 0);
            t1 = min(p.cu_seqlens[seq + 1], p.n_tokens);
        } else {
            t0 = seq * p.tps;
            t1 = min(t0 + p.tps, p.n_tokens);
        }
    } else {
        t0 = seq;
        t1 = seq + 1;
    }
    const int idx = p.state_indices[seq];
    const bool precomputed = p.precomputed != 0;
    const bool g_f32 = p.g_f32 != 0;
    const bool beta_f32 = p.beta_f32 != 0;
    const float dt = precomputed ? 0.f : p.dt_bias[(int64_t)hv * KD + (tid & (KD - 1))];
    const int64_t oq = (int64_t)hq * KD;
    const int64_t ov = (int64_t)hv * KD;
    const char *gbase = static_cast<const char *>(p.g);
    const char *bbase = static_cast<const char *>(p.beta);
    const int g_es = g_f32 ? 4 : 2;
    const int b_es = beta_f32 ? 4 : 2;
    auto g_at = [&](int64_t t) { return gbase + (t * p.g_stride + ov) * g_es; };
    auto beta_at = [&](int64_t t, uint32_t &lo, uint32_t &hi) {
        load_halves(bbase + (t * p.beta_stride + hv) * b_es, beta_f32, lo, hi);
    };

    // Token inputs first (the first chunk's in the token loop), even before
    // the slot index is known: they do not depend on it, so their latency
    // overlaps that of the index; waiting for them later must not wait for
    // the state either.  Token indices are clamped into [0, t1), so every
    // load is in bounds (n_tokens >= 1 whenever the kernel runs) and
    // unconditional; a null or empty sequence simply discards them.
    constexpr int NC = VARLEN ? CHUNK : 1;
    StageIn cin[NC];
    uint32_t blo[NC], bhi[NC];
    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int64_t n = max(min(c0 + i, t1 - 1), 0);
            cin[i] = load_stage(tid, p.q + n * p.q_stride + oq, p.k + n * p.k_stride + oq,
                                p.v + n * p.v_stride + ov, g_at(n), g_f32);
            beta_at(n, blo[i], bhi[i]);
        }
    };
    load_chunk(t0);
    const float a_h = precomputed ? 0.f : __expf(p.A_log[hv]);
    if (idx < 0 || (int64_t)idx >= p.num_slots) {
        if (m == 0)
            for (int t = t0; t < t1; ++t)
                store_zero_bf16<G>(p.out + ((int64_t)t * p.HV + hv) * KD + r_base);
        return;
    }
    if (t1 <= t0) return;
    const size_t es = BF16 ? 2 : 4;
    char *head = reinterpret_cast<char *>(p.state) + ((int64_t)idx * p.slot_stride + (int64_t)hv * (KD * KD)) * es;
    __builtin_amdgcn_sched_barrier(0);

    // Then every state load of this lane.
    typename IO::Raw raw[G];
    uint32_t off[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        off[gi] = IO::off(r_base + gi, m);
        raw[gi] = IO::load(head, off[gi]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // beta: sigmoid of the logits, or the precomputed value itself
    auto beta_of = [&](uint32_t lo, uint32_t hi) {
        const float b = halves_value(lo, hi, beta_f32);
        return precomputed ? b : sigmoid_f(b);
    };
    const bool update = p.update_state != 0;

    if constexpr (!VARLEN) {
        // T=1: the gate transform and the norms overlap the state fetch.
        const StageIn &in = cin[0];
        write_stage(tid, in, a_h, dt, g_f32, precomputed, s_q[0], s_k[0], s_d[0], s_v[0], s_norm[0]);
        const float beta = beta_of(blo[0], bhi[0]);
        __syncthreads();
        TokenOps ops;
        read_token_ops<BF16>(ops, s_q[0], s_k[0], s_d[0], s_norm[0], m, p.scale, p.l2_eps, beta);
        float o[G], c[G];
        // bf16 pools: every row first, then the stores.  A store (counted
        // with the loads in the in-order memory counter) under the read-only
        // branch between two rows made the second row wait for the first
        // row's store; measured 2-6% faster for H=12 bf16 at 64-512 rows.
        // fp32 pools keep each row's store next to its update (storing at
        // the end measured 13-15% slower for H=32 fp32 at 128-512 rows).
        constexpr bool STORE_LAST = BF16;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            float st[8];
            IO::unpack(raw[gi], st);
            o[gi] = row_update(st, ops, s_v[0][r_base + gi], c[gi]);
            raw[gi] = IO::pack(st);
            if (!STORE_LAST && update) IO::store(head, off[gi], raw[gi]);
        }
        if (STORE_LAST && update) {
#pragma unroll
            for (int gi = 0; gi < G; ++gi) IO::store(head, off[gi], raw[gi]);
        }
        if (m == 0) store_out_bf16<G>(p.out + ((int64_t)t0 * p.HV + hv) * KD + r_base, o);
        if (p.t_max > 0) {
            const int64_t row = ((int64_t)idx * p.HV + hv) * p.t_max;
            if (p.corr && m == 0) store_f32<G>(p.corr + row * KD + r_base, c);
            if (p.kg && vs == 0 && tid < KD) store_kg(p.kg, p.kg_f32 != 0, row, tid, in, g_f32);
        }
    } else {
        // Token loop in chunks of up to CHUNK tokens: the inputs of a whole
        // chunk are loaded at once (the first chunk's before the state, each
        // next one while the current one is computed), staged in LDS (gate
        // transform, norm partials, beta), then, after one barrier, the
        // tokens run back to back from LDS with the state in registers: a
        // token needs no barrier, its reductions stay inside DPP rows.  After
        // each token the output, the verify-cache rows and the checkpoint are
        // written; the pool slot once at the end (unless the pool is read
        // only).
        float st[G][8];
#pragma unroll
        for (int gi = 0; gi < G; ++gi) IO::unpack(raw[gi], st[gi]);
        if constexpr (!BF16) {
            // The state has to arrive before the first token anyway; an
            // empty asm reading every state register makes the wait for it
            // sit here, once.  Left to the compiler (fp32 unpacking is a
            // plain copy), the first use falls inside the token loop, which
            // has stores and no loads, and the compiler then drains every
            // outstanding load before each chunk's tokens, the prefetched
            // next chunk included (batched T=8 updates 71.9 against 73.6
            // us, read-only T=32 210.7 against 217.0).  bf16 unpacking reads
            // the registers here already.
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
#pragma unroll
                for (int e = 0; e < 8; ++e) asm volatile("" ::"v"(st[gi][e]));
        }
        const int64_t crow0 = ((int64_t)idx * p.HV + hv) * p.t_max;  // verify-cache row of token t0
        for (int c0 = t0; c0 < t1; c0 += CHUNK) {
            const int nc = min(CHUNK, t1 - c0);
            if (c0 != t0) __syncthreads();  // the previous chunk's stage has been read
#pragma unroll
            for (int i = 0; i < CHUNK; ++i) {
                if (i < nc) {
                    write_stage(tid, cin[i], a_h, dt, g_f32, precomputed, s_q[i], s_k[i], s_d[i], s_v[i],
                                s_norm[i]);
                    if (tid == 0) s_beta[i] = beta_of(blo[i], bhi[i]);
                    const int pos = c0 - t0 + i;
                    if (pos < p.t_max && p.kg && vs == 0 && tid < KD)
                        store_kg(p.kg, p.kg_f32 != 0, crow0 + pos, tid, cin[i], g_f32);
                }
            }
            __syncthreads();
            load_chunk(c0 + CHUNK);  // the next chunk (past the end: the last token again, unused)
            for (int i = 0; i < nc; ++i) {
                const int t = c0 + i;
                const int pos = t - t0;
                TokenOps ops;
                read_token_ops<BF16>(ops, s_q[i], s_k[i], s_d[i], s_norm[i], m, p.scale, p.l2_eps, s_beta[i]);
                float o[G], c[G];
#pragma unroll
                for (int gi = 0; gi < G; ++gi) o[gi] = row_update(st[gi], ops, s_v[i][r_base + gi], c[gi]);
                if (m == 0) store_out_bf16<G>(p.out + ((int64_t)t * p.HV + hv) * KD + r_base, o);
                if (pos < p.t_max && p.corr && m == 0) store_f32<G>(p.corr + (crow0 + pos) * KD + r_base, c);
                if (p.ckpt) {
                    char *ck = reinterpret_cast<char *>(p.ckpt) + ((int64_t)t * p.HV + hv) * (KD * KD) * es;
#pragma unroll
                    for (int gi = 0; gi < G; ++gi) IO::store_ckpt(ck, off[gi], IO::pack(st[gi]));
                }
            }
        }
        if (update) {
#pragma unroll
            for (int gi = 0; gi < G; ++gi) IO::store(head, off[gi], IO::pack(st[gi]));
        }
    }
}

// ---------------------------------------------------------- fused kernel ----
//
// One workgroup per (row, head) with the full V=128 (the gated RMSNorm needs
// all 128 outputs of the head).  Threads 0..383 (two passes of 256) own one
// of the head's 384 q|k|v channels for the conv: each reads its 3 cached
// positions and x, writes the SiLU activation to LDS and shifts its own cache
// column, so no other thread touches that channel.

// One conv channel's inputs: the three cached positions (oldest first), the
// current x and the four taps.
struct ConvIn {
    uint32_t c0, c1, c2, x;  // bf16 bits
    float w0, w1, w2, w3;
};

__device__ __forceinline__ ConvIn load_conv(const uint16_t *cs, const uint16_t *xr, const float *weight,
                                            int cl, int h, int HC, int C3)
{
    const int grp = cl >> 7;
    const int d = cl & (KD - 1);
    const int c = grp * HC + h * KD + d;
    ConvIn in;
    in.c0 = cs[c];
    in.c1 = cs[C3 + c];
    in.c2 = cs[2 * C3 + c];
    in.x = xr[c];
    const float *w = weight + (int64_t)grp * 4 * HC + h * KD + d;
    in.w0 = w[0];
    in.w1 = w[HC];
    in.w2 = w[2 * HC];
    in.w3 = w[3 * HC];
    return in;
}

// y = sum_j w_j hist_j over [c0, c1, c2, x], then SiLU; the channel's cache
// column is shifted to [c1, c2, x] by the same thread that read it.
__device__ __forceinline__ float conv_silu_shift(const ConvIn &in, uint16_t *cs, int cl, int h, int HC, int C3)
{
    const int c = (cl >> 7) * HC + h * KD + (cl & (KD - 1));
    float y = in.w0 * bf16_bits_to_f32(in.c0);
    y = fmaf(in.w1, bf16_bits_to_f32(in.c1), y);
    y = fmaf(in.w2, bf16_bits_to_f32(in.c2), y);
    y = fmaf(in.w3, bf16_bits_to_f32(in.x), y);
    cs[c] = (uint16_t)in.c1;
    cs[C3 + c] = (uint16_t)in.c2;
    cs[2 * C3 + c] = (uint16_t)in.x;
    return y * sigmoid_f(y);
}

template <bool BF16>
__global__ void __launch_bounds__(256) kda_fused_kernel(const FusedParams p)
{
    using IO = StateIO<BF16>;
    constexpr int G = 8;

    __shared__ float s_act[3 * KD];  // q | k | v activations of this head
    __shared__ float s_d[KD];
    __shared__ float s_red[16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int m = lane & 15;
    const int qd = lane >> 4;
    const int row = blockIdx.x / p.H;
    const int h = blockIdx.x - row * p.H;
    const int r_base = wave * (4 * G) + qd * G;
    uint16_t *out = p.out + ((int64_t)row * p.H + h) * KD;

    const int idx = p.state_indices[row];
    if (idx <= 0 || (int64_t)idx >= p.num_slots) {
        if (m == 0) store_zero_bf16<G>(out + r_base);
        return;
    }

    // Channel inputs first (conv history, x, taps, gate), then the state.
    const int HC = p.H * KD;
    const int C3 = 3 * HC;
    uint16_t *cs = p.conv_state + (int64_t)idx * p.conv_slot_stride;
    const uint16_t *xr = p.x + (int64_t)row * p.x_stride;
    const int c_lo = tid & (KD - 1);
    const ConvIn in0 = load_conv(cs, xr, p.weight, tid, h, HC, C3);
    const ConvIn in1 = load_conv(cs, xr, p.weight, 256 + c_lo, h, HC, C3);  // used by tid < 128
    const uint32_t graw = p.graw[(int64_t)row * p.g_stride + h * KD + c_lo];
    const float dt = p.dt_bias[(int64_t)h * KD + c_lo];
    const uint32_t braw = p.braw[(int64_t)row * p.beta_stride + h];
    const float a_h = __expf(p.A_log[h]);
    __builtin_amdgcn_sched_barrier(0);

    const size_t es = BF16 ? 2 : 4;
    char *head = reinterpret_cast<char *>(p.state) + ((int64_t)idx * p.slot_stride + (int64_t)h * (KD * KD)) * es;
    typename IO::Raw raw[G];
    uint32_t off[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        off[gi] = IO::off(r_base + gi, m);
        raw[gi] = IO::load(head, off[gi]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // depthwise causal conv (width 4) + SiLU and the gate, overlapping the state fetch
    s_act[tid] = conv_silu_shift(in0, cs, tid, h, HC, C3);
    if (tid < KD) {
        s_act[tid + 256] = conv_silu_shift(in1, cs, tid + 256, h, HC, C3);
        s_d[tid] = __expf(-a_h * softplus_f(bf16_bits_to_f32(graw) + dt));
    }
    const float beta = sigmoid_f(bf16_bits_to_f32(braw));
    __syncthreads();

    TokenOps ops;
    read_token_ops<BF16>(ops, s_act, s_act + KD, s_d, nullptr, m, p.scale, p.l2_eps, beta);
    float o[G];
    float ss = 0.f;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        float st[8];
        IO::unpack(raw[gi], st);
        o[gi] = row_update(st, ops, s_act[2 * KD + r_base + gi]);
        IO::store(head, off[gi], IO::pack(st));
        ss = fmaf(o[gi], o[gi], ss);
    }
    // gated RMSNorm over the 128 outputs of the head
    if (m == 0) s_red[wave * 4 + qd] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) tot += s_red[i];
    const float inv = rsqrtf(tot * (1.0f / KD) + p.norm_eps);
    if (m == 0) {
        const uint16_t *gate = p.ogate + (int64_t)row * p.ogate_stride + h * KD + r_base;
        float y[G];
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
            y[gi] = o[gi] * inv * p.norm_weight[r_base + gi] * sigmoid_f(bf16_bits_to_f32(gate[gi]));
        store_out_bf16<G>(out + r_base, y);
    }
}

// ------------------------------------------------- packed fused kernel ----
//
// The fused step over packed ragged rows with T >= 1 tokens per sequence.
// One workgroup per (sequence, head) with the full V=128, or, when there are
// few heads, VS workgroups per head that share it by value rows (see the
// kernel).  The sequence starts from the checkpoint slot of its last
// accepted token; the head's state (G value rows per DPP row) and the conv
// windows of its channels (three positions per channel, in the registers of
// the thread that owns the channel) are loaded once and carried across the
// tokens in fp32.
//
// Tokens go in chunks of up to PF_CHUNK: the chunk's inputs are loaded at once
// (one memory round trip); each thread runs its channels' conv over the
// chunk's tokens in order and stages the activations, decays and per-token
// scalars in LDS (a token whose checkpoint column names a live slot stores
// the conv window right there); after one barrier the tokens run back to
// back, each writing its unnormalised output and its RMS partial sums to LDS
// (split heads: its outputs to the caller's scratch) and storing its state
// checkpoint (rounded to bf16 for a bf16 pool); after a second barrier the
// gated RMSNorm of every token of the chunk is applied and stored, one
// (token, value) per thread (split heads: by the last part, at the end).
// Two barriers per chunk: every
// read of a chunk's stage precedes the second barrier and the next chunk's
// stage is written after it; every read of the outputs precedes the next
// chunk's first barrier, after which they are written again.

// One channel of the conv: window (oldest first, bf16 bits) and taps.
struct ConvChan {
    uint32_t c0, c1, c2;
    float w0, w1, w2, w3;
};

__device__ __forceinline__ int conv_channel(int cl, int h, int HC)
{
    return (cl >> 7) * HC + h * KD + (cl & (KD - 1));
}

__device__ __forceinline__ void load_taps(ConvChan &ch, const float *weight, int cl, int h, int HC)
{
    const float *w = weight + (int64_t)(cl >> 7) * 4 * HC + h * KD + (cl & (KD - 1));
    ch.w0 = w[0];
    ch.w1 = w[HC];
    ch.w2 = w[2 * HC];
    ch.w3 = w[3 * HC];
}

// The cached window of channel c (global index) in one slot's cache.
__device__ __forceinline__ void load_window(ConvChan &ch, const uint16_t *cs, int c, int C3)
{
    ch.c0 = cs[c];
    ch.c1 = cs[C3 + c];
    ch.c2 = cs[2 * C3 + c];
}

// Conv + SiLU of one token; the window advances by x.
__device__ __forceinline__ float conv_step(ConvChan &ch, uint32_t x)
{
    float y = ch.w0 * bf16_bits_to_f32(ch.c0);
    y = fmaf(ch.w1, bf16_bits_to_f32(ch.c1), y);
    y = fmaf(ch.w2, bf16_bits_to_f32(ch.c2), y);
    y = fmaf(ch.w3, bf16_bits_to_f32(x), y);
    ch.c0 = ch.c1;
    ch.c1 = ch.c2;
    ch.c2 = x;
    return y * sigmoid_f(y);
}

__device__ __forceinline__ void store_window(uint16_t *cs, const ConvChan &ch, int c, int C3)
{
    cs[c] = (uint16_t)ch.c0;
    cs[C3 + c] = (uint16_t)ch.c1;
    cs[2 * C3 + c] = (uint16_t)ch.c2;
}

// Device-coherent (relaxed, device-scope atomic) accesses: written through
// to, and read from, the level of the memory system shared by all chiplets,
// so a store that has completed is seen by a later such load from any CU.
__device__ __forceinline__ void store_coherent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_coherent(const float *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum over the 64 lanes of a wave; wave-uniform result.
__device__ __forceinline__ float wave_sum(float x)
{
    x = row_sum16(x);
    return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}

// A (sequence, head) is covered by VS workgroups, each owning RW = 128/VS
// value rows, G value rows per DPP row: 2048/(G*VS) threads.  VS=1: G=8
// (256 threads) for large grids, G=4 (512 threads) halves each lane's
// per-token work for smaller ones.  VS>1 spreads one head's per-token work
// over VS compute units when there are too few heads to fill the chip: each
// part runs the conv of all q and k channels (every part needs the full
// normalised q and k) and of its own v channels, updates its rows of the
// state and writes its unnormalised outputs to `partials`; the last part of
// the head to arrive (a per-head counter) applies the gated RMSNorm to the
// whole head and sets the counter back to zero.  No part waits for another.
template <bool BF16, int G, int VS>
__global__ void __launch_bounds__(2048 / (G * VS)) kda_packed_fused_kernel(const PackedFusedParams p)
{
    using IO = StateIO<BF16>;
    constexpr int RW = KD / VS;                  // value rows of this workgroup
    constexpr int NT = 2048 / (G * VS);          // threads
    constexpr int NCL = 2 * KD + RW;             // conv channels: q, k and this part's v
    constexpr int NCH = (NCL + NT - 1) / NT;     // conv channels per thread
    constexpr int NR = NT / 16;                  // DPP rows (RMS partials per token)
    constexpr int TP = NT / KD;                  // tokens per pass of the output phase
    constexpr int NOP = (PF_CHUNK + TP - 1) / TP;  // output passes per chunk
    constexpr bool SPLIT = VS > 1;
    static_assert(RW % (4 * G) == 0 && NT % KD == 0 && NT <= 1024, "bad packed fused geometry");

    __shared__ float s_act[PF_CHUNK][NCL];    // q | k | v activations per token
    __shared__ float s_d[PF_CHUNK][KD];
    __shared__ float s_o[SPLIT ? 1 : PF_CHUNK][KD];    // unnormalised outputs
    __shared__ float s_red[SPLIT ? 1 : PF_CHUNK][NR];  // RMS partial sums
    __shared__ float s_beta[PF_CHUNK];
    __shared__ int s_dst[PF_CHUNK];            // checkpoint slot, or -1
    __shared__ float s_nw[KD];
    __shared__ float s_fin[SPLIT ? NOP : 1][NT / 64];  // split heads: per-wave sums of squares
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int m = lane & 15;
    const int qd = lane >> 4;
    const int item = blockIdx.x / VS;
    const int part = blockIdx.x - item * VS;
    const int seq = item / p.H;
    const int h = item - seq * p.H;
    const int r_loc = wave * (4 * G) + qd * G;  // this lane's first value row in the part
    const int r_base = part * RW + r_loc;       // ... and in the head
    const int HC = p.H * KD;
    const int C3 = 3 * HC;
    auto out_at = [&](int r) { return p.out + ((int64_t)r * p.H + h) * KD + r_base; };

    // The row range, the accepted count and the first PF_CHUNK columns of
    // the row are fetched together and the start column is picked from
    // registers (a dependent load only for a start column past them): one
    // round trip before the state's, not three.  The column index is clamped
    // into the row; its validity is checked below.
    const int q0 = p.qsl[seq];
    const int q1 = p.qsl[seq + 1];
    const int acc = p.accepted[seq];
    const int32_t *cols = p.state_indices + (int64_t)seq * p.indices_stride;
    int head_cols[PF_CHUNK];
#pragma unroll
    for (int j = 0; j < PF_CHUNK; ++j) head_cols[j] = cols[min(j, p.max_tokens - 1)];
    // (the empty asm keeps the compiler from turning the pick below back into
    // one load whose address waits for the accepted count)
#pragma unroll
    for (int j = 0; j < PF_CHUNK; ++j) asm volatile("" : "+s"(head_cols[j]));
    const int a1 = min(max(acc, 1), p.max_tokens) - 1;
    int col_start = head_cols[0];
#pragma unroll
    for (int j = 1; j < PF_CHUNK; ++j)
        if (a1 == j) col_start = head_cols[j];
    if (a1 >= PF_CHUNK) col_start = cols[a1];
    const int t0 = min(max(q0, 0), p.n_rows);
    const int t1 = min(max(q1, t0), p.n_rows);
    // Rows that belong to no sequence: before the first one, after the last.
    if (m == 0) {
        if (seq == 0)
            for (int r = 0; r < t0; ++r) store_zero_bf16<G>(out_at(r));
        if (seq == p.n_seqs - 1)
            for (int r = t1; r < p.n_rows; ++r) store_zero_bf16<G>(out_at(r));
    }
    if (t1 <= t0) return;  // an empty sequence touches nothing

    // What does not depend on the start slot is issued before it is known:
    // the conv taps of this thread's channels (local channel cl = tid + k*NT:
    // q and k channels first, then this part's v channels; a thread past the
    // last one repeats it and never stores), the gate parameters and the norm
    // weight.  Then the slot, the conv windows and the state; the token
    // inputs per chunk.
    //
    // Conv checkpoints of split heads: a part's v channels and state rows are
    // its own, but every part reads the q and k windows of the start slot.
    // They are checkpointed by the part whose share of those 256 channels
    // they fall in, except into the start slot itself (the token in the
    // start column): there they wait in registers for the last part to
    // arrive, when every part has read the slot.
    const int c_lo = tid & (KD - 1);
    ConvChan ch[NCH];
    int gch[NCH];
    bool own[NCH], keep[NCH], is_v[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int cl = tid + k * NT;
        own[k] = cl < NCL;
        const int clc = own[k] ? cl : NCL - 1;
        const int hc = clc < 2 * KD ? clc : clc + part * RW;  // channel in the head's 384
        is_v[k] = own[k] && clc >= 2 * KD;
        keep[k] = own[k] && (clc >= 2 * KD || (clc * VS) / (2 * KD) == part);
        gch[k] = conv_channel(hc, h, HC);
        load_taps(ch[k], p.weight, hc, h, HC);
    }
    uint32_t held[SPLIT ? NCH : 1][3];  // split heads: q/k windows bound for the start slot
    bool hold = false;
    const float dt = p.dt_bias[(int64_t)h * KD + c_lo];
    const float a_h = __expf(p.A_log[h]);
    if (tid < KD) s_nw[tid] = p.norm_weight[tid];

    const int src = (acc >= 1 && acc <= p.max_tokens) ? col_start : -1;
    if (src <= 0 || (int64_t)src >= p.num_slots) {
        if (m == 0)
            for (int r = t0; r < t1; ++r) store_zero_bf16<G>(out_at(r));
        return;
    }
    const uint16_t *cs_src = p.conv_state + (int64_t)src * p.conv_slot_stride;
#pragma unroll
    for (int k = 0; k < NCH; ++k) load_window(ch[k], cs_src, gch[k], C3);
    __builtin_amdgcn_sched_barrier(0);

    const size_t es = BF16 ? 2 : 4;
    const int64_t head_elems = (int64_t)h * (KD * KD);
    const char *head = reinterpret_cast<const char *>(p.state) + ((int64_t)src * p.slot_stride + head_elems) * es;
    typename IO::Raw raw[G];
    uint32_t off[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        off[gi] = IO::off(r_base + gi, m);
        raw[gi] = IO::load(head, off[gi]);
    }
    float st[G][8];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) IO::unpack(raw[gi], st[gi]);

    const int ov = tid & (KD - 1);   // output phase: this thread's value index
    const int otk = tid >> 7;        // ... and its first token of the pass
    for (int c0 = t0; c0 < t1; c0 += PF_CHUNK) {
        const int nc = min(PF_CHUNK, t1 - c0);
        // the chunk's inputs, all at once (rows clamped into [t0, t1); unused past nc)
        uint32_t xin[PF_CHUNK][NCH], gr[PF_CHUNK], br[PF_CHUNK], og[SPLIT ? 1 : NOP];
        int col[PF_CHUNK];
#pragma unroll
        for (int i = 0; i < PF_CHUNK; ++i) {
            const int64_t n = c0 + min(i, nc - 1);
            const uint16_t *xn = p.x + n * p.x_stride;
#pragma unroll
            for (int k = 0; k < NCH; ++k) xin[i][k] = xn[gch[k]];
            gr[i] = p.graw[n * p.g_stride + h * KD + c_lo];
            br[i] = p.braw[n * p.beta_stride + h];
            col[i] = cols[min(c0 - t0 + i, p.max_tokens - 1)];
        }
        if constexpr (!SPLIT) {
#pragma unroll
            for (int k = 0; k < NOP; ++k)
                og[k] = p.ogate[(int64_t)(c0 + min(k * TP + otk, nc - 1)) * p.ogate_stride + h * KD + ov];
        }

        // stage: conv in token order, decays, scalars; conv checkpoints
#pragma unroll
        for (int i = 0; i < PF_CHUNK; ++i) {
            if (i < nc) {
                const int j = c0 - t0 + i;
                const int dst = (j < p.max_tokens && col[i] > 0 && (int64_t)col[i] < p.num_slots) ? col[i] : -1;
#pragma unroll
                for (int k = 0; k < NCH; ++k) {
                    const float a = conv_step(ch[k], xin[i][k]);
                    if (own[k]) s_act[i][tid + k * NT] = a;
                }
                if (tid < KD) s_d[i][tid] = __expf(-a_h * softplus_f(bf16_bits_to_f32(gr[i]) + dt));
                if (tid == 0) {
                    s_beta[i] = sigmoid_f(bf16_bits_to_f32(br[i]));
                    s_dst[i] = dst;
                }
                if (dst > 0) {
                    uint16_t *cs_dst = p.conv_state + (int64_t)dst * p.conv_slot_stride;
                    if (!SPLIT || dst != src) {
#pragma unroll
                        for (int k = 0; k < NCH; ++k)
                            if (keep[k]) store_window(cs_dst, ch[k], gch[k], C3);
                    } else {
                        hold = true;
#pragma unroll
                        for (int k = 0; k < (SPLIT ? NCH : 0); ++k) {
                            if (is_v[k]) store_window(cs_dst, ch[k], gch[k], C3);
                            held[k][0] = ch[k].c0;
                            held[k][1] = ch[k].c1;
                            held[k][2] = ch[k].c2;
                        }
                    }
                }
            }
        }
        __syncthreads();

        // the tokens, back to back
        for (int i = 0; i < nc; ++i) {
            TokenOps ops;
            read_token_ops<BF16>(ops, s_act[i], s_act[i] + KD, s_d[i], nullptr, m, p.scale, p.l2_eps,
                                 s_beta[i]);
            float o[G];
            float ss = 0.f;
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                o[gi] = row_update(st[gi], ops, s_act[i][2 * KD + r_loc + gi]);
                ss = fmaf(o[gi], o[gi], ss);
            }
            if (m == 0) {
                if constexpr (SPLIT) {
                    float *po = p.partials + ((int64_t)(c0 + i) * p.H + h) * KD + r_base;
#pragma unroll
                    for (int gi = 0; gi < G; ++gi) store_coherent(po + gi, o[gi]);
                } else {
                    s_red[i][wave * 4 + qd] = ss;
#pragma unroll
                    for (int gi = 0; gi < G; ++gi) s_o[i][r_base + gi] = o[gi];
                }
            }
            const int dst = s_dst[i];
            if (dst > 0) {
                char *ck = reinterpret_cast<char *>(p.state) + ((int64_t)dst * p.slot_stride + head_elems) * es;
#pragma unroll
                for (int gi = 0; gi < G; ++gi) IO::store(ck, off[gi], IO::pack(st[gi]));
            }
        }
        __syncthreads();

        if constexpr (!SPLIT) {
            // gated RMSNorm of the chunk: thread (otk, ov) handles tokens otk, otk+TP, ...
#pragma unroll
            for (int k = 0; k < NOP; ++k) {
                const int i = k * TP + otk;
                if (i < nc) {
                    float tot = 0.f;
#pragma unroll
                    for (int w = 0; w < NR; ++w) tot += s_red[i][w];
                    const float inv = rsqrtf(tot * (1.0f / KD) + p.norm_eps);
                    const float y = s_o[i][ov] * inv * s_nw[ov] * sigmoid_f(bf16_bits_to_f32(og[k]));
                    p.out[((int64_t)(c0 + i) * p.H + h) * KD + ov] = (uint16_t)(pack_bf16x2(y, 0.0f) & 0xffffu);
                }
            }
        }
    }

    if constexpr (SPLIT) {
        // Arrival: every wave waits until its device-coherent output stores
        // are complete, then one thread counts the part in; the part that
        // finds VS-1 earlier arrivals is the last, and its device-coherent
        // loads see every part's outputs.  (Device-scope fences would do the
        // same by writing back and invalidating the whole L2 of each wave's
        // chiplet, which costs microseconds while the checkpoint stores are
        // in flight.)
        wait_vm_all();
        __syncthreads();
        if (tid == 0) {
            const int prev = __hip_atomic_fetch_add(p.counters + item, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = prev == VS - 1;
        }
        __syncthreads();
        if (!s_last) return;
        if (tid == 0) __hip_atomic_store(p.counters + item, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (hold) {  // every q/k channel's window after the last token whose column is the start slot
            uint16_t *cs_start = p.conv_state + (int64_t)src * p.conv_slot_stride;
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                if (own[k] && !is_v[k]) {
                    cs_start[gch[k]] = (uint16_t)held[k][0];
                    cs_start[C3 + gch[k]] = (uint16_t)held[k][1];
                    cs_start[2 * C3 + gch[k]] = (uint16_t)held[k][2];
                }
            }
        }
        // Gated RMSNorm of the head, PF_CHUNK tokens at a time: thread
        // (otk, ov) takes tokens otk, otk+TP, ... of the chunk, all of whose
        // loads go out together; two waves per token.
        for (int c0 = t0; c0 < t1; c0 += PF_CHUNK) {
            const int nc = min(PF_CHUNK, t1 - c0);
            float o[NOP];
            uint32_t g[NOP];
#pragma unroll
            for (int k = 0; k < NOP; ++k) {
                const int64_t t = c0 + min(k * TP + otk, nc - 1);
                o[k] = load_coherent(p.partials + (t * p.H + h) * KD + ov);
                g[k] = p.ogate[t * p.ogate_stride + h * KD + ov];
            }
#pragma unroll
            for (int k = 0; k < NOP; ++k) {
                const float s = wave_sum(o[k] * o[k]);
                if (lane == 0) s_fin[k][wave] = s;
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < NOP; ++k) {
                if (k * TP + otk < nc) {
                    const float tot = s_fin[k][2 * otk] + s_fin[k][2 * otk + 1];
                    const float inv = rsqrtf(tot * (1.0f / KD) + p.norm_eps);
                    const float y = o[k] * inv * s_nw[ov] * sigmoid_f(bf16_bits_to_f32(g[k]));
                    p.out[((int64_t)(c0 + k * TP + otk) * p.H + h) * KD + ov] =
                        (uint16_t)(pack_bf16x2(y, 0.0f) & 0xffffu);
                }
            }
            __syncthreads();  // s_fin is rewritten by the next chunk
        }
    }
}

// ------------------------------------------------- WY verify kernel ----
//
// Read-only calls ("Frozen / speculative-verify mode": the pool is never
// written back) without checkpoints, with at most VERIFY_WY_MAX_T tokens per
// sequence: the batched form, or the ragged form when the caller declares the
// longest sequence.  Every token then reads the state through the slot's
// initial state S0 (K x V) and the recurrence unrolls.  With L_t the
// log-decay of tokens 0..t summed per key channel, E_t = exp(L_t),
// W_ts = exp(L_t - L_s) (s <= t), k^ and q^ the L2-normalised key and query
// and b_s = beta_s u_s:
//   u_t = v_t - k^_t.(E_t * S0) - sum_{s<t} (k^_t . W_ts k^_s) b_s
//   o_t = scale [ q^_t.(E_t * S0) + sum_{s<=t} (q^_t . W_ts k^_s) b_s ]
// (the pages' WY-parallel form: decay folded into k*exp(cumsum g) and
// q*exp(cumsum g) operands of a product with the state), which equals T
// sequential steps up to rounding.
//
// The products [k_t E_t ; q_t E_t] x S0 (2T x 128 by 128 x 128 per head) run
// on the matrix cores; the T^2 W-weighted channel sums are reduced once per
// head; each value row then runs a T-step forward substitution.  TM (2, 4,
// 8, 12 or 16, the smallest that holds the declared length) sizes the token
// registers and LDS.  Null rows give +0; in the ragged form, tokens past the
// declared length give +0 and record nothing.
constexpr int pow2_at_least(int x)
{
    int q = 2;
    while (q < x) q *= 2;
    return q;
}

// Channel sums of the WY verify kernel: layout A holds |q_t|^2 and
// q_t.W_ts k_s (s <= t), t + 2 sums for token t; layout B |k_t|^2 and
// k_t.W_ts k_s (s < t), t + 1 sums.  They are emitted in chunks of whole
// tokens, each reduced over the wave at once; chunk k holds tokens
// [first(k), first(k + 1)), and token t's sums start at off(t) in its chunk
// (norm first, then s = 0, 1, ...).  Chunks of 4 tokens; with SIX (fp32
// pools at 16 token slots) six chunks of at most 32 sums each instead: a
// chunk of 64 sums keeps 32 more registers live while it is formed, which
// there decides between two and three workgroups per compute unit (bf16
// pools fit three with the four chunks, which take fewer instructions).
template <int TM, bool SIX>
struct WyChunks {
    static_assert(!SIX || TM == 16, "six chunks: 16 token slots");
    static constexpr int NCH = SIX ? 6 : (TM > 4 ? (TM + 3) / 4 : 1);
    static constexpr int first(int k)
    {
        if (SIX) {
            constexpr int b[7] = {0, 6, 9, 11, 13, 15, 16};
            return b[k];
        }
        return TM > 4 ? (4 * k < TM ? 4 * k : TM) : k * TM;
    }
    static constexpr int chunk_of(int t)
    {
        int k = 0;
        while (first(k + 1) <= t) ++k;
        return k;
    }
    // offset of token t in its chunk, layout A or B
    static constexpr int off(int t, bool a)
    {
        int o = 0;
        for (int u = first(chunk_of(t)); u < t; ++u) o += u + (a ? 2 : 1);
        return o;
    }
    static constexpr int size(int k)  // layout A, the larger
    {
        int o = 0;
        for (int u = first(k); u < first(k + 1); ++u) o += u + 2;
        return o;
    }
    static constexpr int P(int k) { return pow2_at_least(size(k)); }
};

// One layout of the channel sums, one key channel per lane, reduced over the
// wave chunk by chunk: layout A (x = q) holds |q_t|^2 and q_t.W_ts k_s
// (s <= t), layout B (x = k) |k_t|^2 and k_t.W_ts k_s (s < t).  kw[s]
// carries k_s * W_ts across the chunks.
template <int TM, bool SIX, int K, bool A>
__device__ __forceinline__ float wy_chunk_layout(float *kw, const float *x, const float *kf, const float *d, int lane)
{
    using C = WyChunks<TM, SIX>;
    constexpr int P = C::P(K);
    float cur[P];
#pragma unroll
    for (int i = 0; i < P; ++i) cur[i] = 0.f;
#pragma unroll
    for (int t = C::first(K); t < C::first(K + 1); ++t) {
#pragma unroll
        for (int s = 0; s < t; ++s) kw[s] *= d[t];  // k_s * W_ts
        kw[t] = kf[t];
        const int o = C::off(t, A);
        cur[o] = x[t] * x[t];
#pragma unroll
        for (int s = 0; s < (A ? t + 1 : t); ++s) cur[o + 1 + s] = x[t] * kw[s];
    }
    return wave_transpose_sum<P>(cur, lane);
}

template <int TM, bool SIX, bool A>
__device__ __forceinline__ void wy_layout_sums(float *r, const float *x, const float *kf, const float *d, int lane)
{
    constexpr int NCH = WyChunks<TM, SIX>::NCH;
    float kw[TM];
    r[0] = wy_chunk_layout<TM, SIX, 0, A>(kw, x, kf, d, lane);
    if constexpr (NCH > 1) r[1] = wy_chunk_layout<TM, SIX, (NCH > 1 ? 1 : 0), A>(kw, x, kf, d, lane);
    if constexpr (NCH > 2) r[2] = wy_chunk_layout<TM, SIX, (NCH > 2 ? 2 : 0), A>(kw, x, kf, d, lane);
    if constexpr (NCH > 3) r[3] = wy_chunk_layout<TM, SIX, (NCH > 3 ? 3 : 0), A>(kw, x, kf, d, lane);
    if constexpr (NCH > 4) r[4] = wy_chunk_layout<TM, SIX, (NCH > 4 ? 4 : 0), A>(kw, x, kf, d, lane);
    if constexpr (NCH > 5) r[5] = wy_chunk_layout<TM, SIX, (NCH > 5 ? 5 : 0), A>(kw, x, kf, d, lane);
}

// Per-head metadata: the sequence's tokens, the pool slot, the heads.
struct WyItem {
    int seq, hv, hq, t0, len, n, idx, live;
};

__device__ __forceinline__ WyItem wy_item(const RecParams &p, int w)
{
    WyItem it;
    it.seq = w / p.HV;
    it.hv = w - it.seq * p.HV;
    it.hq = it.hv / p.group;
    it.idx = p.state_indices[it.seq];
    if (p.cu_seqlens) {
        it.t0 = min(max(p.cu_seqlens[it.seq], 0), p.n_tokens);
        it.len = max(min(p.cu_seqlens[it.seq + 1], p.n_tokens) - it.t0, 0);
    } else {
        it.t0 = it.seq * p.tps;
        it.len = p.tps;
    }
    it.n = min(it.len, p.tps);  // tokens evaluated (p.tps: the declared length, <= TM)
    it.live = it.idx >= 0 && (int64_t)it.idx < p.num_slots && it.n > 0;
    return it;
}

// Matrix-core operand layout of the WY verify kernel.  A product's K order
// (the key channels) is free as long as both operands take the same one; it
// is chosen so that each 16-byte piece a lane loads holds consecutive
// channels and the four lane groups g = lane >> 4 read 64 contiguous bytes
// of a state row per load:
//  * bf16 pools, v_mfma_f32_16x16x32_bf16: K block j (32 channels), element
//    e of group g is channel 32 j + 8 g + e;
//  * fp32 pools, v_mfma_f32_16x16x4_f32: K group j (16 channels, four
//    products), product e of group g takes channel 16 j + 4 g + e.
template <bool BF16>
struct WyLayout {
    static constexpr int NJ = BF16 ? 4 : 8;     // K blocks / groups per row
    static constexpr int CPJ = KD / NJ;         // channels per block / group
    static constexpr int SW = BF16 ? 4 : 4;     // state words per lane and block / group (16 bytes)
    __device__ static constexpr int channel(int j, int g) { return CPJ * j + (CPJ / 4) * g; }
};

// One workgroup (4 waves) per head; each wave owns 32 value rows of it, as
// two 16-row tiles.
//  1. The token inputs of the lane's key channel are loaded before the pool
//     slot is known, and the lane's value row.
//  2. The state is read as whole rows: in each load instruction a wave
//     reads 1 KB of consecutive rows (2 fp32 or 4 bf16 rows) and the four
//     waves side by side 4 KB, so the head streams in order; measured on
//     MI355X, loads in the matrix-core layout (16 rows x 64 bytes per
//     instruction) stream 20-25% slower.  A wave's 32 rows are those of its
//     own load instructions.  The first tile's loads go out first;
//     meanwhile the key channels, one per lane (waves 0-1 layout A with q,
//     waves 2-3 layout B with k): cumulative decays, the token operand
//     column of the channel (q_t E_t, or k_t E_t; zero past the tokens)
//     into LDS once for the head (bf16 pools: as a bf16 head and
//     remainder), and the W-weighted channel sums, each reduced over the
//     wave in registers.  Then the second tile's loads, and one barrier.
//  3. [k_t E_t ; q_t E_t] x S0 on the matrix cores: each tile reaches the
//     matrix-core layout through the wave's LDS buffer in passes of 16
//     columns of 16 bytes (bf16 pools: the exact state by the operand's
//     head and remainder, two bf16 products; fp32 pools: fp32 products,
//     4x4x1 when at most 8 operand columns exist; from 12 token slots bf16
//     heads and remainders of both, three bf16 products), the products
//     through LDS into a row-per-lane layout, then the forward substitution
//     (lanes l and l + 32 own row l & 31; in each pair of tokens both
//     compute the two corrections, the lower half of the wave stores the
//     even token's output and correction, the upper half the odd one's).
// Three to eight workgroups share a compute unit (the VGPRs and the LDS
// decide), so the loads of one overlap the arithmetic of the others.  Consecutive heads
// (which share their sequence's token rows) run on one XCD.  KGC: the call
// records the raw key and gate cache (a kernel of its own, so that calls
// without it carry none of its stores).
template <bool BF16, int TM, bool KGC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TM <= 4 ? (BF16 ? 5 : 4) : (TM <= 8 ? 4 : 3))))
kda_verify_wy_kernel(const RecParams p)
{
    using LY = WyLayout<BF16>;
    constexpr int WROWS = 32;                    // value rows per wave
    constexpr uint32_t ROW_BYTES = KD * (BF16 ? 2 : 4);
    constexpr int NCT = (2 * TM + 15) / 16;      // 16-column tiles of the token operand
    constexpr int NCOL = 2 * TM;                 // columns: k_t E_t at t, q_t E_t at TM + t
    constexpr int OST = NCOL + 4;                // floats per row of the products in LDS
    using CH = WyChunks<TM, !BF16 && TM == 16>;
    constexpr int NCH = CH::NCH;                 // chunks of channel sums
    constexpr int SW = LY::SW;
    constexpr int NCF = 2 * TM * TM + 3 * TM;    // per-wave coefficients
    // fp32 pools: 4x4x1 fp32 products when at most 8 operand columns exist
    // (MF4); 16x16x4 fp32 products at 16 columns; at 32 columns bf16
    // products on a bf16 head and remainder of the state and of the operand
    // (SPL, three products per K block: a fifth of the matrix-core time for
    // some vector work, measured faster only there)
    constexpr bool MF4 = !BF16 && 2 * TM <= 8;
    constexpr bool SPL = !BF16 && 2 * TM > 16;
    constexpr bool OPB = BF16 || SPL;            // operand stored as bf16 head and remainder
    constexpr int BST = OPB ? KD / 2 + 4 : KD + 4;  // words per operand row (bf16: pairs), padded
    static_assert(TM <= VERIFY_WY_MAX_T, "verify tokens");

    constexpr int LPR = ROW_BYTES / 16;          // lanes per state row in a load instruction
    constexpr int RPI = 64 / LPR;                // rows per load instruction of a wave
    constexpr int NLD = 16 / RPI;                // load instructions per 16-row tile
    constexpr int NPASS = LPR / 16;              // passes of 16 columns (16 bytes each) per tile
    constexpr int PASSW = MF4 ? 2048 : 1024;     // a pass of half a tile, or a whole tile (4x4x1)
    constexpr int BUFW = WROWS * OST > PASSW ? WROWS * OST : PASSW;  // the passes, then the products
    __shared__ __align__(16) uint32_t s_T[4][BUFW];          // per wave
    __shared__ __align__(16) uint32_t s_B[OPB ? 2 : 1][NCOL][BST];  // token operand (or its bf16 head, remainder)
    __shared__ float s_sum[2][2][64 * NCH];                   // channel sums: layout, half of the channels
    __shared__ float s_beta[TM];
    __shared__ float s_cf[4][NCF];                            // per wave: C_ts, A'_ts, rk_t, scale*rq_t, beta_t

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4;
    const int n16 = lane & 15;
    const int rloc = lane & 31;
    // Value row of row rho (0..15) of the wave's tile tau: the tile holds the
    // rows of its load instructions NLD tau .. NLD tau + NLD - 1, in each of
    // which the four waves read 4 RPI consecutive rows side by side.
    auto vrow_of = [&](int tau, int rho) { return 4 * RPI * (NLD * tau + rho / RPI) + RPI * wave + rho % RPI; };
    const int vrow = vrow_of(rloc >> 4, rloc & 15);
    const int work = (int)(blockIdx.x & 7u) * (int)(gridDim.x >> 3) + (int)(blockIdx.x >> 3);
    if (work >= p.n_work) return;
    const WyItem it = wy_item(p, work);
    // Token row t of the sequence, clamped to its last evaluated token; a
    // sequence without tokens reads row 0, which exists (a call without any
    // token launches nothing), and uses none of it.  Each input is addressed
    // as a wave-uniform base at the sequence's first row plus a 32-bit
    // per-lane offset (the host takes this kernel only when every input's
    // last token row lies within 2^31 bytes of the first), which keeps the
    // per-token address arithmetic to one multiply and one add.
    const int64_t row0 = it.n > 0 ? (int64_t)it.t0 : 0;
    const int last = it.n > 0 ? it.n - 1 : 0;
    auto rel = [&](int t) { return (uint32_t)min(t, last); };  // row t relative to row0

    // 1. the token inputs of key channel c, and the value row
    const bool A = wave < 2;
    const int c = 64 * (wave & 1) + lane;
    const bool g_f32 = p.g_f32 != 0;
    const bool beta_f32 = p.beta_f32 != 0;
    uint32_t xb[TM], kb[TM], glo[TM], ghi[TM], vb[TM];
    // the value rows' inputs, used only by the forward substitution: from 12
    // token slots on loaded after the channel phase (with the second tile),
    // so that they hold no registers through it
    constexpr bool V_LATE = TM >= 12;
    auto load_v = [&]() {
#pragma unroll
        for (int t = 0; t < TM; ++t)
            vb[t] = *reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(p.v) + row0 * p.v_stride * 2 +
                                                        ((uint32_t)(it.hv * KD + vrow) * 2 + rel(t) * ((uint32_t)p.v_stride * 2)));
    };
    uint32_t beta_lo = 0, beta_hi = 0;
    const bool precomputed = p.precomputed != 0;
    float dtc_raw;
    {
        // (layout B reads k twice rather than copy it: a copy would wait for the load)
        const int ges = g_f32 ? 4 : 2, bes = beta_f32 ? 4 : 2;
        const char *kq = reinterpret_cast<const char *>(p.k) + row0 * p.k_stride * 2;
        const char *xq = reinterpret_cast<const char *>(A ? p.q : p.k) + row0 * (A ? p.q_stride : p.k_stride) * 2;
        const char *gq = static_cast<const char *>(p.g) + row0 * p.g_stride * ges;
        const uint32_t kst = (uint32_t)p.k_stride * 2, xst = (uint32_t)(A ? p.q_stride : p.k_stride) * 2;
        const uint32_t gst = (uint32_t)p.g_stride * (uint32_t)ges;
        const uint32_t kl = (uint32_t)(it.hq * KD + c) * 2, gl = (uint32_t)(it.hv * KD + c) * (uint32_t)ges;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const uint32_t r = rel(t);
            kb[t] = *reinterpret_cast<const uint16_t *>(kq + (kl + r * kst));
            xb[t] = *reinterpret_cast<const uint16_t *>(xq + (kl + r * xst));
            load_halves(gq + (gl + r * gst), g_f32, glo[t], ghi[t]);
        }
        // (every lane loads a beta, lanes t < TM of wave 2 keep token t's:
        // a load under a lane condition would wait for its value at the join)
        load_halves(static_cast<const char *>(p.beta) + row0 * p.beta_stride * bes +
                        (rel(min(lane, TM - 1)) * (uint32_t)p.beta_stride + (uint32_t)it.hv) * (uint32_t)bes,
                    beta_f32, beta_lo, beta_hi);
        // the channel's dt_bias, loaded on every path (a precomputed gate has
        // none: q's first word instead, unused) -- a load under the gate-mode
        // branch made the decays wait for every load issued before them,
        // the state's included
        dtc_raw = precomputed ? *reinterpret_cast<const float *>(p.q) : p.dt_bias[(int64_t)it.hv * KD + c];
        if constexpr (!V_LATE) load_v();
    }
    // (the token inputs stay ahead of the state's loads in the memory counter)
    __builtin_amdgcn_sched_barrier(0);
    if (!it.live) {  // a null head: +0 for each of its tokens
        for (int i = tid; i < it.len * KD; i += 256)
            p.out[((int64_t)(it.t0 + i / KD) * p.HV + it.hv) * KD + (i & (KD - 1))] = 0;
        return;
    }

    // 2. the state, as whole rows: the first tile (the second follows the channel phase)
    uint32_t *buf = s_T[wave];
    const char *hstate = static_cast<const char *>(p.state) +
                         ((int64_t)it.idx * p.slot_stride + (int64_t)it.hv * (KD * KD)) * (BF16 ? 2 : 4);
    const uint32_t lcol = 16u * (uint32_t)(lane % LPR);  // the lane's 16 bytes of a row
    auto load_tile = [&](int tau, u32x4 (&raw)[NLD]) {
#pragma unroll
        for (int i = 0; i < NLD; ++i)
            raw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                hstate + (uint32_t)vrow_of(tau, RPI * i + lane / LPR) * ROW_BYTES + lcol));
    };
    u32x4 raw0[NLD];
    load_tile(0, raw0);

    // verify cache of the raw key and gate (lanes of layout A, their channel).
    // With at most 4 token slots these stores go after the outputs: issued
    // earlier, they sit between the state loads and the waits for them (the
    // in-order memory counter), which cost ~1 us at B=64 H=32; with more
    // slots the registers they keep live cost more than that.
    constexpr bool KG_LATE = TM <= 4;
    auto store_kg_rows = [&]() {
        if (KGC && A) {
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                if (t < it.n && t < p.t_max) {
                    StageIn si{};
                    si.k = kb[t];
                    si.g_lo = glo[t];
                    si.g_hi = ghi[t];
                    store_kg(p.kg, p.kg_f32 != 0, ((int64_t)it.idx * p.HV + it.hv) * p.t_max + t, c, si, g_f32);
                }
            }
        }
    };

    // the key channel: decays, the operand column, the channel sums
    {
        if constexpr (!KG_LATE) store_kg_rows();
        const float a_h = precomputed ? 0.f : __expf(p.A_log[it.hv]);
        const float dtc = precomputed ? 0.f : dtc_raw;
        float xf[TM], kf[TM], d[TM];
        float E = 1.f;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const float gv = halves_value(glo[t], ghi[t], g_f32);
            const float lg = precomputed ? gv : -a_h * softplus_f(gv + dtc);
            d[t] = __expf(lg);
            E *= d[t];
            xf[t] = bf16_bits_to_f32(xb[t]);
            kf[t] = bf16_bits_to_f32(kb[t]);
            // operand column: q_t E_t (layout A) or k_t E_t (layout B)
            const float ov = t < it.n ? xf[t] * E : 0.f;
            const int col = A ? TM + t : t;
            if constexpr (OPB) {
                const __bf16 hb = (__bf16)ov;
                const __bf16 lb = (__bf16)(ov - (float)hb);
                reinterpret_cast<__bf16 *>(s_B[0][col])[c] = hb;
                reinterpret_cast<__bf16 *>(s_B[1][col])[c] = lb;
            } else {
                reinterpret_cast<float *>(s_B[0][col])[c] = ov;
            }
        }
        float r[NCH];
        if (A) wy_layout_sums<TM, !BF16 && TM == 16, true>(r, xf, kf, d, lane);
        else wy_layout_sums<TM, !BF16 && TM == 16, false>(r, xf, kf, d, lane);
        // lanes holding one sum of chunk k
        constexpr int SP[6] = {64 / CH::P(0), 64 / CH::P(NCH > 1 ? 1 : 0), 64 / CH::P(NCH > 2 ? 2 : 0),
                               64 / CH::P(NCH > 3 ? 3 : 0), 64 / CH::P(NCH > 4 ? 4 : 0), 64 / CH::P(NCH > 5 ? 5 : 0)};
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int sp = SP[k];
            if ((lane & (sp - 1)) == 0) s_sum[A ? 0 : 1][wave & 1][64 * k + lane / sp] = r[k];
        }
        if (wave == 2 && lane < TM) {
            const float bv = halves_value(beta_lo, beta_hi, beta_f32);
            s_beta[lane] = precomputed ? bv : sigmoid_f(bv);
        }
    }
    u32x4 raw1[NLD];  // the second tile
    load_tile(1, raw1);
    if constexpr (V_LATE) load_v();
    __syncthreads();

    // coefficients (each wave its own copy): (t, s) = (e / TM, e % TM);
    // token t's first sum: its chunk, then the chunk's earlier tokens.  The
    // per-token scalars first (lanes t < TM), then the T^2 coefficients,
    // which read 1/|k_s| and 1/|k_t| from them instead of evaluating both
    // again for every coefficient.
    float *cf = s_cf[wave];
    {
        auto slot = [&](int t, bool a) {
            int k = 0, f = 0;  // t's chunk and the chunk's first token
#pragma unroll
            for (int kk = 1; kk < NCH; ++kk)
                if (t >= CH::first(kk)) k = kk, f = CH::first(kk);
            return 64 * k + (t - f) * (f + t + (a ? 3 : 1)) / 2;
        };
        auto sum = [&](int a, int i) { return s_sum[a][0][i] + s_sum[a][1][i]; };
        float *rk = cf + 2 * TM * TM;
        if (lane < TM && lane < it.n) {
            rk[lane] = rsqrtf(sum(1, slot(lane, false)) + p.l2_eps);
            rk[TM + lane] = rsqrtf(sum(0, slot(lane, true)) + p.l2_eps) * p.scale;
            rk[2 * TM + lane] = s_beta[lane];
        }
        wave_lds_sync();
#pragma unroll
        for (int e = lane; e < TM * TM; e += 64) {
            const int t = e / TM, s = e - (e / TM) * TM;
            if (t < it.n) {
                const float rks = rk[s];
                cf[e] = s < t ? rk[t] * rks * sum(1, slot(t, false) + 1 + s) : 0.f;
                cf[TM * TM + e] = s <= t ? rks * sum(0, slot(t, true) + 1 + s) : 0.f;
            }
        }
    }

    // 3. the products, tile by tile: column cc = 16 kc + (lane & 15) of the
    // operand at the lane's channels (zero past the 2 TM columns)
    f32x4 acc[2][NCT];
    // K group j of a tile; sa: the lane's 16 bytes of it (row lane & 15)
    auto kgroup = [&](int tau, int j, const u32x4 &sw) {
        const uint32_t sa[SW] = {sw.x, sw.y, sw.z, sw.w};
        {
            const int ch = LY::channel(j, grp);
#pragma unroll
            for (int kc = 0; kc < NCT; ++kc) {
                const int cc = 16 * kc + n16;
                const int ccr = cc < NCOL ? cc : NCOL - 1;
                if constexpr (BF16) {  // exact bf16 state: two products
                    u32x4 bh = *reinterpret_cast<const u32x4 *>(&s_B[0][ccr][ch / 2]);
                    u32x4 bl = *reinterpret_cast<const u32x4 *>(&s_B[1][ccr][ch / 2]);
                    if (cc >= NCOL) bh = bl = u32x4{0u, 0u, 0u, 0u};
                    const bf16x8 a = __builtin_bit_cast(bf16x8, sw);
                    acc[tau][kc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bh),
                                                                          acc[tau][kc], 0, 0, 0);
                    acc[tau][kc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bl),
                                                                          acc[tau][kc], 0, 0, 0);
                } else {  // fp32 state, fp32 products
                    f32x4 b = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(s_B[0][ccr]) + ch);
                    if (cc >= NCOL) b = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[tau][kc] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(sa[e]), b[e],
                                                                           acc[tau][kc], 0, 0, 0);
                }
            }
        }
    };
    // A tile reaches the matrix-core layout (row lane & 15, the 16 bytes
    // of K group j) through the wave's buffer, 16 columns of 16 bytes per
    // pass: column c of row rho at c ^ rho, so that the 16 rows read at one
    // column fall on distinct banks.
    auto tile_products = [&](int tau, const u32x4 (&raw)[NLD]) {
#pragma unroll
        for (int kc = 0; kc < NCT; ++kc) acc[tau][kc] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hh = 0; hh < NPASS; ++hh) {
            const int c = lane % LPR - 16 * hh;
            if (NPASS == 1 || (c >= 0 && c < 16)) {
#pragma unroll
                for (int i = 0; i < NLD; ++i) {
                    const int rho = RPI * i + lane / LPR;
                    *reinterpret_cast<u32x4 *>(buf + 4 * (16 * rho + (c ^ rho))) = raw[i];
                }
            }
            wave_lds_sync();
            if constexpr (SPL) {
                // K blocks 2 hh and 2 hh + 1 (32 channels each): the lane's 8
                // channels 32 jb + 8 g + 0..7 as a bf16 head and remainder
#pragma unroll
                for (int j2 = 0; j2 < 2; ++j2) {
                    const int jb = 2 * hh + j2, c0 = 8 * j2 + 2 * grp;
                    const f32x4 x0 = *reinterpret_cast<const f32x4 *>(buf + 4 * (16 * n16 + (c0 ^ n16)));
                    const f32x4 x1 = *reinterpret_cast<const f32x4 *>(buf + 4 * (16 * n16 + ((c0 + 1) ^ n16)));
                    // (a pair's heads packed once and unpacked by shifts:
                    // converting each value on its own and packing again
                    // took a third more instructions)
                    u32x4 hw, lw;
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const float xa = e2 < 2 ? x0[2 * e2] : x1[2 * e2 - 4];
                        const float xb = e2 < 2 ? x0[2 * e2 + 1] : x1[2 * e2 - 3];
                        const uint32_t h = pack_bf16x2(xa, xb);
                        hw[e2] = h;
                        lw[e2] = pack_bf16x2(xa - __uint_as_float(h << 16), xb - __uint_as_float(h & 0xffff0000u));
                    }
                    const bf16x8 ah = __builtin_bit_cast(bf16x8, hw), al = __builtin_bit_cast(bf16x8, lw);
#pragma unroll
                    for (int kc = 0; kc < NCT; ++kc) {
                        const int cc = 16 * kc + n16;
                        const int ccr = cc < NCOL ? cc : NCOL - 1;
                        u32x4 bh = *reinterpret_cast<const u32x4 *>(&s_B[0][ccr][16 * jb + 4 * grp]);
                        u32x4 bl = *reinterpret_cast<const u32x4 *>(&s_B[1][ccr][16 * jb + 4 * grp]);
                        if (cc >= NCOL) bh = bl = u32x4{0u, 0u, 0u, 0u};
                        const bf16x8 bhv = __builtin_bit_cast(bf16x8, bh), blv = __builtin_bit_cast(bf16x8, bl);
                        acc[tau][kc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bhv, acc[tau][kc], 0, 0, 0);
                        acc[tau][kc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, blv, acc[tau][kc], 0, 0, 0);
                        acc[tau][kc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bhv, acc[tau][kc], 0, 0, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);  // (the next block's reads not hoisted: registers)
                }
            } else {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int j = 4 * hh + jj;
                    kgroup(tau, j, *reinterpret_cast<const u32x4 *>(buf + 4 * (16 * n16 + ((4 * j + grp - 16 * hh) ^ n16))));
                }
            }
            wave_lds_sync();
        }
    };
    // fp32 pools with at most 4 token slots (4 or 8 operand columns) use the
    // 4x4x1 products instead, 16 blocks of 4 rows by 4 columns, so that no
    // operand column is padding: block 4 cp + rg (lanes 16 cp + 4 rg + 0..3)
    // takes rows 4 rg .. 4 rg + 3 of a tile over channel part cp (its 16-byte
    // columns 8 cp .. 8 cp + 7); a whole tile goes through the buffer at once,
    // so the first tile's registers are free before the second's products;
    // the four parts are then summed across the lanes.
    constexpr int NCS = MF4 ? NCOL / 4 : 1;      // 4x4x1: sets of 4 operand columns
    [[maybe_unused]] float mtot[2][NCS];         // 4x4x1: each lane's tile totals
    if constexpr (MF4) {
        const int cp = lane >> 4, rho = lane & 15;  // rho = 4 rg + (lane & 3)
        auto tile4 = [&](int tau, const u32x4 (&raw)[NLD]) {
            f32x4 d[NCS];
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs) d[cs] = f32x4{0.f, 0.f, 0.f, 0.f};
            // the whole tile: 16-byte column c of row r at c ^ r
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int rw = RPI * i + lane / LPR, c = lane % LPR;
                *reinterpret_cast<u32x4 *>(buf + 4 * (32 * rw + (c ^ rw))) = raw[i];
            }
            wave_lds_sync();
#pragma unroll
            for (int sq = 0; sq < 8; ++sq) {
                const int c32 = 8 * cp + sq;  // 16-byte column of the row
                f32x4 bv[NCS];
#pragma unroll
                for (int cs = 0; cs < NCS; ++cs)
                    bv[cs] = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(s_B[0][4 * cs + (lane & 3)]) +
                                                              4 * c32);
                const f32x4 a = *reinterpret_cast<const f32x4 *>(buf + 4 * (32 * rho + (c32 ^ rho)));
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int cs = 0; cs < NCS; ++cs)
                        d[cs] = __builtin_amdgcn_mfma_f32_4x4x1f32(a[e], bv[cs][e], d[cs], 0, 0, 0);
            }
            wave_lds_sync();
            // lane 16 cp + 4 rg + j holds rows 4 rg + r (r = 0..3) of column
            // 4 cs + j over part cp; halving at distances 32 and 16 leaves it
            // the total of row 4 rg + cp
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs)
                mtot[tau][cs] = swap16_sum(swap32_sum(d[cs][0], d[cs][2]), swap32_sum(d[cs][1], d[cs][3]));
        };
        tile4(0, raw0);
        tile4(1, raw1);
    } else {
        tile_products(0, raw0);
        tile_products(1, raw1);
    }

    // the products to LDS, this wave's rows: row 16 tau + 4 g + r, column
    // 16 kc + (lane & 15)
    float *prod = reinterpret_cast<float *>(buf);
    if constexpr (MF4) {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs)
                prod[(16 * tau + 4 * ((lane >> 2) & 3) + (lane >> 4)) * OST + 4 * cs + (lane & 3)] = mtot[tau][cs];
    } else {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int kc = 0; kc < NCT; ++kc)
                if (16 * kc + n16 < NCOL)
#pragma unroll
                    for (int r = 0; r < 4; ++r) prod[(16 * tau + 4 * grp + r) * OST + 16 * kc + n16] = acc[tau][kc][r];
    }
    wave_lds_sync();

    // forward substitution, row rloc of the wave
    const float *pr = prod + rloc * OST;
    float P[TM], Q[TM], bu[TM];
#pragma unroll
    for (int t2 = 0; t2 < TM; t2 += 2) {
        const float2 x = *reinterpret_cast<const float2 *>(pr + t2);
        const float2 y = *reinterpret_cast<const float2 *>(pr + TM + t2);
        P[t2] = x.x; P[t2 + 1] = x.y;
        Q[t2] = y.x; Q[t2 + 1] = y.y;
    }
    const int half = lane >> 5;
    // the value of the lane's half of a token pair, by a bit select on an
    // opaque mask (a plain select of two array elements became an indexed
    // pick over the whole array, through a private array in scratch)
    uint32_t hmask = 0u - (uint32_t)half;  // all ones in the upper half of the wave
    asm("" : "+v"(hmask));
    auto pick = [&](float a, float b) {
        return __uint_as_float(__float_as_uint(a) ^ ((__float_as_uint(a) ^ __float_as_uint(b)) & hmask));
    };
    const int64_t crow0 = ((int64_t)it.idx * p.HV + it.hv) * p.t_max;
    const float *Cm = cf, *Am = cf + TM * TM, *tk = cf + 2 * TM * TM;
#pragma unroll
    for (int j = 0; j < TM / 2; ++j) {
        if (2 * j < it.n) {
#pragma unroll
            for (int t = 2 * j; t < 2 * j + 2; ++t) {
                float x = tk[t] * P[t];
#pragma unroll
                for (int s = 0; s < t; ++s) x = fmaf(Cm[t * TM + s], bu[s], x);
                bu[t] = t < it.n ? tk[2 * TM + t] * (bf16_bits_to_f32(vb[t]) - x) : 0.f;
            }
            const int th = 2 * j + half;
            const float *ar = Am + th * TM;
            float y = pick(Q[2 * j], Q[2 * j + 1]);
#pragma unroll
            for (int s = 0; s <= 2 * j + 1; ++s) y = fmaf(ar[s], bu[s], y);
            y *= tk[TM + th];
            if (th < it.n) {
                p.out[((int64_t)(it.t0 + th) * p.HV + it.hv) * KD + vrow] = (uint16_t)(pack_bf16x2(y, 0.0f) & 0xffffu);
                if (p.corr && th < p.t_max) p.corr[(crow0 + th) * KD + vrow] = pick(bu[2 * j], bu[2 * j + 1]);
            }
        }
    }
    if constexpr (KG_LATE) store_kg_rows();
    // tokens past the declared length: +0
    for (int i = tid; i < (it.len - it.n) * KD; i += 256)
        p.out[((int64_t)(it.t0 + it.n + i / KD) * p.HV + it.hv) * KD + (i & (KD - 1))] = 0;
}

// ------------------------------------------------------------ dispatch ----

template <int G, bool BF16>
hipError_t launch_rec_g(const RecParams &p, const Launch &l, hipStream_t s)
{
    if (l.family == KERNEL_RECURRENT_VARLEN)
        hipLaunchKernelGGL((kda_recurrent_kernel<G, BF16, true>), dim3(l.grid), dim3(l.block), 0, s, p);
    else
        hipLaunchKernelGGL((kda_recurrent_kernel<G, BF16, false>), dim3(l.grid), dim3(l.block), 0, s, p);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_rec_dt(const RecParams &p, const Launch &l, hipStream_t s)
{
    switch (l.rows_per_block) {
    case 128: return launch_rec_g<8, BF16>(p, l, s);
    case 64: return launch_rec_g<4, BF16>(p, l, s);
    case 32: return launch_rec_g<2, BF16>(p, l, s);
    case 16: return launch_rec_g<1, BF16>(p, l, s);
    default: return hipErrorInvalidValue;
    }
}

thread_local char g_hip_err[256];

int record(hipError_t e)
{
    if (e == hipSuccess) return 0;
    const char *n = hipGetErrorString(e);
    int i = 0;
    for (; n && n[i] && i < 255; ++i) g_hip_err[i] = n[i];
    g_hip_err[i] = 0;
    return -9;  // KDA_ERR_LAUNCH
}

}  // namespace

const char *last_hip_error() { return g_hip_err; }

int launch_recurrent(const RecParams &p, const Launch &l, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();  // a stale error must not be blamed on this launch
    if (l.family == KERNEL_VERIFY_WY) {
        // token slots sized to the declared length: 2, 4, 8, 12 or 16, the smallest that holds it
        // (12 slots: T=12 fp32 41.6 against 45.1 us on 16, bf16 29.6 against 35.8; 6 slots measured
        // no faster than 8)
        const dim3 grid(l.grid), block(l.block);
#define KDA_WY(TM_)                                                                                      \
    do {                                                                                                 \
        if (p.kg) {                                                                                      \
            if (l.bf16_state) hipLaunchKernelGGL((kda_verify_wy_kernel<true, TM_, true>), grid, block, 0, s, p);  \
            else hipLaunchKernelGGL((kda_verify_wy_kernel<false, TM_, true>), grid, block, 0, s, p);     \
        } else {                                                                                         \
            if (l.bf16_state) hipLaunchKernelGGL((kda_verify_wy_kernel<true, TM_, false>), grid, block, 0, s, p); \
            else hipLaunchKernelGGL((kda_verify_wy_kernel<false, TM_, false>), grid, block, 0, s, p);    \
        }                                                                                                \
    } while (0)
        if (p.tps <= 2) KDA_WY(2);
        else if (p.tps <= 4) KDA_WY(4);
        else if (p.tps <= 8) KDA_WY(8);
        else if (p.tps <= 12) KDA_WY(12);
        else KDA_WY(16);
#undef KDA_WY
        return record(hipGetLastError());
    }
    hipError_t e = l.bf16_state ? launch_rec_dt<true>(p, l, s) : launch_rec_dt<false>(p, l, s);
    return record(e);
}

int launch_fused(const FusedParams &p, const Launch &l, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (l.bf16_state)
        hipLaunchKernelGGL(kda_fused_kernel<true>, dim3(l.grid), dim3(l.block), 0, s, p);
    else
        hipLaunchKernelGGL(kda_fused_kernel<false>, dim3(l.grid), dim3(l.block), 0, s, p);
    return record(hipGetLastError());
}

int launch_packed_fused(const PackedFusedParams &p, const Launch &l, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const dim3 grid(l.grid), block(l.block);
#define KDA_PF_CASE(VS_, NT_, B_)                                                                         \
    case (VS_ * 2048 + NT_) * 2 + B_:                                                                     \
        hipLaunchKernelGGL((kda_packed_fused_kernel<B_ != 0, 2048 / (NT_ * VS_), VS_>), grid, block, 0, s, p); \
        break
    switch ((l.vsplit * 2048 + l.block) * 2 + l.bf16_state) {
        KDA_PF_CASE(1, 256, 0); KDA_PF_CASE(1, 256, 1);
        KDA_PF_CASE(1, 512, 0); KDA_PF_CASE(1, 512, 1);
        KDA_PF_CASE(2, 512, 0); KDA_PF_CASE(2, 512, 1);
        KDA_PF_CASE(4, 512, 0); KDA_PF_CASE(4, 512, 1);
    default: return record(hipErrorInvalidValue);
    }
#undef KDA_PF_CASE
    return record(hipGetLastError());
}

// The allocation-free packed fused entry point's split scratch: arrival
// counters then unnormalised outputs.  Zero when the code object is loaded;
// every split call returns each counter it uses to zero before it completes
// (all parts of a head arrive, or none), so the counters are zero whenever no
// call is running.  Host code never passes `scratch` itself to a kernel (on
// the host it names a stand-in, not device memory): it takes the device
// address of the current device's copy once, below.
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

int noalloc_scratch(void **ptr)
{
    static std::atomic<void *> known[64];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return record(e);
    if (dev < 0 || dev >= 64) return record(hipErrorInvalidDevice);
    void *p = known[dev].load(std::memory_order_acquire);
    if (!p) {
        // several host threads may race to fill the entry, all with the same value
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return record(e);
        if (!p) return record(hipErrorInvalidSymbol);
        known[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return 0;
}

int device_is_gfx950(int device)
{
    // 0 unknown, 1 gfx950, 2 other; calls from several host threads may race
    // to fill an entry, all with the same value
    static std::atomic<int> known[64];
    if (device < 0) return -1;
    if (device < 64) {
        const int k = known[device].load(std::memory_order_relaxed);
        if (k) return k == 1;
    }
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) {
        record(e);
        return -1;
    }
    int ok = 1;
    const char want[] = "gfx950";
    for (int i = 0; i < 6; ++i)
        if (prop.gcnArchName[i] != want[i]) ok = 0;
    if (device < 64) known[device].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok;
}

int current_device_is_gfx950(int *device_out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        record(e);
        return -1;
    }
    if (device_out) *device_out = dev;
    return device_is_gfx950(dev);
}

}  // namespace kda_detail
