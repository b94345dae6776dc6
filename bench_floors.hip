// bench_floors.hip -- access-pattern floors for bench.py (measurement only;
// not part of the library, never called by it).
//
// Each kernel moves exactly the state bytes of one benchmarked workload, in
// that workload's access pattern (random pool slots, the tile a workgroup
// owns, the lane layout), and does one FMA per element and nothing else.
// Its time is the floor that pattern sets on this chip; bench.py reports it
// next to the kernel that carries the same bytes plus its arithmetic.
//
//  * floor_read_heads: read-only, one 256-thread workgroup per 64 KiB head
//    (fp32 128 x 128), each lane's values summed so that its loads stay
//    live, one float per workgroup stored.  Lane layout 0: whole rows, each wave instruction 1 KiB of
//    consecutive rows and the four waves side by side 4 KiB; layout 1: the
//    16x16 matrix-core operand order (16 rows x 64 bytes per instruction,
//    the two 64-byte halves of a 128-byte line in consecutive instructions).
//  * floor_rmw_slices: in place, one 256-thread workgroup per slice of 4,
//    8, 16 or 32 KiB of a head, each lane 16 bytes per 4 KiB; rows whose slot
//    is negative are skipped (null rows).
//  * floor_read1_write_k: the packed fused call's state traffic, one
//    256-thread workgroup per (sequence, head): the head block of the
//    sequence's first slot is read once and written to each of its K slots
//    (one per token).
//
// All loads and stores are nontemporal dwordx4, like the library's state
// traffic.  Workgroups are numbered XCD by XCD as in the library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int xcd_work()
{
    return (int)(blockIdx.x & 7u) * (int)(gridDim.x >> 3) + (int)(blockIdx.x >> 3);
}

template <int LAYOUT>
__global__ void __launch_bounds__(256) read_heads_kernel(const char *pool, const int *idx, float *out, int n_work,
                                                         int H)
{
    const int work = xcd_work();
    if (work >= n_work) return;
    const int seq = work / H, h = work - (work / H) * H;
    const char *head = pool + ((int64_t)idx[seq] * H + h) * 65536;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    f32x4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        uint32_t off;
        if constexpr (LAYOUT == 0) {
            off = (uint32_t)i * 4096u + 16u * (uint32_t)tid;
        } else {
            const int tau = i >> 3, j = i & 7;
            const int row = 32 * wave + 16 * tau + (lane & 15);
            off = (uint32_t)(row * 512 + (16 * j + 4 * (lane >> 4)) * 4);
        }
        v[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(head + off));
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = acc * 0.5f + v[i];
    // every lane's sum is live (a store no value in practice takes), so
    // every lane's loads stay in the kernel
    const float sum = acc.x + acc.y + acc.z + acc.w;
    if (tid == 0 || sum == -1.2345e-30f) out[work] = sum;
}

template <int NP>
__global__ void __launch_bounds__(256) rmw_slices_kernel(char *pool, const int *idx, int n_work, int H,
                                                         int head_bytes, int ns)
{
    const int work = xcd_work();
    if (work >= n_work) return;
    const int vs = work % ns, item = work / ns;
    const int seq = item / H, h = item - (item / H) * H;
    const int slot = idx[seq];
    if (slot < 0) return;
    char *base = pool + ((int64_t)slot * H + h) * head_bytes + (int64_t)vs * (NP * 4096);
    const uint32_t t16 = 16u * threadIdx.x;
    f32x4 v[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) v[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(base + i * 4096 + t16));
#pragma unroll
    for (int i = 0; i < NP; ++i)
        __builtin_nontemporal_store(v[i] * 0.999f + 0.001f, reinterpret_cast<f32x4 *>(base + i * 4096 + t16));
}

template <int NP>
__global__ void __launch_bounds__(256) read1_write_k_kernel(char *pool, const int *idx, int n_work, int H,
                                                            int head_bytes, int K)
{
    const int work = xcd_work();
    if (work >= n_work) return;
    const int seq = work / H, h = work - (work / H) * H;
    const int *row = idx + (int64_t)seq * K;
    const uint32_t t16 = 16u * threadIdx.x;
    const char *src = pool + ((int64_t)row[0] * H + h) * head_bytes;
    f32x4 v[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) v[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src + i * 4096 + t16));
    for (int k = 0; k < K; ++k) {
        char *dst = pool + ((int64_t)row[k] * H + h) * head_bytes;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            v[i] = v[i] * 0.999f + 0.001f;
            __builtin_nontemporal_store(v[i], reinterpret_cast<f32x4 *>(dst + i * 4096 + t16));
        }
    }
}

}  // namespace

// n_seqs x H heads of 64 KiB, head (s, h) at pool + ((idx[s] * H) + h) * 64 KiB;
// out: n_seqs * H floats.  Returns 0, -1 for a bad argument, -2 for a launch error.
extern "C" __attribute__((visibility("default"))) int floor_read_heads(const void *pool, const int *idx, float *out,
                                                                       int n_seqs, int H, int layout, void *stream)
{
    if (!pool || !idx || !out || n_seqs <= 0 || H <= 0 || (layout != 0 && layout != 1)) return -1;
    const int n_work = n_seqs * H;
    const dim3 grid((unsigned)((n_work + 7) & ~7)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (layout == 0) hipLaunchKernelGGL(read_heads_kernel<0>, grid, block, 0, s, (const char *)pool, idx, out, n_work, H);
    else hipLaunchKernelGGL(read_heads_kernel<1>, grid, block, 0, s, (const char *)pool, idx, out, n_work, H);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// n_rows x H heads of head_bytes, each in slices of slice_bytes (4, 8, 16 or
// 32 KiB, dividing head_bytes), updated in place; idx[r] < 0 skips row r.
extern "C" __attribute__((visibility("default"))) int floor_rmw_slices(void *pool, const int *idx, int n_rows, int H,
                                                                       int head_bytes, int slice_bytes, void *stream)
{
    if (!pool || !idx || n_rows <= 0 || H <= 0 || slice_bytes <= 0 || head_bytes <= 0 || head_bytes % slice_bytes)
        return -1;
    const int ns = head_bytes / slice_bytes;
    const int n_work = n_rows * H * ns;
    const dim3 grid((unsigned)((n_work + 7) & ~7)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *p = static_cast<char *>(pool);
    switch (slice_bytes) {
    case 4096: hipLaunchKernelGGL(rmw_slices_kernel<1>, grid, block, 0, s, p, idx, n_work, H, head_bytes, ns); break;
    case 8192: hipLaunchKernelGGL(rmw_slices_kernel<2>, grid, block, 0, s, p, idx, n_work, H, head_bytes, ns); break;
    case 16384: hipLaunchKernelGGL(rmw_slices_kernel<4>, grid, block, 0, s, p, idx, n_work, H, head_bytes, ns); break;
    case 32768: hipLaunchKernelGGL(rmw_slices_kernel<8>, grid, block, 0, s, p, idx, n_work, H, head_bytes, ns); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// n_seqs x H heads of head_bytes (32 or 64 KiB); idx: n_seqs x K slots; head
// (s, h) is read from slot idx[s][0] and written to idx[s][0..K).
extern "C" __attribute__((visibility("default"))) int floor_read1_write_k(void *pool, const int *idx, int n_seqs, int H,
                                                                          int head_bytes, int K, void *stream)
{
    if (!pool || !idx || n_seqs <= 0 || H <= 0 || K <= 0 || (head_bytes != 32768 && head_bytes != 65536)) return -1;
    const int n_work = n_seqs * H;
    const dim3 grid((unsigned)((n_work + 7) & ~7)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *p = static_cast<char *>(pool);
    if (head_bytes == 65536) hipLaunchKernelGGL(read1_write_k_kernel<16>, grid, block, 0, s, p, idx, n_work, H, head_bytes, K);
    else hipLaunchKernelGGL(read1_write_k_kernel<8>, grid, block, 0, s, p, idx, n_work, H, head_bytes, K);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
