// Achievable-peak probes for the benchmark (not part of the KDA library):
// streaming device copies (the HBM bandwidth a plain kernel reaches) and a
// loop of independent bf16 16x16x32 matrix-core products (the MFMA issue rate
// a plain kernel reaches).  Built into libkda_probe.so; bench.py calls them
// through ctypes and reports the KDA kernels' fractions against both these
// and the published peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming kernels: workgroup w moves the 1024 consecutive 16-byte units
// starting at unit 1024 w (16 KB), each thread four units 256 apart (every
// instruction covers 4 KB of consecutive bytes across the workgroup), with
// non-temporal loads and stores.  Of the forms tried on MI355X (spans of 16
// KB to 1 MB per workgroup, 4 or 8 units in flight, 256 or 512 threads,
// cached or non-temporal), this one moved the most bytes per second.
constexpr int SPAN = 1024;   // units per workgroup
constexpr int UNITS = 4;     // units per thread

// dst[i] = src[i]
__global__ void __launch_bounds__(256) probe_copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst)
{
    const size_t base = (size_t)blockIdx.x * SPAN + threadIdx.x;
    u32x4 x[UNITS];
#pragma unroll
    for (int u = 0; u < UNITS; ++u) x[u] = __builtin_nontemporal_load(&src[base + 256 * u]);
#pragma unroll
    for (int u = 0; u < UNITS; ++u) __builtin_nontemporal_store(x[u], &dst[base + 256 * u]);
}

// buf[i] ^= mask in place (read and write the same lines, as a state update does)
__global__ void __launch_bounds__(256) probe_update_kernel(u32x4 *__restrict__ buf, uint32_t mask)
{
    const size_t base = (size_t)blockIdx.x * SPAN + threadIdx.x;
    u32x4 x[UNITS];
#pragma unroll
    for (int u = 0; u < UNITS; ++u) x[u] = __builtin_nontemporal_load(&buf[base + 256 * u]);
#pragma unroll
    for (int u = 0; u < UNITS; ++u) __builtin_nontemporal_store(x[u] ^ mask, &buf[base + 256 * u]);
}
static_assert(SPAN == UNITS * 256, "one pass per workgroup");

// Each wave runs `iters` rounds of NACC independent bf16 matrix-core products
// (16x16x32: 2 * 16 * 16 * 32 FLOP each; 32x32x16: 2 * 32 * 32 * 16) and
// writes one float per lane so nothing is optimised away.
constexpr int NACC = 8;
template <bool BIG>
__global__ void __launch_bounds__(256) probe_mfma_kernel(float *__restrict__ out, int iters)
{
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    typedef typename std::conditional<BIG, f32x16, f32x4>::type acc_t;
    constexpr int NA = BIG ? NACC / 2 : NACC;
    const unsigned t = threadIdx.x + 1u;
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(float)((t * (i + 3)) & 7) * (__bf16)0.125f;
        b[i] = (__bf16)(float)((t * (i + 5)) & 7) * (__bf16)0.0625f;
    }
    acc_t acc[NA];
    for (int j = 0; j < NA; ++j) acc[j] = acc_t{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < NA; ++j) {
            if constexpr (BIG) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
            else acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
        }
    }
    float s = 0.f;
    for (int j = 0; j < NA; ++j)
        for (int e = 0; e < (BIG ? 16 : 4); ++e) s += acc[j][e];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Copy `bytes` (a multiple of 16384, at most 2^44; both pointers 16-byte
// aligned) on `stream`.
int kda_probe_copy(const void *src, void *dst, size_t bytes, void *stream)
{
    const size_t span = (size_t)SPAN * 16;
    if (!src || !dst || bytes == 0 || bytes % span || bytes / span > 0x7FFFFFFFu || ((uintptr_t)src | (uintptr_t)dst) & 15) return 1;
    hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)(bytes / span)), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4 *)src, (u32x4 *)dst);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

// buf ^= mask in place over `bytes` (as for the copy).
int kda_probe_update(void *buf, size_t bytes, unsigned mask, void *stream)
{
    const size_t span = (size_t)SPAN * 16;
    if (!buf || bytes == 0 || bytes % span || bytes / span > 0x7FFFFFFFu || (uintptr_t)buf & 15) return 1;
    hipLaunchKernelGGL(probe_update_kernel, dim3((unsigned)(bytes / span)), dim3(256), 0, (hipStream_t)stream,
                       (u32x4 *)buf, (uint32_t)mask);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

// `blocks` workgroups of four waves, `iters` rounds each; `out` holds
// blocks * 256 floats.  big = 0: FLOP = blocks * 4 * iters * 8 * 16384
// (16x16x32); big = 1: blocks * 4 * iters * 4 * 32768 (32x32x16).
int kda_probe_mfma(float *out, int blocks, int iters, int big, void *stream)
{
    if (!out || blocks <= 0 || iters <= 0) return 1;
    if (big)
        hipLaunchKernelGGL(probe_mfma_kernel<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    else
        hipLaunchKernelGGL(probe_mfma_kernel<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
