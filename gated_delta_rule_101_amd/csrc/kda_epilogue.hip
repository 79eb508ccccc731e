// Output epilogue of the KDA read for gfx950: per (token, head) row of dv
// value channels,
//   y = o / sqrt(mean_j o_j^2 + eps) * weight * sigmoid(z).
//
// "Kimi K3 - Lesson 3 of 14 - Sequence axis", the output-gate paragraph: after
// the recurrent read a full-rank, input-dependent gate decides which channels
// of the result pass; "K3 Architecture Illustrated", the KDA section under
// FIG 21: the module includes normalisation and output gating.  The form is
// not given: RMS normalisation over the head's dv channels with a learnable
// per-channel weight, then a sigmoid gate from per-token logits z.
//
// The normalisation spans a whole dv row, which the chunk kernels split across
// workgroups (independent value slabs), so after a chunked forward this is a
// pass of its own: o, z read once, y written once, bound by HBM bandwidth.
// (The decode kernel holds whole rows and applies the same epilogue in place
// of its output store.)
//
// Layout: 16 lanes per row; lane l holds channels 64 j + 4 l + (0..3) for
// j < dv / 64, so each quarter-wave access covers 256 contiguous bytes of fp32
// (128 of bf16).  The row's sum of squares is reduced across its 16 lanes
// with cross-lane shuffles.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// o and z are read once and y written once: non-temporal accesses keep the
// stream from displacing cache lines that other work reuses (0.47 -> 0.44 ms
// over the training-shape reads).
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void nt_load4(Raw4<float> &r, const float *p) {
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    r.a = make_float4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void nt_load4(Raw4<uint16_t> &r, const uint16_t *p) {
    const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    r.a = make_uint2(t[0], t[1]);
}
__device__ __forceinline__ void nt_store4(float *p, const float (&x)[4]) {
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4 *>(p));
}
__device__ __forceinline__ void nt_store4(uint16_t *p, const float (&x)[4]) {
    const uint32_t lo = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
    __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2 *>(p));
}

constexpr int NTHREADS = 256;
constexpr int ROW_LANES = 16;
constexpr int ROWS_PER_BLOCK = NTHREADS / ROW_LANES;
constexpr unsigned MAX_BLOCKS = 1u << 20;   // grid-stride beyond this

// `o` and `y` may be the same buffer (each lane reads its elements before
// writing them), so neither is restrict-qualified.
template <int NJ, typename OT, typename ZT, typename YT>
__global__ void __launch_bounds__(NTHREADS)
kda_output_gate_kernel(const OT *o, const ZT *__restrict__ z, const float *__restrict__ weight, YT *y,
                       int64_t rows, float eps)
{
    constexpr int DV = 64 * NJ;
    const int l = threadIdx.x % ROW_LANES;

    float w[NJ][4];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const float4 t = *reinterpret_cast<const float4 *>(weight + 64 * j + 4 * l);
        w[j][0] = t.x; w[j][1] = t.y; w[j][2] = t.z; w[j][3] = t.w;
    }

    for (int64_t r0 = (int64_t)blockIdx.x * ROWS_PER_BLOCK; r0 < rows; r0 += (int64_t)gridDim.x * ROWS_PER_BLOCK) {
        const int64_t row = r0 + threadIdx.x / ROW_LANES;
        const bool live = row < rows;
        // a dead row (only in the last block) re-reads the last row, so every
        // lane of a 16-lane group takes part in the shuffles below
        const size_t base = (size_t)(live ? row : rows - 1) * DV + 4 * l;

        float ov[NJ][4], zv[NJ][4];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            Raw4<OT> ro;
            Raw4<ZT> rz;
            nt_load4(ro, o + base + 64 * j);
            nt_load4(rz, z + base + 64 * j);
            ro.to_f32(ov[j]);
            rz.to_f32(zv[j]);
        }
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) ss += ov[j][c] * ov[j][c];
#pragma unroll
        for (int m = 1; m < ROW_LANES; m <<= 1) ss += __shfl_xor(ss, m, ROW_LANES);
        const float inv = rsqrtf(ss * (1.f / DV) + eps);

        if (live) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                float yv[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) yv[c] = ov[j][c] * inv * w[j][c] * sigmoid_f32(zv[j][c]);
                nt_store4(y + base + 64 * j, yv);
            }
        }
    }
}

template <int NJ, typename OT, typename ZT, typename YT>
hipError_t launch(const OutputGateArgs &a, hipStream_t stream)
{
    const int64_t blocks = (a.rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
    const unsigned grid = (unsigned)(blocks < (int64_t)MAX_BLOCKS ? blocks : (int64_t)MAX_BLOCKS);
    kda_output_gate_kernel<NJ, OT, ZT, YT><<<grid, NTHREADS, 0, stream>>>(
        (const OT *)a.o, (const ZT *)a.z, a.weight, (YT *)a.y, a.rows, a.eps);
    return hipGetLastError();
}

template <int NJ, typename OT, typename ZT>
hipError_t dispatch_y(const OutputGateArgs &a, hipStream_t s)
{
    return a.y_bf16 ? launch<NJ, OT, ZT, uint16_t>(a, s) : launch<NJ, OT, ZT, float>(a, s);
}

template <int NJ>
hipError_t dispatch_dtypes(const OutputGateArgs &a, hipStream_t s)
{
    if (a.o_bf16)
        return a.z_bf16 ? dispatch_y<NJ, uint16_t, uint16_t>(a, s) : dispatch_y<NJ, uint16_t, float>(a, s);
    return a.z_bf16 ? dispatch_y<NJ, float, uint16_t>(a, s) : dispatch_y<NJ, float, float>(a, s);
}

}  // namespace

hipError_t launch_output_gate(const OutputGateArgs &a, hipStream_t stream)
{
    (void)hipGetLastError();
    switch (a.dv) {
    case 64: return dispatch_dtypes<1>(a, stream);
    case 128: return dispatch_dtypes<2>(a, stream);
    case 192: return dispatch_dtypes<3>(a, stream);
    case 256: return dispatch_dtypes<4>(a, stream);
    case 320: return dispatch_dtypes<5>(a, stream);
    case 384: return dispatch_dtypes<6>(a, stream);
    case 448: return dispatch_dtypes<7>(a, stream);
    case 512: return dispatch_dtypes<8>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
