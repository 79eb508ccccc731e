// Sequence-parallel chunked forward for grids too small to fill the device.
//
// Between chunks the chunkwise form is sequential ("Kimi K3 - Lesson 3 of 14 -
// Sequence axis", the chunkwise diagram: sequential between chunks, parallel
// within), but each chunk's step is affine in the state,
//   S' = (Diag(Gamma_C) - K-bar^T T Diag(beta) K~) S + K-bar^T T Diag(beta) V,
// so a run of chunks is too: S_out = M S_in + N.  The sequence is cut into P
// segments of T / P tokens, which the pipelined kernel runs side by side as a
// batch of B P sequences (the [B, T, H, d] layouts are already [B P, T / P, H,
// d]):
//   1. every segment from a zero state, its value slabs giving N_p and extra
//      transition slabs (identity start, zero values) giving M_p;
//   2. the segments' true starting states in order, S_{p+1} = M_p S_p + N_p
//      (fp32, this file), the last one being the final state;
//   3. every segment again from its true starting state, writing o.
// Steps 1 and 3 are each T / P chunks long instead of T; step 2 is P small
// products.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

// One workgroup per (b, h, CW state columns): S <- S0 (or 0); for each
// segment p, S_start[p] = S and S <- M_p S + N_p; S_final <- S.  fp32
// throughout.  M_p sits in LDS (rows padded to 16-byte multiples).  A thread
// takes one row of the product, all CW columns, over one of KS slices of the
// inner index; lanes RW apart hold the slices of one row, so the 16 lanes of
// an LDS read phase read 16 rows (no bank conflict), and the slices are added
// with cross-lane shuffles.  N and M are loaded ahead into two register sets
// used in turn, and M_{p+1} is written to the second LDS buffer once M_p's
// product is done.
template <int DK, int CW, int CT>
__global__ void __launch_bounds__(CT) seqpar_combine_kernel(const float *__restrict__ M, const float *__restrict__ N,
                                                            const float *S0, float *__restrict__ S_start,
                                                            float *S_final, int H, int P, int dv)
{
    constexpr int LDM = DK + 4;
    constexpr int KS = CT / DK;             // slices of the inner index
    constexpr int RW = 64 / KS;             // rows per wave
    constexpr int KL = DK / KS;             // inner length per slice
    constexpr int MV = DK * DK / 4 / CT;    // 16-byte pieces of M per thread
    static_assert(KS * DK == CT && RW * KS == 64 && CW % 4 == 0 && MV * 4 * CT == DK * DK, "thread layout");
    __shared__ alignas(16) float sM[2][DK * LDM];
    __shared__ alignas(16) float sS[DK][CW];
    const int ncg = dv / CW;
    const int bh = blockIdx.x / ncg, j0 = (blockIdx.x % ncg) * CW;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid % 64;
    const int row = (tid / 64) * RW + lane % RW, kq = lane / RW;
    auto seg = [&](int p) { return (size_t)(b * P + p) * H + h; };   // (sequence, head) of segment p

    struct Set {
        f32x4v m[MV];
        float n[CW];
    };
    auto fetch = [&](int p, Set &x) {
        if (p >= P) return;
        const float *n = N + (seg(p) * DK + row) * dv + j0;
#pragma unroll
        for (int j = 0; j < CW; ++j) x.n[j] = kq == 0 ? n[j] : 0.f;
        const f32x4v *src = reinterpret_cast<const f32x4v *>(M + seg(p) * DK * DK);
#pragma unroll
        for (int u = 0; u < MV; ++u) x.m[u] = src[tid + CT * u];
    };
    auto put = [&](float *dst, const Set &x) {
#pragma unroll
        for (int u = 0; u < MV; ++u) {
            const int e = 4 * (tid + CT * u);
            *reinterpret_cast<f32x4v *>(&dst[(e / DK) * LDM + e % DK]) = x.m[u];
        }
    };
    // segment p: `a` holds N_p and then receives segment p + 2; `nx` holds
    // segment p + 1, which goes to LDS once M_p's product is done
    auto step = [&](int p, Set &a, const Set &nx) {
        const float *Mr = sM[p & 1] + row * LDM + kq * KL;
        float acc[CW];
#pragma unroll
        for (int j = 0; j < CW; ++j) acc[j] = a.n[j];
        fetch(p + 2, a);
        for (int e = tid; e < DK * CW; e += CT) {
            const int r = e / CW, j = e % CW;
            S_start[(seg(p) * DK + r) * dv + j0 + j] = sS[r][j];
        }
#pragma unroll 2
        for (int kk = 0; kk < KL; kk += 4) {
            const f32x4v m4 = *reinterpret_cast<const f32x4v *>(&Mr[kk]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float *sr = sS[kq * KL + kk + u];
#pragma unroll
                for (int j = 0; j < CW; j += 4) {
                    const f32x4v s4 = *reinterpret_cast<const f32x4v *>(&sr[j]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[j + i] = fmaf(m4[u], s4[i], acc[j + i]);
                }
            }
        }
#pragma unroll
        for (int m = RW; m < 64; m *= 2)
#pragma unroll
            for (int j = 0; j < CW; ++j) acc[j] += __shfl_xor(acc[j], m);
        __syncthreads();   // every read of sS and of M_p is done
        if (kq == 0)
#pragma unroll
            for (int j = 0; j < CW; j += 4)
                *reinterpret_cast<f32x4v *>(&sS[row][j]) = f32x4v{acc[j], acc[j + 1], acc[j + 2], acc[j + 3]};
        if (p + 1 < P) put(sM[(p + 1) & 1], nx);
        __syncthreads();
    };

    for (int e = tid; e < DK * CW; e += CT) {
        const int r = e / CW, j = e % CW;
        sS[r][j] = S0 ? S0[((size_t)bh * DK + r) * dv + j0 + j] : 0.f;
    }
    Set x, y;
    fetch(0, x);
    fetch(1, y);
    put(sM[0], x);
    __syncthreads();
    for (int p = 0; p < P; p += 2) {
        step(p, x, y);
        if (p + 1 < P) step(p + 1, y, x);
    }
    if (S_final)
        for (int e = tid; e < DK * CW; e += CT) {
            const int r = e / CW, j = e % CW;
            S_final[((size_t)bh * DK + r) * dv + j0 + j] = sS[r][j];
        }
}

template <int DK>
void launch_combine(const float *M, const float *N, const float *S0, float *S_start, float *S_final, int B, int H,
                    int P, int dv, hipStream_t stream)
{
    // 4 columns per workgroup while 8 would leave CUs idle; each M_p is then
    // read by twice as many workgroups (from L2)
    const size_t wg8 = (size_t)B * H * (dv / 8);
    if (wg8 >= 256)
        seqpar_combine_kernel<DK, 8, 256><<<(unsigned)wg8, 256, 0, stream>>>(M, N, S0, S_start, S_final, H, P, dv);
    else {
        seqpar_combine_kernel<DK, 4, 256><<<(unsigned)(2 * wg8), 256, 0, stream>>>(M, N, S0, S_start, S_final, H, P, dv);
    }
}

}  // namespace

size_t chunk_seqpar_workspace_bytes(int B, int H, int dk, int dv, int P)
{
    const size_t n = (size_t)B * P * H;
    return n * ((size_t)2 * dk * dv + (size_t)dk * dk) * sizeof(float);
}

hipError_t launch_chunk_fwd_seqpar(const ChunkFwdArgs &a, int P, void *workspace, hipStream_t stream)
{
    (void)hipGetLastError();
    if (P < 1 || a.T % P != 0 || !a.qkv_bf16 || a.lengths || a.A_log || a.dv % 8) return hipErrorInvalidValue;
    const size_t n = (size_t)a.B * P * a.H;
    float *N = static_cast<float *>(workspace);
    float *M = N + n * a.dk * a.dv;
    float *S_start = M + n * a.dk * a.dk;

    // 1. each segment from a zero state: N (value slabs) and M (transition slabs)
    ChunkFwdArgs e = a;
    e.B = a.B * P;
    e.T = a.T / P;
    e.S0 = nullptr;
    e.o = nullptr;
    e.S_final = N;
    hipError_t err = launch_chunk_fwd_bf16_trans(e, M, stream);
    if (err != hipSuccess) return err;

    // 2. the segments' starting states and the final state
    if (a.dk == 64)
        launch_combine<64>(M, N, a.S0, S_start, a.S_final, a.B, a.H, P, a.dv, stream);
    else
        launch_combine<128>(M, N, a.S0, S_start, a.S_final, a.B, a.H, P, a.dv, stream);
    err = hipGetLastError();
    if (err != hipSuccess) return err;

    // 3. each segment from its true starting state, writing o
    ChunkFwdArgs f = a;
    f.B = a.B * P;
    f.T = a.T / P;
    f.S0 = S_start;
    f.S_final = nullptr;
    return launch_chunk_fwd_bf16(f, stream);
}

}  // namespace kda
