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
// Steps 1 and 3 each carry the state over T / P tokens instead of T; step 2
// is P small products in sequence.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int CT = 256;   // threads per combine workgroup
constexpr int CW_MIN = 4; // state columns per combine workgroup: 4, or 8 where 4 would overfill the device

// One workgroup per (b, h, CW state columns): S <- S0 (or 0); for each segment
// p, S_start[p] = S and S <- M_p S + N_p; S_final <- S.  fp32 throughout.
//
// Thread (slice, rg) computes a 4 x CW block of each product -- rows rg + R i
// (R = DK / 4, i = 0..3), all CW columns -- over one of KS slices of KL
// inner indices (lane bits 0 .. log2 KS - 1 are the slice).  Its M_p entries
// (4 rows x KL) come straight from global memory into registers, loaded two
// segments ahead into two register sets used in turn.  S sits in LDS,
// double-buffered so that one barrier per segment separates the reads of S_p
// from the writes of S_{p+1}, with one padding row per slice so that the
// slices' reads of one instruction fall in distinct banks.  The slices are
// added by a reduce-scatter over DPP row patterns, after which each lane holds
// 4 CW / KS of the block's sums.
template <int L> struct Level { static constexpr int value = L; };

// Reduce-scatter level k over the 16 lanes of a DPP row: lane x pairs with
// x ^ 15 (row mirror), x ^ 7 within its half (half-row mirror), x ^ 1 or x ^ 2
// (quad permutations).  The masks span the four slice bits, and the slice bit
// that decides which half a lane keeps, {3, 2, 0, 1}, is one in which the pair
// differs and which every later level's pairs share.
constexpr int dpp_ctrl(int k) { return k == 0 ? 0x140 : k == 1 ? 0x141 : k == 2 ? 0xB1 : 0x4E; }
constexpr int dpp_bit(int k) { return k == 0 ? 3 : k == 1 ? 2 : k == 2 ? 0 : 1; }
template <int CTRL> __device__ __forceinline__ float dpp_from(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int DK, int CW>
__global__ void __launch_bounds__(CT) seqpar_combine_kernel(const float *__restrict__ M, const float *__restrict__ N,
                                                            const float *S0, float *__restrict__ S_start,
                                                            float *S_final, int H, int P, int dv)
{
    constexpr int R = DK / 4;                // row groups
    constexpr int KS = CT / R;               // slices of the inner index
    constexpr int KL = DK / KS;              // inner indices per slice
    constexpr int LOGKS = KS == 8 ? 3 : 4;
    constexpr int NACC = 4 * CW;             // sums per thread before the reduce-scatter
    constexpr int LOGO = CW == 4 ? 4 : 5;    // bits of a block index
    constexpr int NOUT = NACC / KS;          // sums per lane after it
    constexpr int SROWS = DK + KS;           // S rows in LDS, one padding row per slice
    static_assert(KS * R == CT && (1 << LOGKS) == KS && KL % 4 == 0 && NOUT >= 1 && DK * CW % CT == 0 &&
                  (1 << LOGO) == NACC, "thread layout");
    static_assert(LOGKS == 3 || LOGKS == 4, "the slices of a group lie in one 16-lane DPP row");
    __shared__ alignas(16) float sS[2][SROWS][CW];
    const int ncg = dv / CW;
    const int bh = blockIdx.x / ncg, j0 = (blockIdx.x % ncg) * CW;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x;
    const int slice = tid % KS, rg = tid / KS;   // slice = the low bits of the lane
    auto seg = [&](int p) { return (size_t)(b * P + p) * H + h; };   // (sequence, head) of segment p
    auto srow = [](int k) { return k + k / KL; };                     // LDS row of state row k

    // this lane's sums after the reduce-scatter: level l fixes bit LOGO - 1 - l
    // of the block index o (row rg + R (o / CW), column o % CW) from slice bit
    // dpp_bit(l + FIRST); the remaining low bits of o are j
    constexpr int FIRST = 4 - LOGKS;   // dk = 128 (8 slices) starts at the half-row mirror
    int out_row[NOUT], out_col[NOUT];
#pragma unroll
    for (int j = 0; j < NOUT; ++j) {
        int o = 0;
#pragma unroll
        for (int L = 0; L < LOGKS; ++L) o |= ((slice >> dpp_bit(L + FIRST)) & 1) << (LOGO - 1 - L);
        o |= j;
        out_row[j] = rg + R * (o / CW);
        out_col[j] = o % CW;
    }

    f32x4v mx[4][KL / 4], my[4][KL / 4];
    float nx[NOUT], ny[NOUT];
    // past the last segment a fetch reloads the last one (every call issues the
    // same loads)
    auto fetch = [&](int p, f32x4v (&m)[4][KL / 4], float (&n)[NOUT]) {
        p = p < P ? p : P - 1;
        const float *Mp = M + seg(p) * DK * DK;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int u = 0; u < KL / 4; ++u)
                m[i][u] = *reinterpret_cast<const f32x4v *>(&Mp[(size_t)(rg + R * i) * DK + KL * slice + 4 * u]);
#pragma unroll
        for (int j = 0; j < NOUT; ++j) n[j] = N[(seg(p) * DK + out_row[j]) * dv + j0 + out_col[j]];
    };

    for (int e = tid; e < DK * CW; e += CT) {
        const int r = e / CW, j = e % CW;
        sS[0][srow(r)][j] = S0 ? S0[((size_t)bh * DK + r) * dv + j0 + j] : 0.f;
    }
    fetch(0, mx, nx);
    fetch(1, my, ny);
    __syncthreads();

    // segment p: M_p and N_p in (m, n), which then receive segment p + 2
    auto step = [&](int p, f32x4v (&m)[4][KL / 4], float (&n)[NOUT]) {
        const int cur = p & 1;
#pragma unroll
        for (int u = 0; u < DK * CW / CT; ++u) {   // a fixed number of stores, as for the loads
            const int e = tid + CT * u, r = e / CW, j = e % CW;
            S_start[(seg(p) * DK + r) * dv + j0 + j] = sS[cur][srow(r)][j];
        }
        float acc[NACC];
#pragma unroll
        for (int o = 0; o < NACC; ++o) acc[o] = 0.f;
#pragma unroll
        for (int u = 0; u < KL / 4; ++u) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int c4 = 0; c4 < CW / 4; ++c4) {
                    const f32x4v s4 = *reinterpret_cast<const f32x4v *>(&sS[cur][srow(KL * slice + 4 * u + kk)][4 * c4]);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            acc[CW * i + 4 * c4 + c] = fmaf(m[i][u][kk], s4[c], acc[CW * i + 4 * c4 + c]);
                }
            }
        }
        float nn[NOUT];
#pragma unroll
        for (int j = 0; j < NOUT; ++j) nn[j] = n[j];
        fetch(p + 2, m, n);
        // reduce-scatter: at level L a lane keeps the half of its sums whose
        // index bit LOGO - 1 - L equals its slice bit dpp_bit(L + FIRST) and
        // adds the partner's copy of that half
        auto level = [&](auto lv) __attribute__((always_inline)) {
            constexpr int L = decltype(lv)::value, K = L + FIRST, cnt = (NACC / 2) >> L;
            const bool hi = (slice >> dpp_bit(K)) & 1;
#pragma unroll
            for (int j = 0; j < cnt; ++j) {
                const float send = hi ? acc[j] : acc[j + cnt];
                const float keep = hi ? acc[j + cnt] : acc[j];
                acc[j] = keep + dpp_from<dpp_ctrl(K)>(send);
            }
        };
        level(Level<0>{});
        level(Level<1>{});
        level(Level<2>{});
        if constexpr (LOGKS == 4) level(Level<3>{});
        float *nxt = &sS[cur ^ 1][0][0];
#pragma unroll
        for (int j = 0; j < NOUT; ++j) nxt[srow(out_row[j]) * CW + out_col[j]] = acc[j] + nn[j];
        __syncthreads();
    };
    for (int p = 0; p < P; p += 2) {
        step(p, mx, nx);
        if (p + 1 < P) step(p + 1, my, ny);
    }
    if (S_final)
        for (int e = tid; e < DK * CW; e += CT) {
            const int r = e / CW, j = e % CW;
            S_final[((size_t)bh * DK + r) * dv + j0 + j] = sS[P & 1][srow(r)][j];
        }
}

// 8 columns per workgroup where 4 would give more workgroups than the device
// has compute units: the workgroups of a head each read all of M_p, so fewer of
// them read less of it
template <int DK>
void launch_combine(const float *M, const float *N, const float *S0, float *S_start, float *S_final, int B, int H,
                    int P, int dv, int cus, hipStream_t stream)
{
    const size_t groups4 = (size_t)B * H * (dv / 4);
    if (dv % 8 == 0 && groups4 > (size_t)cus)
        seqpar_combine_kernel<DK, 8><<<(unsigned)(groups4 / 2), CT, 0, stream>>>(M, N, S0, S_start, S_final, H, P, dv);
    else
        seqpar_combine_kernel<DK, 4><<<(unsigned)groups4, CT, 0, stream>>>(M, N, S0, S_start, S_final, H, P, dv);
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
    if (P < 1 || a.T % P != 0 || !a.qkv_bf16 || a.lengths || a.dv % CW_MIN) return hipErrorInvalidValue;
    int dev = 0, cus = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
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
    err = launch_chunk_fwd_bf16_trans(e, M, stream);
    if (err != hipSuccess) return err;

    // 2. the segments' starting states and the final state
    if (a.dk == 64)
        launch_combine<64>(M, N, a.S0, S_start, a.S_final, a.B, a.H, P, a.dv, cus, stream);
    else
        launch_combine<128>(M, N, a.S0, S_start, a.S_final, a.B, a.H, P, a.dv, cus, stream);
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
