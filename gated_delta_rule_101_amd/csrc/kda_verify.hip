// Speculative verify and commit of up to 16 draft tokens per state on the
// matrix cores.
//
// "K3 Architecture Illustrated", speculative decoding: the target verifies a
// batch of draft tokens; KDA's state must be rolled back after rejections, so
// verify only reads the state.  Up to 16 drafts are one tile of the chunkwise
// form ("Kimi K3 - Lesson 3 of 14 - Sequence axis"), referenced to the state:
// with b the inclusive cumsum of the drafts' g (at most 80 in magnitude over
// 16 tokens under g >= -5),
//   Q~ = e^b q,  K~ = e^b k,  K^ = e^-b k  (<= e^80),
//   A_qk = tril(Q~ K^T),  A_kk = strict_tril(K~ K^T),
//   U = (I + Diag(beta) A_kk)^-1 Diag(beta) (V - K~ S),
//   O = Q~ S + A_qk U.
// Only the two products with the state are large: [Q~; K~] S is 32 x dk x dv
// per state, against the token loop's per-token state update.  Commit applies
// the first n = accepted[b] drafts (the rest enter as identity tokens) and
// needs no queries: with Gamma_n the decay of the whole prefix and
// K-bar = e^{b_n - b} k the keys decayed to its end,
//   S' = Diag(Gamma_n) S + K-bar^T U
// (the chunk-end state update of the chunkwise form), accumulated in the
// registers that loaded S and written back once.
//
// One 4-wave workgroup per state; wave w owns value columns
// [w dv/4, (w+1) dv/4) and streams its dk x dv/4 slice of S from HBM straight
// into matrix-core B operands (lane (kq, r16) reads dv/64 consecutive floats
// of row 16 kb + 4 kq + i: 16 lanes cover one contiguous row segment), so S
// never passes through LDS and the state is read exactly once.  For
// bfloat16 drafts the two state products take fp16 operands
// (v_mfma_f32_16x16x32_f16; the state must stay below the fp16 limit 65504,
// as in the bfloat16 chunk kernel), single fp16 terms for verify's
// outputs and two-term fp16 on both sides for the state commit keeps;
// everything else, and the whole float32 draft path, uses float32 operands
// (v_mfma_f32_16x16x4_f32).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int KT = 16;          // drafts per tile
constexpr int NTH = 256;
constexpr float LOG2E = 1.4426950408889634f;
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Loads element i unconditionally (i built from a draft index clamped into
// [0, K)) and zeroes it for drafts past the end; a branch around the load
// would make the code after it wait for each load in turn.
template <typename X>
__device__ __forceinline__ float ld_live(const X *p, size_t i, bool live)
{
    const float v = to_f32(p[i]);
    return live ? v : 0.f;
}

__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// At most 168 VGPRs, so three workgroups share a CU.
template <int DK, int DV, typename QT, typename GT, typename OT, bool COMMIT>
__global__ void __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(3)))
kda_verify_tile_kernel(const QT *__restrict__ q, const QT *__restrict__ k, const QT *__restrict__ v,
                       const GT *__restrict__ g, const GT *__restrict__ beta, float *__restrict__ S,
                       OT *__restrict__ o, const int *__restrict__ accepted, int K, int H)
{
    constexpr int CW = DV / 4;      // value columns per wave
    constexpr int NC = CW / 16;     // columns per lane (1 or 2)
    constexpr int LK = DK + 4, LV = DV + 4;
    __shared__ alignas(16) float sQt[KT][LK], sKt[KT][LK], sKh[KT][LK];
    __shared__ alignas(16) float sX[KT][LV];    // V - K~ S, then U
    __shared__ float sA[KT][KT + 4], sL[KT][KT + 4], sN[KT][KT + 4];
    __shared__ float sbeta[KT];
    __shared__ float sGam[DK];   // commit: decay of the whole accepted prefix, per key channel
    // commit: K-bar^T (keys decayed to the end of the accepted prefix), channel-major,
    // in the storage of the queries, which commit does not read
    static_assert(DK * KT <= KT * LK, "K-bar^T fits where the queries would go");
    float(*sKbT)[KT] = reinterpret_cast<float(*)[KT]>(&sQt[0][0]);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, kq = lane >> 4;
    const int col0 = wave * CW + NC * r16;   // this lane's first value column

    // The wave's dk x dv/4 slice of the state, in B-operand order (block kb,
    // step i: key channel 16 kb + 4 kq + i), requested before anything else
    // so its HBM latency overlaps the draft preparation.
    float sv[DK / 16][4][NC];
    auto load_state = [&](int bh) {
        const float *Sp = S + (size_t)bh * DK * DV;
#pragma unroll
        for (int kb = 0; kb < DK / 16; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float *p = Sp + (size_t)(16 * kb + 4 * kq + i) * DV + col0;
                if constexpr (NC == 2) {
                    const f32x2 t = __builtin_nontemporal_load(reinterpret_cast<const f32x2 *>(p));
                    sv[kb][i][0] = t[0];
                    sv[kb][i][1] = t[1];
                } else {
                    sv[kb][i][0] = __builtin_nontemporal_load(p);
                }
            }
    };

    const int bh = xcd_contiguous(blockIdx.x, gridDim.x);   // one state per workgroup
    load_state(bh);
    {
        const int b = bh / H, h = bh % H;
        // drafts applied: all K (verify), the accepted prefix (commit); the
        // others enter as identity tokens (zero key, value, decay and beta)
        const int n = COMMIT ? max(0, min(accepted[b], K)) : K;
        auto row = [&](int t) { return ((size_t)b * K + t) * H + h; };   // draft token t of (b, h)
        // drafts past the applied ones load the last applied draft's row (row 0
        // when none is applied; K >= 1) and are zeroed: their lines are already
        // being fetched, so commit reads only the accepted prefix from memory
        const int t_last = n > 0 ? n - 1 : 0;
        auto live_row = [&](int t) { return row(t < n ? t : t_last); };

        // this lane's draft values for X = V - K~ S (C layout: drafts 4 kq + i)
        float vv[4][NC];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * kq + i;
#pragma unroll
            for (int c = 0; c < NC; ++c) vv[i][c] = ld_live(v, live_row(t) * DV + col0 + c, t < n);
        }
        // drafts: raw q, k, g into LDS by the whole workgroup (g parked in sKh),
        // then the cumsum of g down each key channel and the scaled rows
        static_assert(KT * DK % (4 * NTH) == 0, "whole 4-channel groups per thread");
        // 4 consecutive channels per thread and load (8 or 16 bytes; rows are
        // 16-byte aligned and DK is a multiple of 4); fixed count, so all
        // loads issue first
#pragma unroll
        for (int it = 0; it < KT * DK / (4 * NTH); ++it) {
            const int e = tid + NTH * it, t = e / (DK / 4), x = 4 * (e % (DK / 4));
            const bool live = t < n;
            const size_t i = live_row(t) * DK + x;
            Raw4<QT> rq, rk;
            Raw4<GT> rg;
            if constexpr (!COMMIT) rq.load(q + i);
            else rq.zero();
            rk.load(k + i);
            rg.load(g + i);
            float fq[4], fk[4], fg[4];
            rq.to_f32(fq);
            rk.to_f32(fk);
            rg.to_f32(fg);
            f32x4 vq, vk, vg;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vq[j] = live ? fq[j] : 0.f;
                vk[j] = live ? fk[j] : 0.f;
                vg[j] = live ? fg[j] : 0.f;
            }
            if constexpr (!COMMIT) *reinterpret_cast<f32x4 *>(&sQt[t][x]) = vq;
            *reinterpret_cast<f32x4 *>(&sKt[t][x]) = vk;
            *reinterpret_cast<f32x4 *>(&sKh[t][x]) = vg;
        }
        if (tid < KT) sbeta[tid] = ld_live(beta, live_row(tid), tid < n);
        __syncthreads();
        if (tid < DK) {
            const int x = tid;
            float acc = 0.f;
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                acc += sKh[t][x];
                const float e = __builtin_amdgcn_exp2f(acc * LOG2E), ei = __builtin_amdgcn_exp2f(-acc * LOG2E);
                const float kv = sKt[t][x];
                if constexpr (!COMMIT) sQt[t][x] *= e;
                sKt[t][x] = kv * e;
                sKh[t][x] = kv * ei;
            }
            if constexpr (COMMIT) {
                // acc is the log-decay of the whole prefix (identity tokens add 0)
                const float ge = __builtin_amdgcn_exp2f(acc * LOG2E);
                sGam[x] = ge;
#pragma unroll
                for (int t = 0; t < KT; ++t) sKbT[x][t] = sKh[t][x] * ge;   // k e^{b_end - b_t} <= |k|
            }
        }
        __syncthreads();

        // [Q~; K~] S for this wave's columns
        f32x4 aq[NC], ak[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) aq[c] = ak[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (sizeof(QT) == 2) {
            // bfloat16 drafts: fp16 operands (Q~, K~ <= |q|, |k|; the state
            // below the fp16 limit), 16x16x32 products; single terms for
            // verify's outputs, two-term for the state commit keeps.  k-items of block pair
            // p: key channels 32p + 4kq + (0..3) and 32p + 16 + 4kq + (0..3),
            // which are exactly this lane's state rows of blocks 2p and 2p + 1.
#pragma unroll
            for (int p = 0; p < DK / 32; ++p) {
                const int x = 32 * p + 4 * kq;
                const f16x8 qa = h16::pack8(*reinterpret_cast<const f32x4 *>(&sQt[r16][x]),
                                                 *reinterpret_cast<const f32x4 *>(&sQt[r16][x + 16]));
                const f32x4 k0 = *reinterpret_cast<const f32x4 *>(&sKt[r16][x]);
                const f32x4 k1 = *reinterpret_cast<const f32x4 *>(&sKt[r16][x + 16]);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const f32x4 s0 = {sv[2 * p][0][c], sv[2 * p][1][c], sv[2 * p][2][c], sv[2 * p][3][c]};
                    const f32x4 s1 = {sv[2 * p + 1][0][c], sv[2 * p + 1][1][c], sv[2 * p + 1][2][c], sv[2 * p + 1][3][c]};
                    if constexpr (!COMMIT) {
                        const f16x8 sb = h16::pack8(s0, s1);
                        aq[c] = h16::mma32(qa, sb, aq[c]);
                        ak[c] = h16::mma32(h16::pack8(k0, k1), sb, ak[c]);
                    } else {
                        // the committed state persists: two-term fp16 on both
                        // sides (about 22 significant bits), three products
                        f16x8 kh, kl, sh, sl;
                        h16::split8(k0, k1, kh, kl);
                        h16::split8(s0, s1, sh, sl);
                        ak[c] = h16::mma32(kh, sh, ak[c]);
                        ak[c] = h16::mma32(kh, sl, ak[c]);
                        ak[c] = h16::mma32(kl, sh, ak[c]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int kb = 0; kb < DK / 16; ++kb) {
                const int x = 16 * kb + 4 * kq;
                const f32x4 qa = *reinterpret_cast<const f32x4 *>(&sQt[r16][x]);
                const f32x4 ka = *reinterpret_cast<const f32x4 *>(&sKt[r16][x]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        if constexpr (!COMMIT) aq[c] = mma(qa[i], sv[kb][i][c], aq[c]);
                        ak[c] = mma(ka[i], sv[kb][i][c], ak[c]);
                    }
            }
        }
        // aq[c], ak[c]: lane (kq, r16) holds draft rows 4 kq + i of column col0 + c.
        // X = V - K~ S to LDS (the B operand of the solve below).
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < NC; ++c) sX[4 * kq + i][col0 + c] = vv[i][c] - ak[c][i];
        // Gram tiles: wave 0 A_qk = tril(Q~ K^T) (verify only), wave 1 A_kk0 = strict_tril(K~ K^T)
        if (COMMIT ? wave == 1 : wave < 2) {
            const float(*L)[LK] = wave == 0 ? sQt : sKt;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < DK / 16; ++kb) {
                const int x = 16 * kb + 4 * kq;
                const f32x4 a = *reinterpret_cast<const f32x4 *>(&L[r16][x]);
                const f32x4 bb = *reinterpret_cast<const f32x4 *>(&sKh[r16][x]);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = mma(a[i], bb[i], acc);
            }
            // acc[i]: row 4 kq + i, column r16
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * kq + i, s = r16;
                if (wave == 0) sA[r][s] = s <= r ? acc[i] : 0.f;
                else sL[r][s] = s < r ? acc[i] : 0.f;
            }
        }
        __syncthreads();
        if (tid < KT) {   // column tid of N = (I + Diag(beta) A_kk0)^-1
            // forward substitution by columns: once x_l is final, every later
            // row takes its term at once (a dependent chain of KT steps)
            const int j = tid;
            float xs[KT];
#pragma unroll
            for (int i = 0; i < KT; ++i) xs[i] = i == j ? 1.f : 0.f;
#pragma unroll
            for (int l = 0; l < KT - 1; ++l) {
                const float nx = -xs[l];
#pragma unroll
                for (int i = l + 1; i < KT; ++i) xs[i] += (sbeta[i] * sL[i][l]) * nx;
            }
#pragma unroll
            for (int i = 0; i < KT; ++i) sN[i][j] = xs[i];
        }
        __syncthreads();
        // U = N Diag(beta) X for this wave's columns (lane (kq, r16) feeds
        // draft index 4 kq + i; the result lands in the same C layout as aq)
        f32x4 au[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) au[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = 4 * kq + i;
            const float a = sN[r16][s] * sbeta[s];
#pragma unroll
            for (int c = 0; c < NC; ++c) au[c] = mma(a, sX[s][col0 + c], au[c]);
        }
        if constexpr (COMMIT) {
            // S' = Diag(Gamma_end) S + K-bar^T U, accumulated in the registers
            // that hold S: output tile (channel block kb, column tile c) has lane
            // (kq, r16) on channels 16 kb + 4 kq + i of column tile c's column
            // r16, which is sv[kb][i][c].  The k-items are the drafts 4 kq +
            // (0..3), as U's accumulator layout gives them, so au[c] is the B
            // operand as it stands; A is read from K-bar^T's rows.
#pragma unroll
            for (int kb = 0; kb < DK / 16; ++kb) {
                const f32x4 gam = *reinterpret_cast<const f32x4 *>(&sGam[16 * kb + 4 * kq]);
                const f32x4 kbt = *reinterpret_cast<const f32x4 *>(&sKbT[16 * kb + r16][4 * kq]);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    f32x4 acc;
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = gam[i] * sv[kb][i][c];
                    if constexpr (sizeof(QT) == 2) {
                        // two-term fp16 K-bar (<= |k|) and U, three products
                        f16x4 kh, kl, uh, ul;
                        h16::split4(kbt, kh, kl);
                        h16::split4(au[c], uh, ul);
                        acc = h16::mma16(kh, uh, acc);
                        acc = h16::mma16(kh, ul, acc);
                        acc = h16::mma16(kl, uh, acc);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc = mma(kbt[i], au[c][i], acc);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) sv[kb][i][c] = acc[i];
                }
            }
            // written back where it was read; no accepted draft leaves S untouched
            if (n > 0) {
                float *Sp = S + (size_t)bh * DK * DV;
#pragma unroll
                for (int kb = 0; kb < DK / 16; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float *p = Sp + (size_t)(16 * kb + 4 * kq + i) * DV + col0;
                        if constexpr (NC == 2)
                            __builtin_nontemporal_store(f32x2{sv[kb][i][0], sv[kb][i][1]}, reinterpret_cast<f32x2 *>(p));
                        else
                            __builtin_nontemporal_store(sv[kb][i][0], p);
                    }
            }
        } else {
            __syncthreads();   // every wave has read its X before U overwrites it
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c = 0; c < NC; ++c) sX[4 * kq + i][col0 + c] = au[c][i];
            __syncthreads();
            // O = Q~ S + A_qk U, accumulated onto aq
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 4 * kq + i;
                const float a = sA[r16][s];
#pragma unroll
                for (int c = 0; c < NC; ++c) aq[c] = mma(a, sX[s][col0 + c], aq[c]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * kq + i;
                if (t < K) {
                    OT *op = o + row(t) * DV + col0;
#pragma unroll
                    for (int c = 0; c < NC; ++c) op[c] = from_f32<OT>(aq[c][i]);
                }
            }
        }
    }
}

template <int DK, int DV, typename QT, typename GT, typename OT, bool COMMIT>
hipError_t launch(const SpecArgs &a, hipStream_t s)
{
    kda_verify_tile_kernel<DK, DV, QT, GT, OT, COMMIT><<<(unsigned)(a.B * a.H), NTH, 0, s>>>(
        (const QT *)a.q, (const QT *)a.k, (const QT *)a.v, (const GT *)a.g, (const GT *)a.beta, a.S, (OT *)a.o,
        a.accepted, a.K, a.H);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t dispatch(const SpecArgs &a, hipStream_t s)
{
    typedef uint16_t b16;
    if (a.accepted) {   // commit: no outputs
        if (a.qkv_bf16)
            return a.gate_bf16 ? launch<DK, DV, b16, b16, float, true>(a, s) : launch<DK, DV, b16, float, float, true>(a, s);
        return a.gate_bf16 ? launch<DK, DV, float, b16, float, true>(a, s) : launch<DK, DV, float, float, float, true>(a, s);
    }
    if (a.qkv_bf16) {
        if (a.gate_bf16)
            return a.out_bf16 ? launch<DK, DV, b16, b16, b16, false>(a, s) : launch<DK, DV, b16, b16, float, false>(a, s);
        return a.out_bf16 ? launch<DK, DV, b16, float, b16, false>(a, s) : launch<DK, DV, b16, float, float, false>(a, s);
    }
    if (a.gate_bf16)
        return a.out_bf16 ? launch<DK, DV, float, b16, b16, false>(a, s) : launch<DK, DV, float, b16, float, false>(a, s);
    return a.out_bf16 ? launch<DK, DV, float, float, b16, false>(a, s) : launch<DK, DV, float, float, float, false>(a, s);
}

}  // namespace

hipError_t launch_verify_tile(const SpecArgs &a, hipStream_t stream)
{
    (void)hipGetLastError();
    if (a.dk == 64) return a.dv == 64 ? dispatch<64, 64>(a, stream) : dispatch<64, 128>(a, stream);
    return a.dv == 64 ? dispatch<128, 64>(a, stream) : dispatch<128, 128>(a, stream);
}

}  // namespace kda
