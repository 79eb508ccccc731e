// Chunkwise KDA forward for gfx950.
//
// One workgroup of 4 waves owns one (sequence, head, 64-wide slab of value
// columns) and walks that head's chunks of 64 tokens in order, carrying its
// dk x 64 slab of the float32 state in registers the whole way.  The value
// columns of S evolve independently (each column follows
// s <- (I - beta k k^T) Diag(alpha) s + beta k v_col), so slabs of one head
// never exchange data.
//
// Per chunk ("Kimi K3 - Lesson 3 of 14 - Sequence axis": sequential between
// chunks, parallel within; output = inter-chunk (Gamma . Q) S plus masked
// intra-chunk A V~; keys rescaled by 1/Gamma inside 16-token tiles, which
// the g_min = -5 floor keeps below e^80):
//
//   prep   wave m takes tile m (16 tokens).  b = within-tile inclusive
//          cumsum of g (a DPP scan across the 16 lanes of a row), f = e^b
//          (in [e^-80, 1]), 1/f (at most e^80), tile totals D_m.  Builds
//          Gamma.Q and Gamma.K (Gamma = decay from chunk start), the keys
//          decayed to the chunk end (K-bar, for the state update) and to
//          their tile end (for off-diagonal tile products).
//   Gram   wave m computes block row m of A_qk (lower, diagonal included)
//          and of the erase matrix L = StrictLower(Diag(beta) A_kk), where
//          A(r,s) = sum_c x_rc k_sc e^{b_rc - b_sc}.  The diagonal tile pairs
//          f-scaled rows with 1/f-scaled keys, both referenced to the tile
//          start, so every factor stays within [e^-80, e^80] and the tile is
//          one dense matrix-core product; off-diagonal tiles pair f-scaled
//          rows with keys decayed to their own tile end, times the whole
//          tiles in between.  Wave m then inverts its unit-lower diagonal
//          block I + L_mm by column-oriented forward substitution.
//   state  wave w owns value columns 16w..16w+15 of the slab:
//            X = V - (Gamma.K) S,   U = (I + L)^-1 Diag(beta) X  (blocked
//            forward substitution over the four 16-token tiles),
//            O = (Gamma.Q) S + A_qk U,   S <- Diag(Gamma_C) S + K-bar^T U.
//
// The algebra is the token recurrence re-associated (exact up to rounding).
//
// Precision with bfloat16 inputs.  The output is sensitive to four products:
// the A_qk Gram, (Gamma.Q) S, A_qk U and K-bar^T U.  Each of them splits both
// operands into high + low bfloat16 parts and sums three matrix-core products
// (hi.hi + hi.lo + lo.hi), about 16 significant bits.  (Gamma.K) S, the A_kk
// Gram and L U use single bfloat16 operands; the diagonal inverses are
// applied to a split right-hand side.  float32 inputs use float32 operands
// throughout (no split).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int C = 64;             // tokens per chunk
constexpr int TILE = 16;          // tokens per tile
constexpr int NT = C / TILE;      // tiles per chunk
constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int WV = 16 * NWAVES;   // value columns per workgroup
constexpr float LOG2E = 1.4426950408889634f;

// Off-diagonal tile pairs (m, n), n < m, in the order (1,0) (2,0) (2,1) (3,0) (3,1) (3,2).
__host__ __device__ constexpr int pair_index(int m, int n) { return m * (m - 1) / 2 + n; }
constexpr int NPAIRS = NT * (NT - 1) / 2;

template <int DK, bool BF>
struct ChunkSmem {
    typedef typename Prec<BF>::elem E;
    static constexpr int NP = BF ? 2 : 1;            // split parts kept: hi (+ lo)
    static constexpr int PAD = 16 / (int)sizeof(E);  // 16 bytes per row
    static constexpr int LDK = DK + PAD;             // token x channel rows
    static constexpr int LDC = C + PAD;              // 64-wide rows
    static constexpr int LD16 = TILE + 4;            // 16-wide rows of the inverses
    // Keys of tile n decayed to the start of tile m, one 16-row block per
    // off-diagonal pair (m, n): read only by the Gram products, then the same
    // storage holds the Gram results.
    struct KvarBuf { E K[NPAIRS][NP][TILE * LDK]; };
    struct GramBuf {
        E Aqk[NP][C * LDC];          // A_qk                          [token][token]
        E L[C * LDC];                // StrictLower(Diag(beta) A_kk)   [token][token]
        float Ld[NT][TILE][TILE];    // diagonal blocks of L, transposed: [m][col][row]
    };
    union U {
        KvarBuf kv;
        GramBuf gr;
    };
    E Qt[NP][C * LDK];               // Gamma . Q                  [token][channel]
    E Kt[C * LDK];                   // Gamma . K                  [token][channel]
    E KbT[NP][DK * LDC];             // K decayed to chunk end     [channel][token]
    U u;
    E Inv[NT][TILE * LD16];          // (I + L_mm)^-1              [m][row][col]
    float D[NT][DK];                 // total decay of each tile
    float GamC[DK];                  // total decay of the chunk
    float beta[C];
};

// Everything one chunk reads from HBM, as raw storage bits.
template <int DK, typename QT, typename GT>
struct ChunkIn {
    static constexpr int KB = DK / 32;
    Raw8<QT> q[KB], k[KB];   // row (tile = wave, row = lane%16), channels 32j + 8(lane/16) + 0..7
    Raw8<GT> g[KB];
    GT beta;
    QT v[NT][4];             // rows 16m + 4(lane/16) + i, column 16*wave + lane%16 of the slab
};

template <int DK, bool QBF, bool GBF, bool OBF, bool GL>
__global__ void __launch_bounds__(NTHREADS, 1)
kda_chunk_fwd_kernel(const typename Store<QBF>::type *__restrict__ q,
                     const typename Store<QBF>::type *__restrict__ k,
                     const typename Store<QBF>::type *__restrict__ v,
                     const typename Store<GBF>::type *__restrict__ g,
                     const typename Store<GBF>::type *__restrict__ beta,
                     const float *S0, typename Store<OBF>::type *__restrict__ o,
                     float *S_final, const int *__restrict__ lengths, const float *__restrict__ A_log,
                     int B, int T, int H, int dv, int nslab)
{
    typedef Prec<QBF> P;
    typedef typename P::elem E;
    typedef typename P::frag8 F8;
    typedef typename P::frag4 F4;
    typedef typename Store<QBF>::type QT;
    typedef typename Store<GBF>::type GT;
    typedef typename Store<OBF>::type OT;
    typedef ChunkSmem<DK, QBF> SM;
    constexpr bool SPLIT = P::SPLIT;
    constexpr int KB = DK / 32;   // 32-channel blocks
    constexpr int KT = DK / 16;   // 16-channel tiles
    constexpr int LDK = SM::LDK, LDC = SM::LDC, LD16 = SM::LD16;

    __shared__ SM sm;
    E(&Kv)[NPAIRS][SM::NP][TILE * LDK] = sm.u.kv.K;
    E(&Aqk)[SM::NP][C * LDC] = sm.u.gr.Aqk;
    E(&Lm)[C * LDC] = sm.u.gr.L;
    float(&Ld)[NT][TILE][TILE] = sm.u.gr.Ld;

    const int lane = threadIdx.x & 63;
    // wave index, made explicitly uniform: every branch on it (and the matrix-core
    // instructions inside those branches, which ignore the exec mask) stays scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15;     // row / column inside a 16x16 tile
    const int gq = lane >> 4;    // lane group: k-items, or output rows 4gq..4gq+3

    // Workgroup -> (b, h, slab).  Workgroups are dealt to the 8 XCDs round
    // robin; give the slabs of one head the same XCD so they share its L2
    // for the q, k, g reads they have in common.
    const int BH = B * H;
    int bh, slab;
    if ((BH & 7) == 0) {
        const int rest = blockIdx.x >> 3;
        slab = rest % nslab;
        bh = (rest / nslab) * 8 + (blockIdx.x & 7);
    } else {
        bh = blockIdx.x / nslab;
        slab = blockIdx.x % nslab;
    }
    const int b = bh / H, h = bh % H;
    const int col0 = slab * WV + 16 * wave;   // first value column owned by this wave
    const int nchunks = (T + C - 1) / C;
    // tokens from `len` on are identity tokens (no decay, no write)
    const int len = lengths ? max(0, min(lengths[b], T)) : T;
    const float gate_scale = GL ? __expf(A_log[h]) : 1.f;   // exp(A_h), gate logits only

    auto row_qk = [&](int t) -> size_t { return ((size_t)b * T + t) * H + h; };

    // ------------------------------------------------ initial state slab
    f32x4 S[KT];
    const size_t s_base = (size_t)bh * DK * dv + col0 + r;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[kt][i] = S0 ? S0[s_base + (size_t)(16 * kt + 4 * gq + i) * dv] : 0.f;

    // Loads are unconditional: a token past the end re-reads the last real
    // token (or token 0), so padding content never enters the arithmetic, and
    // is turned into an identity token where its values are used (g, beta, q,
    // k zeroed; its v only meets beta = 0).  A branch
    // around the loads would make the code after it wait for each of them.
    const int last = len > 0 ? len - 1 : 0;   // what a token past the end re-reads
    auto load_chunk = [&](ChunkIn<DK, QT, GT> &in, int c) {
        const int t = c * C + TILE * wave + r;
        const size_t rr = row_qk(t < len ? t : last);
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            in.q[j].load(q + rr * DK + 32 * j + 8 * gq);
            in.k[j].load(k + rr * DK + 32 * j + 8 * gq);
            in.g[j].load(g + rr * DK + 32 * j + 8 * gq);
        }
        in.beta = beta[rr];
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t2 = c * C + TILE * m + 4 * gq + i;
                in.v[m][i] = v[row_qk(t2 < len ? t2 : last) * dv + col0 + r];
            }
    };

    // One set of input registers: the prep consumes q, k, g, beta, then the
    // loads of the next chunk are issued into the same registers while the
    // Gram and state parts run; only v is kept back for the state part.
    ChunkIn<DK, QT, GT> cur;
    if (nchunks > 0) load_chunk(cur, 0);

    for (int c = 0; c < nchunks; ++c) {

        // ====================================================== prep (wave m = tile m)
        const int m = wave;
        const bool live = c * C + TILE * m + r < len;   // else an identity token
        float fdec[KB][8];   // f = decay since the tile start, in [e^-80, 1]
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            float gl[8];
            cur.g[j].to_f32(gl);
            if constexpr (GL) {   // an identity token keeps g = 0, not the gate of logit 0
#pragma unroll
                for (int i = 0; i < 8; ++i) gl[i] = live ? gate_from_logit(gl[i], gate_scale) : 0.f;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) gl[i] = live ? gl[i] : 0.f;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                fdec[j][i] = fast_exp2(row_inclusive_scan(gl[i] * LOG2E));
            if (r == TILE - 1) {
                *reinterpret_cast<f32x4 *>(&sm.D[m][32 * j + 8 * gq]) = f32x4{fdec[j][0], fdec[j][1], fdec[j][2], fdec[j][3]};
                *reinterpret_cast<f32x4 *>(&sm.D[m][32 * j + 8 * gq + 4]) = f32x4{fdec[j][4], fdec[j][5], fdec[j][6], fdec[j][7]};
            }
        }
        lds_barrier();

        // f-scaled rows of tile m (query: split, key: single), kept for the
        // Gram products, and the 1/f-scaled keys of the diagonal tile.  This
        // loop issues no matrix-core instruction: every accumulation chain
        // sits in the straight-line Gram block below.
        F8 aqh[KB], aql[KB], akh[KB], bih[KB], bil[KB];

#pragma unroll
        for (int j = 0; j < KB; ++j) {
            const int ch = 32 * j + 8 * gq;
            float Dt[NT][8];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const f32x4 x0 = *reinterpret_cast<const f32x4 *>(&sm.D[t][ch]);
                const f32x4 x1 = *reinterpret_cast<const f32x4 *>(&sm.D[t][ch + 4]);
#pragma unroll
                for (int i = 0; i < 4; ++i) { Dt[t][i] = x0[i]; Dt[t][4 + i] = x1[i]; }
            }
            // whole-tile decay before and after tile m (m is uniform per wave), and
            // from the end of tile m to the starts of tiles m + 2 and m + 3
            float before[8], after[8], Dm[8], p1[8], p2[8];
            switch (m) {
            case 0:
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    before[i] = 1.f; Dm[i] = Dt[0][i]; p1[i] = Dt[1][i]; p2[i] = Dt[1][i] * Dt[2][i];
                    after[i] = p2[i] * Dt[3][i];
                }
                break;
            case 1:
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    before[i] = Dt[0][i]; Dm[i] = Dt[1][i]; p1[i] = Dt[2][i]; p2[i] = 1.f;
                    after[i] = Dt[2][i] * Dt[3][i];
                }
                break;
            case 2:
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    before[i] = Dt[0][i] * Dt[1][i]; Dm[i] = Dt[2][i]; p1[i] = 1.f; p2[i] = 1.f;
                    after[i] = Dt[3][i];
                }
                break;
            default:
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    before[i] = Dt[0][i] * Dt[1][i] * Dt[2][i]; Dm[i] = Dt[3][i]; p1[i] = 1.f; p2[i] = 1.f;
                    after[i] = 1.f;
                }
                break;
            }
            if (m == 0 && r == 0) {
                f32x4 g0, g1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    g0[i] = after[i] * Dm[i];
                    g1[i] = after[4 + i] * Dm[4 + i];
                }
                *reinterpret_cast<f32x4 *>(&sm.GamC[ch]) = g0;
                *reinterpret_cast<f32x4 *>(&sm.GamC[ch + 4]) = g1;
            }
            float qv[8], kv[8];
            cur.q[j].to_f32(qv);
            cur.k[j].to_f32(kv);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                qv[i] = live ? qv[i] : 0.f;
                kv[i] = live ? kv[i] : 0.f;
            }
            float qt[8], ktv[8], kh[8], kb[8], qf[8], kf[8], ki[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float f = fdec[j][i];
                qf[i] = qv[i] * f;
                kf[i] = kv[i] * f;
                ki[i] = kv[i] * fast_rcp(f);          // 1/f-scaled key, <= e^80 |k|
                kh[i] = ki[i] * Dm[i];                // decayed to the tile end, <= |k|
                qt[i] = qf[i] * before[i];
                ktv[i] = kf[i] * before[i];
                kb[i] = kh[i] * after[i];
            }
            P::split8(qf, aqh[j], aql[j]);
            akh[j] = P::pack8(kf);
            P::split8(ki, bih[j], bil[j]);
            P::split_sts8(&sm.Qt[0][(TILE * m + r) * LDK + ch], &sm.Qt[SM::NP - 1][(TILE * m + r) * LDK + ch], qt);
            P::sts8(&sm.Kt[(TILE * m + r) * LDK + ch], ktv);
            // keys of tile m decayed to the start of each later tile m + d: pair (m + d, m)
            if (m + 1 < NT) {
                const int pi = pair_index(m + 1, m);
                P::split_sts8(&Kv[pi][0][r * LDK + ch], &Kv[pi][SM::NP - 1][r * LDK + ch], kh);
            }
            if (m + 2 < NT) {
                float kvv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) kvv[i] = kh[i] * p1[i];
                const int pi = pair_index(m + 2, m);
                P::split_sts8(&Kv[pi][0][r * LDK + ch], &Kv[pi][SM::NP - 1][r * LDK + ch], kvv);
            }
            if (m + 3 < NT) {
                float kvv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) kvv[i] = kh[i] * p2[i];
                const int pi = pair_index(m + 3, m);
                P::split_sts8(&Kv[pi][0][r * LDK + ch], &Kv[pi][SM::NP - 1][r * LDK + ch], kvv);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                E hi, lo;
                P::split1(kb[i], hi, lo);
                sm.KbT[0][(ch + i) * LDC + TILE * m + r] = hi;
                if constexpr (SPLIT) sm.KbT[1][(ch + i) * LDC + TILE * m + r] = lo;
            }
        }
        if (gq == 0) sm.beta[TILE * m + r] = live ? to_f32(cur.beta) : 0.f;
        lds_barrier();

        // ====================================================== Gram (wave m = block row m)
        // Straight-line: the diagonal tile, then the three tiles to its left
        // (n = m - d); a wave with fewer than three reads a valid stand-in and
        // discards the result, so no matrix-core chain sits under a branch.
        f32x4 gq_d = {0.f, 0.f, 0.f, 0.f}, gk_d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            gq_d = P::mma32(aqh[j], bih[j], gq_d);
            if constexpr (SPLIT) {
                gq_d = P::mma32(aqh[j], bil[j], gq_d);
                gq_d = P::mma32(aql[j], bih[j], gq_d);
            }
            gk_d = P::mma32(akh[j], bih[j], gk_d);
        }
        f32x4 gq_o[NT - 1], gk_o[NT - 1];
#pragma unroll
        for (int d = 1; d < NT; ++d) {
            const int pi = (m - d >= 0) ? pair_index(m, m - d) : 0;
            f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                const int ch = 32 * j + 8 * gq;
                F8 bh, bl;
                bh = P::lds8(&Kv[pi][0][r * LDK + ch]);
                if constexpr (SPLIT) bl = P::lds8(&Kv[pi][1][r * LDK + ch]);
                aq = P::mma32(aqh[j], bh, aq);
                if constexpr (SPLIT) {
                    aq = P::mma32(aqh[j], bl, aq);
                    aq = P::mma32(aql[j], bh, aq);
                }
                ak = P::mma32(akh[j], bh, ak);
            }
            gq_o[d - 1] = aq;
            gk_o[d - 1] = ak;
        }
        const f32x4 bet = *reinterpret_cast<const f32x4 *>(&sm.beta[TILE * m + 4 * gq]);
        lds_barrier();   // every wave is done reading the key variants (their storage is reused)
        f32x4 ldiag;
        {
            E qh[4], ql[4], kl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * gq + i;   // row inside the tile; the column is r
                const float aq = (r > row) ? 0.f : gq_d[i];            // keep s <= t
                const float ak = (r >= row) ? 0.f : gk_d[i] * bet[i];  // keep s <  t
                ldiag[i] = ak;
                P::split1(aq, qh[i], ql[i]);
                kl[i] = P::cvt(ak);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int a = (TILE * m + 4 * gq + i) * LDC + TILE * m + r;
                Aqk[0][a] = qh[i];
                if constexpr (SPLIT) Aqk[1][a] = ql[i];
                Lm[a] = kl[i];
            }
        }
#pragma unroll
        for (int d = 1; d < NT; ++d) {
            E qh[4], ql[4], kl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                P::split1(gq_o[d - 1][i], qh[i], ql[i]);
                kl[i] = P::cvt(gk_o[d - 1][i] * bet[i]);
            }
            const int n = m - d;
            if (n >= 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int a = (TILE * m + 4 * gq + i) * LDC + TILE * n + r;
                    Aqk[0][a] = qh[i];
                    if constexpr (SPLIT) Aqk[1][a] = ql[i];
                    Lm[a] = kl[i];
                }
            }
        }
        *reinterpret_cast<f32x4 *>(&Ld[m][r][4 * gq]) = ldiag;

        // next chunk's inputs: issued here, they land during the inverse and state parts
        QT vcur[NT][4];
#pragma unroll
        for (int mm = 0; mm < NT; ++mm)
#pragma unroll
            for (int i = 0; i < 4; ++i) vcur[mm][i] = cur.v[mm][i];
        if (c + 1 < nchunks) load_chunk(cur, c + 1);
        lds_wave_sync();

        // (I + L_mm)^-1: lane column r, column-oriented forward substitution
        {
            float X[TILE];
#pragma unroll
            for (int i = 0; i < TILE; ++i) X[i] = (i == r) ? 1.f : 0.f;
#pragma unroll
            for (int jj = 0; jj < TILE - 1; ++jj) {
                float Lc[TILE];   // column jj of L_mm
#pragma unroll
                for (int i4 = 0; i4 < TILE / 4; ++i4) {
                    const f32x4 x = *reinterpret_cast<const f32x4 *>(&Ld[m][jj][4 * i4]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) Lc[4 * i4 + i] = x[i];
                }
#pragma unroll
                for (int ii = jj + 1; ii < TILE; ++ii) X[ii] -= Lc[ii] * X[jj];
            }
            if (gq == 0) {
#pragma unroll
                for (int i = 0; i < TILE; ++i) sm.Inv[m][i * LD16 + r] = P::cvt(X[i]);
            }
        }
        lds_barrier();

        // ====================================================== state part (wave w = columns)
        F8 Sh[KB], Sl[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) P::split8(S[2 * j], S[2 * j + 1], Sh[j], Sl[j]);

        f32x4 accQ[NT], Y[NT];
#pragma unroll
        for (int mm = 0; mm < NT; ++mm) {
            f32x4 aQ = {0.f, 0.f, 0.f, 0.f}, aK = {0.f, 0.f, 0.f, 0.f};
            const int row = TILE * mm + r;
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                const int ch = row * LDK + 32 * j + 4 * gq;
                const F8 qh = P::lds4x2(&sm.Qt[0][ch], &sm.Qt[0][ch + 16]);
                aQ = P::mma32(qh, Sh[j], aQ);
                if constexpr (SPLIT) {
                    const F8 ql = P::lds4x2(&sm.Qt[1][ch], &sm.Qt[1][ch + 16]);
                    aQ = P::mma32(qh, Sl[j], aQ);
                    aQ = P::mma32(ql, Sh[j], aQ);
                }
                aK = P::mma32(P::lds4x2(&sm.Kt[ch], &sm.Kt[ch + 16]), Sh[j], aK);
            }
            accQ[mm] = aQ;
            const f32x4 bt = *reinterpret_cast<const f32x4 *>(&sm.beta[TILE * mm + 4 * gq]);
#pragma unroll
            for (int i = 0; i < 4; ++i) Y[mm][i] = bt[i] * (to_f32(vcur[mm][i]) - aK[i]);
        }

        // U = (I + L)^-1 Diag(beta) X, one 16-token tile at a time
        F4 Uh[NT], Ul[NT];
        f32x4 U[NT];
#pragma unroll
        for (int mm = 0; mm < NT; ++mm) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int n = 0; n < mm; ++n)
                acc = P::mma16(P::lds4(&Lm[(TILE * mm + r) * LDC + TILE * n + 4 * gq]), Uh[n], acc);
            F4 rh, rl;
            P::split4(Y[mm] - acc, rh, rl);
            const F4 inv = P::lds4(&sm.Inv[mm][r * LD16 + 4 * gq]);
            f32x4 u = P::mma16(inv, rh, f32x4{0.f, 0.f, 0.f, 0.f});
            if constexpr (SPLIT) u = P::mma16(inv, rl, u);
            U[mm] = u;
            P::split4(u, Uh[mm], Ul[mm]);
        }

        // O = (Gamma.Q) S + A_qk U, stored straight from the accumulators
#pragma unroll
        for (int mm = 0; mm < NT; ++mm) {
            f32x4 acc = accQ[mm];
#pragma unroll
            for (int n = 0; n <= mm; ++n) {
                const int a = (TILE * mm + r) * LDC + TILE * n + 4 * gq;
                const F4 ah = P::lds4(&Aqk[0][a]);
                acc = P::mma16(ah, Uh[n], acc);
                if constexpr (SPLIT) {
                    acc = P::mma16(ah, Ul[n], acc);
                    acc = P::mma16(P::lds4(&Aqk[1][a]), Uh[n], acc);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = c * C + TILE * mm + 4 * gq + i;
                if (o && t < T) o[row_qk(t) * dv + col0 + r] = from_f32<OT>(acc[i]);
            }
        }

        // S <- Diag(Gamma_C) S + K-bar^T U
        F8 Ubh[2], Ubl[2];
        P::split8(U[0], U[1], Ubh[0], Ubl[0]);
        P::split8(U[2], U[3], Ubh[1], Ubl[1]);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const f32x4 gcv = *reinterpret_cast<const f32x4 *>(&sm.GamC[16 * kt + 4 * gq]);
            f32x4 acc = S[kt] * gcv;
            const int row = (16 * kt + r) * LDC;
#pragma unroll
            for (int j2 = 0; j2 < 2; ++j2) {
                const int tk = row + 32 * j2 + 4 * gq;
                const F8 kh = P::lds4x2(&sm.KbT[0][tk], &sm.KbT[0][tk + 16]);
                acc = P::mma32(kh, Ubh[j2], acc);
                if constexpr (SPLIT) {
                    acc = P::mma32(kh, Ubl[j2], acc);
                    acc = P::mma32(P::lds4x2(&sm.KbT[1][tk], &sm.KbT[1][tk + 16]), Ubh[j2], acc);
                }
            }
            S[kt] = acc;
        }
        lds_barrier();
    }

    if (S_final) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S_final[s_base + (size_t)(16 * kt + 4 * gq + i) * dv] = S[kt][i];
    }
}

template <int DK, bool QBF, bool GBF, bool OBF, bool GL>
hipError_t launch(const ChunkFwdArgs &a, hipStream_t stream)
{
    typedef typename Store<QBF>::type QT;
    typedef typename Store<GBF>::type GT;
    typedef typename Store<OBF>::type OT;
    const int nslab = a.dv / WV;
    const unsigned grid = (unsigned)(a.B * a.H * nslab);
    kda_chunk_fwd_kernel<DK, QBF, GBF, OBF, GL><<<grid, NTHREADS, 0, stream>>>(
        (const QT *)a.q, (const QT *)a.k, (const QT *)a.v, (const GT *)a.g, (const GT *)a.beta,
        a.S0, (OT *)a.o, a.S_final, a.lengths, a.A_log, a.B, a.T, a.H, a.dv, nslab);
    return hipGetLastError();
}

template <int DK, bool QBF, bool GBF, bool GL>
hipError_t dispatch_gate(const ChunkFwdArgs &a, hipStream_t s)
{
    return a.out_bf16 ? launch<DK, QBF, GBF, true, GL>(a, s) : launch<DK, QBF, GBF, false, GL>(a, s);
}

template <int DK, bool QBF, bool GBF>
hipError_t dispatch_out(const ChunkFwdArgs &a, hipStream_t s)
{
    return a.A_log ? dispatch_gate<DK, QBF, GBF, true>(a, s) : dispatch_gate<DK, QBF, GBF, false>(a, s);
}

template <int DK>
hipError_t dispatch_dtypes(const ChunkFwdArgs &a, hipStream_t s)
{
    return a.gate_bf16 ? dispatch_out<DK, false, true>(a, s) : dispatch_out<DK, false, false>(a, s);
}

}  // namespace

hipError_t launch_chunk_fwd(const ChunkFwdArgs &a, hipStream_t stream)
{
    if (a.qkv_bf16) return launch_chunk_fwd_bf16(a, stream);
    (void)hipGetLastError();   // report only this launch's own failure
    if (a.dk == 64) return dispatch_dtypes<64>(a, stream);
    return dispatch_dtypes<128>(a, stream);
}

}  // namespace kda
