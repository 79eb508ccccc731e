// Speculative-decoding verify and commit for gfx950: K draft tokens per
// (sequence, head) state, applied one after another to the state held in
// registers.
//
// "K3 Architecture Illustrated", speculative decoding: a draft proposes
// several tokens, the target verifies them in a batch, and the recurrent
// state has to roll back to the accepted prefix.  Verify runs the drafts
// through a register copy of S and writes their outputs; S in memory is not
// touched.  Commit runs the first accepted[b] drafts of each sequence and
// writes the state back; the rest are never applied.  Either way S is read
// once from HBM (and written once by commit), like a decode step.  The
// library runs this token loop for more than 16 drafts; up to 16 go through
// one tile of the chunkwise form on the matrix cores instead.
//
// Layout as the decode kernel: one 256-thread workgroup per state (dk x dv,
// float32, dv contiguous); thread (row group rg, column group cg) holds
// columns 4cg..4cg+3 of rows rg, rg + NRG, ...; a wave's two halves read two
// adjacent full rows per 16-byte load.  Per token, with alpha = exp(g):
//   p = S^T (alpha . k),  r = S^T (alpha . q),  w = beta (v - p),
//   o = r + (q . k) w,    S <- Diag(alpha) S + k w^T
// (one token of the recurrence: fade, erase/write, read after the write;
// "Review A - Sequence and depth", Free recall).  The column sums over dk are
// reduced through LDS, double-buffered so each token costs one barrier.
// The drafts' q, k, alpha, v and beta are staged in LDS 16 tokens at a time;
// the arithmetic is float32 throughout.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int NTHREADS = 256;
constexpr int KBLK = 16;   // draft tokens staged per pass

template <int DK, int DV, bool QBF, bool GBF, bool OBF, bool COMMIT>
__global__ void __launch_bounds__(NTHREADS)
kda_spec_kernel(const typename Store<QBF>::type *__restrict__ q,
                const typename Store<QBF>::type *__restrict__ k,
                const typename Store<QBF>::type *__restrict__ v,
                const typename Store<GBF>::type *__restrict__ g,
                const typename Store<GBF>::type *__restrict__ beta,
                float *__restrict__ S, typename Store<OBF>::type *__restrict__ o,
                const int *__restrict__ accepted, int K, int H)
{
    typedef typename Store<OBF>::type OT;
    constexpr int NCG = DV / 4;            // column groups of 4
    constexpr int NRG = NTHREADS / NCG;    // row groups
    constexpr int RPT = DK / NRG;          // rows per thread
    static_assert(RPT * NRG == DK && RPT % 4 == 0, "rows must split evenly, four at a time");

    // Per-token key-side rows are stored permuted: the RPT rows a thread owns
    // (rg, rg + NRG, ...) sit next to each other at rg * RPT, so it fetches
    // them with RPT / 4 16-byte reads (broadcast across its column groups).
    __shared__ alignas(16) float s_q[KBLK][DK], s_k[KBLK][DK], s_a[KBLK][DK];
    __shared__ alignas(16) float s_v[KBLK][DV];
    __shared__ float s_b[KBLK];
    __shared__ f32x4 s_p[2][NRG][NCG], s_r[2][NRG][NCG];
    __shared__ float s_qk[2][NRG];

    const int bh = xcd_contiguous(blockIdx.x, gridDim.x), b = bh / H, h = bh % H;   // one state per workgroup
    const int cg = threadIdx.x % NCG;
    const int rg = threadIdx.x / NCG;
    f32x4 *Sp = reinterpret_cast<f32x4 *>(S + (size_t)bh * DK * DV);
    // tokens [0, n) are applied: all K for verify, the accepted prefix for commit
    const int n = COMMIT ? max(0, min(accepted[b], K)) : K;

    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(&Sp[(rg + NRG * i) * NCG + cg]);

    int par = 0;
    for (int t0 = 0; t0 < n; t0 += KBLK) {
        const int nb = min(KBLK, n - t0);
        if (t0 > 0) lds_barrier();   // every thread is done with the previous block
        // stage the block: token t of (b, h) sits at row (b K + t) H + h.  A
        // fixed count of unconditional loads (slots past the block re-read
        // its last token and are never used), so every load issues before
        // the first wait.
#pragma unroll
        for (int it = 0; it < KBLK * DK / NTHREADS; ++it) {
            const int e = threadIdx.x + NTHREADS * it, j = e / DK, c = e % DK;
            const size_t row = ((size_t)b * K + t0 + min(j, nb - 1)) * H + h;
            const int pc = (c % NRG) * RPT + c / NRG;
            if constexpr (!COMMIT) s_q[j][pc] = to_f32(q[row * DK + c]);
            s_k[j][pc] = to_f32(k[row * DK + c]);
            s_a[j][pc] = __expf(to_f32(g[row * DK + c]));
        }
#pragma unroll
        for (int it = 0; it < KBLK * DV / NTHREADS; ++it) {
            const int e = threadIdx.x + NTHREADS * it, j = e / DV, c = e % DV;
            s_v[j][c] = to_f32(v[(((size_t)b * K + t0 + min(j, nb - 1)) * H + h) * DV + c]);
        }
        if (threadIdx.x < KBLK)
            s_b[threadIdx.x] = to_f32(beta[((size_t)b * K + t0 + min((int)threadIdx.x, nb - 1)) * H + h]);
        lds_barrier();

        for (int j = 0; j < nb; ++j) {
            float a[RPT], kk[RPT], qq[RPT];
#pragma unroll
            for (int i = 0; i < RPT; i += 4) {
                *reinterpret_cast<f32x4 *>(&a[i]) = *reinterpret_cast<const f32x4 *>(&s_a[j][rg * RPT + i]);
                *reinterpret_cast<f32x4 *>(&kk[i]) = *reinterpret_cast<const f32x4 *>(&s_k[j][rg * RPT + i]);
                if constexpr (!COMMIT)
                    *reinterpret_cast<f32x4 *>(&qq[i]) = *reinterpret_cast<const f32x4 *>(&s_q[j][rg * RPT + i]);
            }
            f32x4 p = {0.f, 0.f, 0.f, 0.f}, rd = {0.f, 0.f, 0.f, 0.f};
            float qk = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                p += s[i] * (a[i] * kk[i]);
                if constexpr (!COMMIT) {
                    rd += s[i] * (a[i] * qq[i]);
                    qk += qq[i] * kk[i];
                }
            }
            s_p[par][rg][cg] = p;
            if constexpr (!COMMIT) {
                s_r[par][rg][cg] = rd;
                if (cg == 0) s_qk[par][rg] = qk;
            }
            lds_barrier();

            f32x4 pt = {0.f, 0.f, 0.f, 0.f}, rt = {0.f, 0.f, 0.f, 0.f};
            float qkt = 0.f;
#pragma unroll
            for (int x = 0; x < NRG; ++x) {
                pt += s_p[par][x][cg];
                if constexpr (!COMMIT) {
                    rt += s_r[par][x][cg];
                    qkt += s_qk[par][x];
                }
            }
            const f32x4 vv = *reinterpret_cast<const f32x4 *>(&s_v[j][4 * cg]);
            const f32x4 w = s_b[j] * (vv - pt);
            if constexpr (!COMMIT) {
                if (rg == 0) {
                    OT *op = o + (((size_t)b * K + t0 + j) * H + h) * DV + 4 * cg;
#pragma unroll
                    for (int c = 0; c < 4; ++c) op[c] = from_f32<OT>(rt[c] + qkt * w[c]);
                }
            }
#pragma unroll
            for (int i = 0; i < RPT; ++i) s[i] = a[i] * s[i] + kk[i] * w;
            par ^= 1;
        }
    }

    if constexpr (COMMIT) {
        if (n > 0) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) __builtin_nontemporal_store(s[i], &Sp[(rg + NRG * i) * NCG + cg]);
        }
    }
}

template <int DK, int DV, bool QBF, bool GBF, bool OBF, bool COMMIT>
hipError_t launch(const SpecArgs &a, hipStream_t stream)
{
    typedef typename Store<QBF>::type QT;
    typedef typename Store<GBF>::type GT;
    typedef typename Store<OBF>::type OT;
    kda_spec_kernel<DK, DV, QBF, GBF, OBF, COMMIT><<<(unsigned)(a.B * a.H), NTHREADS, 0, stream>>>(
        (const QT *)a.q, (const QT *)a.k, (const QT *)a.v, (const GT *)a.g, (const GT *)a.beta,
        a.S, (OT *)a.o, a.accepted, a.K, a.H);
    return hipGetLastError();
}

template <int DK, int DV, bool QBF, bool GBF>
hipError_t dispatch_mode(const SpecArgs &a, hipStream_t s)
{
    if (a.accepted) return launch<DK, DV, QBF, GBF, false, true>(a, s);
    return a.out_bf16 ? launch<DK, DV, QBF, GBF, true, false>(a, s) : launch<DK, DV, QBF, GBF, false, false>(a, s);
}

template <int DK, int DV>
hipError_t dispatch_dtypes(const SpecArgs &a, hipStream_t s)
{
    if (a.qkv_bf16)
        return a.gate_bf16 ? dispatch_mode<DK, DV, true, true>(a, s) : dispatch_mode<DK, DV, true, false>(a, s);
    return a.gate_bf16 ? dispatch_mode<DK, DV, false, true>(a, s) : dispatch_mode<DK, DV, false, false>(a, s);
}

}  // namespace

hipError_t launch_spec_step(const SpecArgs &a, hipStream_t stream)
{
    (void)hipGetLastError();
    if (a.dk == 64) return a.dv == 64 ? dispatch_dtypes<64, 64>(a, stream) : dispatch_dtypes<64, 128>(a, stream);
    return a.dv == 64 ? dispatch_dtypes<128, 64>(a, stream) : dispatch_dtypes<128, 128>(a, stream);
}

}  // namespace kda
