// Single-token KDA decode for gfx950: one streaming pass over the fp32 state.
//
// One workgroup of 256 threads owns one (sequence, head) state S (dk x dv,
// float32, dv contiguous).  Thread (row group rg, column group cg) holds
// columns 4cg..4cg+3 of rows rg, rg + NRG, rg + 2 NRG, ...; a wave's two
// halves read two adjacent full rows per 16-byte load, so every load and
// store instruction moves whole 512-byte rows.  S is read once and written
// once with non-temporal hints: the step is bound by HBM bandwidth.
//
// With D = Diag(exp g) (fade each key channel first, "Review A - Sequence
// and depth", Free recall; "K3 Architecture Illustrated", FIG 21):
//   p = S^T (alpha . k)          what the key retrieves from the faded state
//   w = beta (v - p)             the correction the delta rule writes
//   o = S^T (alpha . q) + (q.k) w   the read of the updated state
//   S <- D S + k w^T
// which is one token of the recurrence with a single read and write of S.
//
// With the output epilogue fused (OG), each thread's four outputs are
// normalised by the RMS of the head's dv outputs (reduced across the row
// group's lanes), scaled by the per-channel weight and gated by
// sigmoid(z_out) before the store ("Kimi K3 - Lesson 3 of 14", the output-gate
// paragraph; the form is read as RMS normalisation then a sigmoid gate).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int NTHREADS = 256;

template <int DK, int DV, bool QBF, bool GBF, bool OBF, bool GL, bool OG>
__global__ void __launch_bounds__(NTHREADS)
kda_decode_kernel(const typename Store<QBF>::type *__restrict__ q,
                  const typename Store<QBF>::type *__restrict__ k,
                  const typename Store<QBF>::type *__restrict__ v,
                  const typename Store<GBF>::type *__restrict__ g,
                  const typename Store<GBF>::type *__restrict__ beta,
                  float *__restrict__ S, typename Store<OBF>::type *__restrict__ o,
                  const float *__restrict__ A_log, int H,
                  const typename Store<QBF>::type *__restrict__ z_out, const float *__restrict__ weight, float eps)
{
    typedef typename Store<QBF>::type QT;
    typedef typename Store<OBF>::type OT;
    constexpr int NCG = DV / 4;            // column groups of 4
    constexpr int NRG = NTHREADS / NCG;    // row groups
    constexpr int RPT = DK / NRG;          // rows per thread
    static_assert(RPT * NRG == DK, "rows must split evenly");

    __shared__ float s_ak[DK], s_aq[DK], s_k[DK], s_q[DK], s_alpha[DK];
    __shared__ f32x4 s_p[NRG][NCG], s_r[NRG][NCG];
    __shared__ float s_qk[NRG];

    const int bh = xcd_contiguous(blockIdx.x, gridDim.x);   // one state per workgroup
    const int cg = threadIdx.x % NCG;
    const int rg = threadIdx.x / NCG;
    f32x4 *Sp = reinterpret_cast<f32x4 *>(S + (size_t)bh * DK * DV);

    // issue the whole state slice first: it is the only large transfer
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(&Sp[(rg + NRG * i) * NCG + cg]);

    if (threadIdx.x < DK) {
        const int c = threadIdx.x;
        float gc = to_f32(g[(size_t)bh * DK + c]);
        if constexpr (GL) gc = gate_from_logit(gc, __expf(A_log[bh % H]));
        const float alpha = __expf(gc);
        const float kc = to_f32(k[(size_t)bh * DK + c]);
        const float qc = to_f32(q[(size_t)bh * DK + c]);
        s_alpha[c] = alpha;
        s_k[c] = kc;
        s_q[c] = qc;
        s_ak[c] = alpha * kc;
        s_aq[c] = alpha * qc;
    }
    const float bt = to_f32(beta[bh]);
    float vv[4];
    {
        const QT *vp = v + (size_t)bh * DV + 4 * cg;
#pragma unroll
        for (int c = 0; c < 4; ++c) vv[c] = to_f32(vp[c]);
    }
    float zo[4], wo[4];
    if constexpr (OG) {
        Raw4<QT> rz;
        rz.load(z_out + (size_t)bh * DV + 4 * cg);
        rz.to_f32(zo);
        const float4 t = *reinterpret_cast<const float4 *>(weight + 4 * cg);
        wo[0] = t.x; wo[1] = t.y; wo[2] = t.z; wo[3] = t.w;
    }
    lds_barrier();

    f32x4 p = {0.f, 0.f, 0.f, 0.f}, rd = {0.f, 0.f, 0.f, 0.f};
    float qk = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + NRG * i;
        const float ak = s_ak[row], aq = s_aq[row];
        p += s[i] * ak;
        rd += s[i] * aq;
        if (cg == 0) qk += s_q[row] * s_k[row];   // q.k over this thread's rows
    }
    s_p[rg][cg] = p;
    s_r[rg][cg] = rd;
    if (cg == 0) s_qk[rg] = qk;
    lds_barrier();

    f32x4 pt = {0.f, 0.f, 0.f, 0.f}, rt = {0.f, 0.f, 0.f, 0.f};
    float qkt = 0.f;
#pragma unroll
    for (int x = 0; x < NRG; ++x) {
        pt += s_p[x][cg];
        rt += s_r[x][cg];
        qkt += s_qk[x];
    }
    f32x4 w;
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = bt * (vv[c] - pt[c]);
    if constexpr (OG) {
        // every row group holds the full outputs; reduce over one group's lanes
        float oc[4], ss = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            oc[c] = rt[c] + qkt * w[c];
            ss += oc[c] * oc[c];
        }
#pragma unroll
        for (int m = 1; m < NCG; m <<= 1) ss += __shfl_xor(ss, m, NCG);
        const float inv = rsqrtf(ss * (1.f / DV) + eps);
        if (rg == 0) {
            float yv[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) yv[c] = oc[c] * inv * wo[c] * sigmoid_f32(zo[c]);
            store4(o + (size_t)bh * DV + 4 * cg, yv);
        }
    } else if (rg == 0) {
        OT *op = o + (size_t)bh * DV + 4 * cg;
#pragma unroll
        for (int c = 0; c < 4; ++c) op[c] = from_f32<OT>(rt[c] + qkt * w[c]);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + NRG * i;
        const float a = s_alpha[row], kc = s_k[row];
        const f32x4 ns = a * s[i] + kc * w;
        __builtin_nontemporal_store(ns, &Sp[row * NCG + cg]);
    }
}

template <int DK, int DV, bool QBF, bool GBF, bool OBF, bool GL, bool OG>
hipError_t launch(const DecodeArgs &a, hipStream_t stream)
{
    typedef typename Store<QBF>::type QT;
    typedef typename Store<GBF>::type GT;
    typedef typename Store<OBF>::type OT;
    kda_decode_kernel<DK, DV, QBF, GBF, OBF, GL, OG><<<(unsigned)(a.B * a.H), NTHREADS, 0, stream>>>(
        (const QT *)a.q, (const QT *)a.k, (const QT *)a.v, (const GT *)a.g, (const GT *)a.beta,
        a.S, (OT *)a.o, a.A_log, a.H, (const QT *)a.z_out, a.weight, a.eps);
    return hipGetLastError();
}

template <int DK, int DV, bool QBF, bool GBF, bool OBF, bool GL>
hipError_t dispatch_epilogue(const DecodeArgs &a, hipStream_t s)
{
    return a.z_out ? launch<DK, DV, QBF, GBF, OBF, GL, true>(a, s) : launch<DK, DV, QBF, GBF, OBF, GL, false>(a, s);
}

template <int DK, int DV, bool QBF, bool GBF, bool GL>
hipError_t dispatch_gate(const DecodeArgs &a, hipStream_t s)
{
    return a.out_bf16 ? dispatch_epilogue<DK, DV, QBF, GBF, true, GL>(a, s)
                      : dispatch_epilogue<DK, DV, QBF, GBF, false, GL>(a, s);
}

template <int DK, int DV, bool QBF, bool GBF>
hipError_t dispatch_out(const DecodeArgs &a, hipStream_t s)
{
    return a.A_log ? dispatch_gate<DK, DV, QBF, GBF, true>(a, s) : dispatch_gate<DK, DV, QBF, GBF, false>(a, s);
}

template <int DK, int DV>
hipError_t dispatch_dtypes(const DecodeArgs &a, hipStream_t s)
{
    if (a.qkv_bf16)
        return a.gate_bf16 ? dispatch_out<DK, DV, true, true>(a, s) : dispatch_out<DK, DV, true, false>(a, s);
    return a.gate_bf16 ? dispatch_out<DK, DV, false, true>(a, s) : dispatch_out<DK, DV, false, false>(a, s);
}

}  // namespace

hipError_t launch_decode_step(const DecodeArgs &a, hipStream_t stream)
{
    (void)hipGetLastError();
    if (a.dk == 64) return a.dv == 64 ? dispatch_dtypes<64, 64>(a, stream) : dispatch_dtypes<64, 128>(a, stream);
    return a.dv == 64 ? dispatch_dtypes<128, 64>(a, stream) : dispatch_dtypes<128, 128>(a, stream);
}

}  // namespace kda
