// C ABI of libkda.so: host-side validation, then one kernel launch on the
// caller's stream.  Declarations and the full contract are in include/kda.h.
#include "../../include/kda.h"
#include "kda_internal.h"

#include <stdint.h>

namespace {

bool valid_dtype(kda_dtype_t d) { return d == KDA_F32 || d == KDA_BF16; }
size_t dsize(kda_dtype_t d) { return d == KDA_BF16 ? 2 : 4; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

struct Span {
    uintptr_t lo, hi;   // [lo, hi)
};
Span span(const void *p, size_t bytes) { return Span{(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

}  // namespace

namespace {

// Host-side checks shared by every chunked entry point.  `o` and `q` may be
// absent only where the caller says so (commit writes no output and reads no
// query).  Returns KDA_OK when the launch may proceed.
kda_status_t check_chunk(const void *q, const void *k, const void *v, const void *g, const void *beta,
                         const float *S0, const void *o, const float *S_final, const float *A_log,
                         const int *lengths, int B, int T, int H, int dk, int dv,
                         kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                         bool need_q, bool need_o)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
    if (!valid_dtype(qkv_dtype) || !valid_dtype(gate_dtype) || !valid_dtype(out_dtype))
        return KDA_ERR_INVALID_ARG;
    if (dk != 64 && dk != 128) return KDA_ERR_UNSUPPORTED;
    if (dv % 64 != 0 || dv > 512) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)B * T >= ((int64_t)1 << 31) || (int64_t)B * H * (dv / 64) >= ((int64_t)1 << 31))
        return KDA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return KDA_OK;

    const size_t tok = (size_t)B * T * H;
    const size_t sq = dsize(qkv_dtype), sg = dsize(gate_dtype), so = dsize(out_dtype);
    const Span sp_q = span(need_q ? q : nullptr, need_q ? tok * dk * sq : 0), sp_k = span(k, tok * dk * sq);
    const Span sp_v = span(v, tok * dv * sq), sp_o = span(need_o ? o : nullptr, need_o ? tok * dv * so : 0);
    const Span sp_g = span(g, tok * dk * sg), sp_b = span(beta, tok * sg);
    const Span sp_a = span(A_log, A_log ? (size_t)H * sizeof(float) : 0);
    const Span sp_l = span(lengths, lengths ? (size_t)B * sizeof(int) : 0);
    const size_t state_bytes = (size_t)B * H * dk * dv * sizeof(float);
    const Span sp_s0 = span(S0, S0 ? state_bytes : 0), sp_sf = span(S_final, S_final ? state_bytes : 0);

    if (T > 0) {
        if ((need_q && !q) || !k || !v || !g || !beta || (need_o && !o)) return KDA_ERR_INVALID_ARG;
        if ((need_q && !aligned16(q)) || !aligned16(k) || !aligned16(v) || !aligned16(g) || (need_o && !aligned16(o)))
            return KDA_ERR_INVALID_ARG;
        if (need_o) {
            const Span ins[] = {sp_q, sp_k, sp_v, sp_g, sp_b, sp_s0, sp_sf, sp_a, sp_l};
            for (const Span &s : ins)
                if (overlap(sp_o, s)) return KDA_ERR_INVALID_ARG;
        }
    }
    if ((S0 && !aligned16(S0)) || (S_final && !aligned16(S_final))) return KDA_ERR_INVALID_ARG;
    if ((A_log && ((uintptr_t)A_log & 3u)) || (lengths && ((uintptr_t)lengths & 3u))) return KDA_ERR_INVALID_ARG;
    if (S_final) {
        const Span ins[] = {sp_q, sp_k, sp_v, sp_g, sp_b, sp_a, sp_l};
        if (T > 0)
            for (const Span &s : ins)
                if (overlap(sp_sf, s)) return KDA_ERR_INVALID_ARG;
        if (S0 && S0 != S_final && overlap(sp_sf, sp_s0)) return KDA_ERR_INVALID_ARG;
    }
    return KDA_OK;
}

kda_status_t run_chunk(kda::ChunkFwdArgs &a, void *stream)
{
    if (a.B == 0 || a.H == 0) return KDA_OK;
    if (a.T == 0 && !a.S_final) return KDA_OK;
    return kda::launch_chunk_fwd(a, (hipStream_t)stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda::ChunkFwdArgs chunk_args(const void *q, const void *k, const void *v, const void *g, const void *beta,
                             const float *S0, void *o, float *S_final, int B, int T, int H, int dk, int dv,
                             kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype)
{
    kda::ChunkFwdArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.S0 = S0; a.o = o; a.S_final = S_final;
    a.B = B; a.T = T; a.H = H; a.dk = dk; a.dv = dv;
    a.qkv_bf16 = qkv_dtype == KDA_BF16;
    a.gate_bf16 = gate_dtype == KDA_BF16;
    a.out_bf16 = out_dtype == KDA_BF16;
    return a;
}

// kda_chunk_fwd / kda_chunk_fwd_gate with a workspace: the prep/state kernel
// where it applies, otherwise (or with no workspace) the same kernels as
// without one.
kda_status_t chunk_ws(const void *q, const void *k, const void *v, const void *g, const float *A_log,
                      const void *beta, const float *S0, void *o, float *S_final, void *workspace,
                      size_t workspace_bytes, int B, int T, int H, int dk, int dv,
                      kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype, void *stream)
{
    const kda_status_t st = check_chunk(q, k, v, g, beta, S0, o, S_final, A_log, nullptr, B, T, H, dk, dv,
                                        qkv_dtype, gate_dtype, out_dtype, true, true);
    if (st != KDA_OK) return st;
    if (B == 0 || H == 0) return KDA_OK;
    const size_t need = kda::chunk_ps_workspace_bytes(B, H, dk, dv);
    if (workspace && T > 0) {
        if (!aligned16(workspace) || workspace_bytes < need) return KDA_ERR_INVALID_ARG;
        const size_t tok = (size_t)B * T * H;
        const size_t sq = dsize(qkv_dtype), sg = dsize(gate_dtype), so = dsize(out_dtype);
        const size_t state_bytes = (size_t)B * H * dk * dv * sizeof(float);
        const Span sp_w = span(workspace, workspace_bytes);
        const Span others[] = {span(q, tok * dk * sq), span(k, tok * dk * sq), span(v, tok * dv * sq),
                               span(g, tok * dk * sg), span(beta, tok * sg), span(o, tok * dv * so),
                               span(S0, S0 ? state_bytes : 0), span(S_final, S_final ? state_bytes : 0),
                               span(A_log, A_log ? (size_t)H * sizeof(float) : 0)};
        for (const Span &x : others)
            if (overlap(sp_w, x)) return KDA_ERR_INVALID_ARG;
    }
    kda::ChunkFwdArgs a = chunk_args(q, k, v, g, beta, S0, o, S_final, B, T, H, dk, dv,
                                     qkv_dtype, gate_dtype, out_dtype);
    a.A_log = A_log;
    if (workspace && T > 0) {
        bool used = false;
        const hipError_t e = kda::launch_chunk_fwd_ps(a, workspace, workspace_bytes, (hipStream_t)stream, used);
        if (used) return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
    }
    return run_chunk(a, stream);
}

kda::SpecArgs spec_args(const void *q, const void *k, const void *v, const void *g, const void *beta,
                        float *S, int B, int K, int H, int dk, int dv,
                        kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype)
{
    kda::SpecArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S = S;
    a.B = B; a.K = K; a.H = H; a.dk = dk; a.dv = dv;
    a.qkv_bf16 = qkv_dtype == KDA_BF16;
    a.gate_bf16 = gate_dtype == KDA_BF16;
    a.out_bf16 = out_dtype == KDA_BF16;
    return a;
}

// Checks of the output epilogue's own arguments: z_out [n, dv] (storage
// `z_bytes` per value), weight [dv] float32, eps >= 0 and finite.
bool epilogue_args_ok(const void *z_out, const float *weight, float eps)
{
    if (!z_out || !weight) return false;
    if (!aligned16(weight)) return false;
    return eps >= 0.f && eps <= 3.0e38f;   // rejects NaN and inf too
}

kda_status_t decode(const void *q, const void *k, const void *v, const void *g, const void *beta,
                    const float *A_log, float *S, void *o, int B, int H, int dk, int dv,
                    kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype, void *stream,
                    const void *z_out = nullptr, const float *weight = nullptr, float eps = 0.f,
                    bool gated = false)
{
    if (B < 0 || H < 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
    if (!valid_dtype(qkv_dtype) || !valid_dtype(gate_dtype) || !valid_dtype(out_dtype))
        return KDA_ERR_INVALID_ARG;
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)B * H >= ((int64_t)1 << 31)) return KDA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !S || !o) return KDA_ERR_INVALID_ARG;
    if (!aligned16(S)) return KDA_ERR_INVALID_ARG;
    if (A_log && ((uintptr_t)A_log & 3u)) return KDA_ERR_INVALID_ARG;
    // the fused epilogue stores y with 8- or 16-byte vector stores
    if (gated && (!epilogue_args_ok(z_out, weight, eps) || !aligned16(z_out) || !aligned16(o)))
        return KDA_ERR_INVALID_ARG;

    const size_t n = (size_t)B * H;
    const size_t sq = dsize(qkv_dtype), sg = dsize(gate_dtype), so = dsize(out_dtype);
    const Span sp_q = span(q, n * dk * sq), sp_k = span(k, n * dk * sq), sp_v = span(v, n * dv * sq);
    const Span sp_g = span(g, n * dk * sg), sp_b = span(beta, n * sg);
    const Span sp_a = span(A_log, A_log ? (size_t)H * sizeof(float) : 0);
    const Span sp_s = span(S, n * dk * dv * sizeof(float)), sp_o = span(o, n * dv * so);
    const Span sp_z = span(gated ? z_out : nullptr, gated ? n * dv * sq : 0);
    const Span sp_w = span(gated ? weight : nullptr, gated ? (size_t)dv * sizeof(float) : 0);
    const Span ins[] = {sp_q, sp_k, sp_v, sp_g, sp_b, sp_a, sp_z, sp_w};
    for (const Span &s : ins)
        if (overlap(sp_o, s) || overlap(sp_s, s)) return KDA_ERR_INVALID_ARG;
    if (overlap(sp_o, sp_s)) return KDA_ERR_INVALID_ARG;

    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S = S; a.o = o; a.A_log = A_log;
    if (gated) {
        a.z_out = z_out; a.weight = weight; a.eps = eps;
    }
    a.B = B; a.H = H; a.dk = dk; a.dv = dv;
    a.qkv_bf16 = qkv_dtype == KDA_BF16;
    a.gate_bf16 = gate_dtype == KDA_BF16;
    a.out_bf16 = out_dtype == KDA_BF16;
    return kda::launch_decode_step(a, (hipStream_t)stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v, const void *g,
                           const void *beta, const float *S0, void *o, float *S_final,
                           int B, int T, int H, int dk, int dv,
                           kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                           void *stream)
{
    const kda_status_t st = check_chunk(q, k, v, g, beta, S0, o, S_final, nullptr, nullptr, B, T, H, dk, dv,
                                        qkv_dtype, gate_dtype, out_dtype, true, true);
    if (st != KDA_OK) return st;
    kda::ChunkFwdArgs a = chunk_args(q, k, v, g, beta, S0, o, S_final, B, T, H, dk, dv,
                                     qkv_dtype, gate_dtype, out_dtype);
    return run_chunk(a, stream);
}

kda_status_t kda_chunk_fwd_gate(const void *q, const void *k, const void *v, const void *z,
                                const float *A_log, const void *beta, const float *S0, void *o,
                                float *S_final, int B, int T, int H, int dk, int dv,
                                kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                                void *stream)
{
    if (!A_log && B > 0 && H > 0) return KDA_ERR_INVALID_ARG;
    const kda_status_t st = check_chunk(q, k, v, z, beta, S0, o, S_final, A_log, nullptr, B, T, H, dk, dv,
                                        qkv_dtype, gate_dtype, out_dtype, true, true);
    if (st != KDA_OK) return st;
    kda::ChunkFwdArgs a = chunk_args(q, k, v, z, beta, S0, o, S_final, B, T, H, dk, dv,
                                     qkv_dtype, gate_dtype, out_dtype);
    a.A_log = A_log;
    return run_chunk(a, stream);
}

kda_status_t kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, const float *S0, void *o, float *S_final,
                                   int B, int T, int H, int dk, int dv,
                                   kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                                   void *stream)
{
    const kda_status_t st = check_chunk(q, k, v, g, beta, S0, o, S_final, nullptr, nullptr, B, T, H, dk, dv,
                                        qkv_dtype, gate_dtype, out_dtype, true, true);
    if (st != KDA_OK) return st;
    if (B == 0 || H == 0) return KDA_OK;
    kda::ChunkFwdArgs a = chunk_args(q, k, v, g, beta, S0, o, S_final, B, T, H, dk, dv,
                                     qkv_dtype, gate_dtype, out_dtype);
    const size_t need = T > 0 && qkv_dtype == KDA_BF16 ? kda::chunk_ps_workspace_bytes(B, H, dk, dv) : 0;
    if (need > 0) {
        // the ring kernel applies: its ring goes into the library's own scratch
        if (need > kda::noalloc_scratch_bytes()) return KDA_ERR_SCRATCH;
        void *ws = nullptr;
        if (kda::noalloc_scratch((hipStream_t)stream, &ws) != hipSuccess) return KDA_ERR_LAUNCH;
        bool used = false;
        const hipError_t e = kda::launch_chunk_fwd_ps(a, ws, kda::noalloc_scratch_bytes(), (hipStream_t)stream, used);
        if (used) return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
    }
    return run_chunk(a, stream);
}

size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv)
{
    if (T <= 0) return 0;
    return kda::chunk_ps_workspace_bytes(B, H, dk, dv);
}

kda_status_t kda_chunk_fwd_ws(const void *q, const void *k, const void *v, const void *g,
                              const void *beta, const float *S0, void *o, float *S_final,
                              void *workspace, size_t workspace_bytes,
                              int B, int T, int H, int dk, int dv,
                              kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                              void *stream)
{
    return chunk_ws(q, k, v, g, nullptr, beta, S0, o, S_final, workspace, workspace_bytes, B, T, H, dk, dv,
                    qkv_dtype, gate_dtype, out_dtype, stream);
}

kda_status_t kda_chunk_fwd_gate_ws(const void *q, const void *k, const void *v, const void *z,
                                   const float *A_log, const void *beta, const float *S0, void *o,
                                   float *S_final, void *workspace, size_t workspace_bytes,
                                   int B, int T, int H, int dk, int dv,
                                   kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                                   void *stream)
{
    if (!A_log && B > 0 && H > 0) return KDA_ERR_INVALID_ARG;
    return chunk_ws(q, k, v, z, A_log, beta, S0, o, S_final, workspace, workspace_bytes, B, T, H, dk, dv,
                    qkv_dtype, gate_dtype, out_dtype, stream);
}

size_t kda_chunk_fwd_seqpar_workspace_bytes(int B, int T, int H, int dk, int dv, int segments)
{
    if (B <= 0 || T <= 0 || H <= 0 || segments < 1 || segments > KDA_SEQPAR_MAX_SEGMENTS || T % segments) return 0;
    if ((dk != 64 && dk != 128) || dv % 64 || dv <= 0 || dv > 512) return 0;
    return kda::chunk_seqpar_workspace_bytes(B, H, dk, dv, segments);
}

int kda_chunk_fwd_seqpar_segments(int B, int T, int H, int dk, int dv, int cus)
{
    if (B <= 0 || T <= 0 || H <= 0 || (dk != 64 && dk != 128) || dv % 64 || dv <= 0 || dv > 512) return 1;
    if (cus <= 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return 1;
    }
    // Estimated call time in microseconds, from kernel traces on MI355X: a
    // pass of the pipelined kernel over n chunks of 64 tokens takes about
    // (n + 1) x 5 us per round of workgroups (one workgroup per CU; the extra
    // period is the producers' head start) plus 3 us; the combine about
    // 6 + 1.9 P us; the three launches of the sequence-parallel call about
    // 10 us more than one.  (The sequence-parallel first pass, which skips the
    // query side, runs nearer 4.1 us per period; counting it so tips near
    // ties the wrong way on the shapes measured, so both passes count 5.)
    const auto chunks = [](int t) { return (int64_t)(t + 63) / 64; };
    const auto pass = [cus](int64_t workgroups, int64_t n) {
        return (double)((workgroups + cus - 1) / cus) * (double)(n + 1) * 5.0 + 3.0;
    };
    const int64_t heads = (int64_t)B * H;
    double best = pass(heads * (dv / 64), chunks(T));
    int pick = 1;
    for (int P = 2; P <= KDA_SEQPAR_MAX_SEGMENTS && P <= T; ++P) {
        if (T % P) continue;
        const int64_t n = chunks(T / P);
        const double est = pass(heads * P * (dv / 64 + dk / 64), n) + 6.0 + 1.9 * P + pass(heads * P * (dv / 64), n) + 10.0;
        if (est < best) { best = est; pick = P; }
    }
    return pick;
}

namespace {
// kda_chunk_fwd_seqpar and kda_chunk_fwd_gate_seqpar (gate logits with A_log)
kda_status_t run_seqpar(const void *q, const void *k, const void *v, const void *g, const float *A_log,
                        const void *beta, const float *S0, void *o, float *S_final, void *workspace,
                        size_t workspace_bytes, int B, int T, int H, int dk, int dv, int segments,
                        kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype, void *stream)
{
    const kda_status_t st = check_chunk(q, k, v, g, beta, S0, o, S_final, A_log, nullptr, B, T, H, dk, dv,
                                        qkv_dtype, gate_dtype, out_dtype, true, true);
    if (st != KDA_OK) return st;
    if (segments < 1 || segments > KDA_SEQPAR_MAX_SEGMENTS || (T > 0 && T % segments)) return KDA_ERR_INVALID_ARG;
    if (qkv_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)B * segments * H * (dv / 64 + dk / 64) >= ((int64_t)1 << 31)) return KDA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return KDA_OK;
    kda::ChunkFwdArgs a = chunk_args(q, k, v, g, beta, S0, o, S_final, B, T, H, dk, dv,
                                     qkv_dtype, gate_dtype, out_dtype);
    a.A_log = A_log;
    if (T == 0) return run_chunk(a, stream);
    const size_t need = kda::chunk_seqpar_workspace_bytes(B, H, dk, dv, segments);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need) return KDA_ERR_INVALID_ARG;
    {
        const size_t tok = (size_t)B * T * H;
        const size_t sq = dsize(qkv_dtype), sg = dsize(gate_dtype), so = dsize(out_dtype);
        const size_t state_bytes = (size_t)B * H * dk * dv * sizeof(float);
        const Span sp_w = span(workspace, workspace_bytes);
        const Span others[] = {span(q, tok * dk * sq), span(k, tok * dk * sq), span(v, tok * dv * sq),
                               span(g, tok * dk * sg), span(beta, tok * sg), span(o, tok * dv * so),
                               span(S0, S0 ? state_bytes : 0), span(S_final, S_final ? state_bytes : 0),
                               span(A_log, A_log ? (size_t)H * sizeof(float) : 0)};
        for (const Span &x : others)
            if (overlap(sp_w, x)) return KDA_ERR_INVALID_ARG;
    }
    // the final state is written by the combine step, which reads S0 first:
    // S_final may alias S0 as in kda_chunk_fwd
    return kda::launch_chunk_fwd_seqpar(a, segments, workspace, (hipStream_t)stream) == hipSuccess ? KDA_OK
                                                                                          : KDA_ERR_LAUNCH;
}
}  // namespace

kda_status_t kda_chunk_fwd_seqpar(const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, const float *S0, void *o, float *S_final,
                                  void *workspace, size_t workspace_bytes,
                                  int B, int T, int H, int dk, int dv, int segments,
                                  kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                                  void *stream)
{
    return run_seqpar(q, k, v, g, nullptr, beta, S0, o, S_final, workspace, workspace_bytes, B, T, H, dk, dv,
                      segments, qkv_dtype, gate_dtype, out_dtype, stream);
}

kda_status_t kda_chunk_fwd_gate_seqpar(const void *q, const void *k, const void *v, const void *z,
                                       const float *A_log, const void *beta, const float *S0, void *o,
                                       float *S_final, void *workspace, size_t workspace_bytes,
                                       int B, int T, int H, int dk, int dv, int segments,
                                       kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                                       void *stream)
{
    if (!A_log && B > 0 && H > 0) return KDA_ERR_INVALID_ARG;
    return run_seqpar(q, k, v, z, A_log, beta, S0, o, S_final, workspace, workspace_bytes, B, T, H, dk, dv,
                      segments, qkv_dtype, gate_dtype, out_dtype, stream);
}

unsigned kda_debug_set_spin_limit(unsigned limit) { return kda::set_spin_limit(limit); }

kda_status_t kda_verify_step(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, const float *S, void *o,
                             int B, int K, int H, int dk, int dv,
                             kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                             void *stream)
{
    if (!S && B > 0 && H > 0) return KDA_ERR_INVALID_ARG;
    const kda_status_t st = check_chunk(q, k, v, g, beta, S, o, nullptr, nullptr, nullptr, B, K, H, dk, dv,
                                        qkv_dtype, gate_dtype, out_dtype, true, true);
    if (st != KDA_OK) return st;
    if (K == 0 || B == 0 || H == 0) return KDA_OK;
    if ((dk == 64 || dk == 128) && (dv == 64 || dv == 128)) {   // one workgroup per state
        kda::SpecArgs a = spec_args(q, k, v, g, beta, const_cast<float *>(S), B, K, H, dk, dv,
                                    qkv_dtype, gate_dtype, out_dtype);
        a.o = o;
        // up to 16 drafts: one tile on the matrix cores; more: the token loop
        const hipError_t e = K <= 16 ? kda::launch_verify_tile(a, (hipStream_t)stream)
                                     : kda::launch_spec_step(a, (hipStream_t)stream);
        return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
    }
    kda::ChunkFwdArgs a = chunk_args(q, k, v, g, beta, S, o, nullptr, B, K, H, dk, dv,
                                     qkv_dtype, gate_dtype, out_dtype);
    return run_chunk(a, stream);
}

kda_status_t kda_commit_step(const void *k, const void *v, const void *g, const void *beta,
                             const int *accepted, float *S, int B, int K, int H, int dk, int dv,
                             kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, void *stream)
{
    if ((!S || !accepted) && B > 0 && H > 0) return KDA_ERR_INVALID_ARG;
    const kda_status_t st = check_chunk(nullptr, k, v, g, beta, S, nullptr, S, nullptr, accepted, B, K, H,
                                        dk, dv, qkv_dtype, gate_dtype, KDA_F32, false, false);
    if (st != KDA_OK) return st;
    if (K == 0 || B == 0 || H == 0) return KDA_OK;
    if ((dk == 64 || dk == 128) && (dv == 64 || dv == 128)) {   // one workgroup per state
        kda::SpecArgs a = spec_args(nullptr, k, v, g, beta, S, B, K, H, dk, dv, qkv_dtype, gate_dtype, KDA_F32);
        a.accepted = accepted;
        // up to 16 drafts: one tile on the matrix cores; more: the token loop
        const hipError_t e = K <= 16 ? kda::launch_verify_tile(a, (hipStream_t)stream)
                                     : kda::launch_spec_step(a, (hipStream_t)stream);
        return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
    }
    // the chunk kernels read a query row for every token; the keys stand in (no output is written)
    kda::ChunkFwdArgs a = chunk_args(k, k, v, g, beta, S, nullptr, S, B, K, H, dk, dv,
                                     qkv_dtype, gate_dtype, KDA_F32);
    a.lengths = accepted;
    return run_chunk(a, stream);
}

kda_status_t kda_decode_step(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, float *S, void *o, int B, int H, int dk, int dv,
                             kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                             void *stream)
{
    return decode(q, k, v, g, beta, nullptr, S, o, B, H, dk, dv, qkv_dtype, gate_dtype, out_dtype, stream);
}

kda_status_t kda_decode_step_gate(const void *q, const void *k, const void *v, const void *z,
                                  const float *A_log, const void *beta, float *S, void *o,
                                  int B, int H, int dk, int dv,
                                  kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                                  void *stream)
{
    if (!A_log && B > 0 && H > 0) return KDA_ERR_INVALID_ARG;
    return decode(q, k, v, z, beta, A_log, S, o, B, H, dk, dv, qkv_dtype, gate_dtype, out_dtype, stream);
}

kda_status_t kda_decode_step_gated(const void *q, const void *k, const void *v, const void *g,
                                   const float *A_log, const void *beta, float *S, const void *z_out,
                                   const float *weight, float eps, void *y, int B, int H, int dk, int dv,
                                   kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                                   void *stream)
{
    return decode(q, k, v, g, beta, A_log, S, y, B, H, dk, dv, qkv_dtype, gate_dtype, out_dtype, stream,
                  z_out, weight, eps, true);
}

kda_status_t kda_output_gate(const void *o, const void *z, const float *weight, float eps, void *y,
                             int64_t rows, int dv, kda_dtype_t o_dtype, kda_dtype_t z_dtype,
                             kda_dtype_t y_dtype, void *stream)
{
    if (rows < 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
    if (!valid_dtype(o_dtype) || !valid_dtype(z_dtype) || !valid_dtype(y_dtype)) return KDA_ERR_INVALID_ARG;
    if (dv % 64 != 0 || dv > 512) return KDA_ERR_UNSUPPORTED;
    if (rows > ((int64_t)1 << 40)) return KDA_ERR_UNSUPPORTED;
    if (rows == 0) return KDA_OK;
    if (!o || !y || !epilogue_args_ok(z, weight, eps)) return KDA_ERR_INVALID_ARG;
    if (!aligned16(o) || !aligned16(z) || !aligned16(y)) return KDA_ERR_INVALID_ARG;
    const size_t n = (size_t)rows * dv;
    const Span sp_o = span(o, n * dsize(o_dtype)), sp_z = span(z, n * dsize(z_dtype));
    const Span sp_w = span(weight, (size_t)dv * sizeof(float)), sp_y = span(y, n * dsize(y_dtype));
    // y may be o itself (same dtype): each element is read before it is written
    const bool in_place = y == o && y_dtype == o_dtype;
    if ((!in_place && overlap(sp_y, sp_o)) || overlap(sp_y, sp_z) || overlap(sp_y, sp_w)) return KDA_ERR_INVALID_ARG;

    kda::OutputGateArgs a;
    a.o = o; a.z = z; a.weight = weight; a.y = y;
    a.rows = rows; a.dv = dv; a.eps = eps;
    a.o_bf16 = o_dtype == KDA_BF16;
    a.z_bf16 = z_dtype == KDA_BF16;
    a.y_bf16 = y_dtype == KDA_BF16;
    return kda::launch_output_gate(a, (hipStream_t)stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv)
{
    if (B <= 0 || T <= 0 || H <= 0 || (dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return 0;
    return kda::chunk_bwd_workspace_floats(B, T, H, dk, dv) * sizeof(float);
}

kda_status_t kda_chunk_bwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                           const float *S0, const void *dO, const float *dS_final,
                           float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dS0,
                           void *workspace, size_t workspace_bytes,
                           int B, int T, int H, int dk_dim, int dv_dim,
                           kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t do_dtype, void *stream)
{
    if (B < 0 || T < 0 || H < 0 || dk_dim <= 0 || dv_dim <= 0) return KDA_ERR_INVALID_ARG;
    if (!valid_dtype(qkv_dtype) || !valid_dtype(gate_dtype) || !valid_dtype(do_dtype)) return KDA_ERR_INVALID_ARG;
    if ((dk_dim != 64 && dk_dim != 128) || (dv_dim != 64 && dv_dim != 128)) return KDA_ERR_UNSUPPORTED;
    const int64_t nc = ((int64_t)T + 31) / 32;
    if ((int64_t)B * T >= ((int64_t)1 << 31) || (int64_t)B * H * nc >= ((int64_t)1 << 31)) return KDA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return KDA_OK;

    const size_t tok = (size_t)B * T * H, st = (size_t)B * H * dk_dim * dv_dim * sizeof(float);
    const size_t sq = dsize(qkv_dtype), sg = dsize(gate_dtype), so = dsize(do_dtype);
    const size_t need = kda_chunk_bwd_workspace_bytes(B, T, H, dk_dim, dv_dim);
    if (T > 0) {
        const void *req[] = {q, k, v, g, beta, dO, dq, dk, dv, dg, dbeta};
        for (const void *p : req)
            if (!p || !aligned16(p)) return KDA_ERR_INVALID_ARG;
        if (!workspace || !aligned16(workspace) || workspace_bytes < need) return KDA_ERR_INVALID_ARG;
    }
    if ((S0 && !aligned16(S0)) || (dS_final && !aligned16(dS_final)) || (dS0 && !aligned16(dS0)))
        return KDA_ERR_INVALID_ARG;
    const bool run = T > 0;
    const Span ins[] = {span(run ? q : nullptr, run ? tok * dk_dim * sq : 0), span(run ? k : nullptr, run ? tok * dk_dim * sq : 0),
                        span(run ? v : nullptr, run ? tok * dv_dim * sq : 0), span(run ? g : nullptr, run ? tok * dk_dim * sg : 0),
                        span(run ? beta : nullptr, run ? tok * sg : 0), span(run ? dO : nullptr, run ? tok * dv_dim * so : 0),
                        span(S0, S0 ? st : 0), span(dS_final, dS_final ? st : 0)};
    const Span outs[] = {span(run ? dq : nullptr, run ? tok * dk_dim * 4 : 0), span(run ? dk : nullptr, run ? tok * dk_dim * 4 : 0),
                         span(run ? dv : nullptr, run ? tok * dv_dim * 4 : 0), span(run ? dg : nullptr, run ? tok * dk_dim * 4 : 0),
                         span(run ? dbeta : nullptr, run ? tok * 4 : 0), span(dS0, dS0 ? st : 0),
                         span(run ? workspace : nullptr, run ? need : 0)};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Span &s : ins)
            if (overlap(outs[i], s)) return KDA_ERR_INVALID_ARG;
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (overlap(outs[i], outs[j])) return KDA_ERR_INVALID_ARG;
    }
    if (T == 0 && !dS0) return KDA_OK;

    kda::ChunkBwdArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S0 = S0; a.dO = dO; a.dS_final = dS_final;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dS0 = dS0;
    a.ws = kda::chunk_bwd_workspace(run ? (float *)workspace : nullptr, B, T, H, dk_dim, dv_dim);
    a.B = B; a.T = T; a.H = H; a.dk_dim = dk_dim; a.dv_dim = dv_dim;
    a.qkv_bf16 = qkv_dtype == KDA_BF16;
    a.gate_bf16 = gate_dtype == KDA_BF16;
    a.do_bf16 = do_dtype == KDA_BF16;
    return kda::launch_chunk_bwd(a, (hipStream_t)stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

const char *kda_status_string(kda_status_t status)
{
    switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: null, misaligned or overlapping pointer, bad size or dtype";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: dk/dv combination not provided";
    case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH: the HIP runtime rejected the kernel launch";
    case KDA_ERR_SCRATCH: return "KDA_ERR_SCRATCH: the input needs more scratch than kda_chunk_fwd_noalloc holds";
    default: break;
    }
    return "KDA_ERR_UNKNOWN";
}

int kda_abi_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
