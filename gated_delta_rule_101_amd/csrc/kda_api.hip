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

extern "C" {

kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v, const void *g,
                           const void *beta, const float *S0, void *o, float *S_final,
                           int B, int T, int H, int dk, int dv,
                           kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                           void *stream)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
    if (!valid_dtype(qkv_dtype) || !valid_dtype(gate_dtype) || !valid_dtype(out_dtype))
        return KDA_ERR_INVALID_ARG;
    if (dk != 64 && dk != 128) return KDA_ERR_UNSUPPORTED;
    if (dv % 64 != 0 || dv > 512) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)B * T >= ((int64_t)1 << 31) || (int64_t)B * H * (dv / 64) >= ((int64_t)1 << 31))
        return KDA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return KDA_OK;   // nothing to compute

    const size_t tok = (size_t)B * T * H;
    const size_t sq = dsize(qkv_dtype), sg = dsize(gate_dtype), so = dsize(out_dtype);
    const Span sp_q = span(q, tok * dk * sq), sp_k = span(k, tok * dk * sq);
    const Span sp_v = span(v, tok * dv * sq), sp_o = span(o, tok * dv * so);
    const Span sp_g = span(g, tok * dk * sg), sp_b = span(beta, tok * sg);
    const size_t state_bytes = (size_t)B * H * dk * dv * sizeof(float);
    const Span sp_s0 = span(S0, S0 ? state_bytes : 0), sp_sf = span(S_final, S_final ? state_bytes : 0);

    if (T > 0) {
        if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o))
            return KDA_ERR_INVALID_ARG;
        const Span ins[] = {sp_q, sp_k, sp_v, sp_g, sp_b, sp_s0, sp_sf};
        for (const Span &s : ins)
            if (overlap(sp_o, s)) return KDA_ERR_INVALID_ARG;
    }
    if ((S0 && !aligned16(S0)) || (S_final && !aligned16(S_final))) return KDA_ERR_INVALID_ARG;
    if (S_final) {
        const Span ins[] = {sp_q, sp_k, sp_v, sp_g, sp_b};
        if (T > 0)
            for (const Span &s : ins)
                if (overlap(sp_sf, s)) return KDA_ERR_INVALID_ARG;
        if (S0 && S0 != S_final && overlap(sp_sf, sp_s0)) return KDA_ERR_INVALID_ARG;
    }
    if (T == 0 && !S_final) return KDA_OK;

    kda::ChunkFwdArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.S0 = S0; a.o = o; a.S_final = S_final;
    a.B = B; a.T = T; a.H = H; a.dk = dk; a.dv = dv;
    a.qkv_bf16 = qkv_dtype == KDA_BF16;
    a.gate_bf16 = gate_dtype == KDA_BF16;
    a.out_bf16 = out_dtype == KDA_BF16;
    return kda::launch_chunk_fwd(a, (hipStream_t)stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_decode_step(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, float *S, void *o, int B, int H, int dk, int dv,
                             kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                             void *stream)
{
    if (B < 0 || H < 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
    if (!valid_dtype(qkv_dtype) || !valid_dtype(gate_dtype) || !valid_dtype(out_dtype))
        return KDA_ERR_INVALID_ARG;
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)B * H >= ((int64_t)1 << 31)) return KDA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !S || !o) return KDA_ERR_INVALID_ARG;
    if (!aligned16(S)) return KDA_ERR_INVALID_ARG;

    const size_t n = (size_t)B * H;
    const size_t sq = dsize(qkv_dtype), sg = dsize(gate_dtype), so = dsize(out_dtype);
    const Span sp_q = span(q, n * dk * sq), sp_k = span(k, n * dk * sq), sp_v = span(v, n * dv * sq);
    const Span sp_g = span(g, n * dk * sg), sp_b = span(beta, n * sg);
    const Span sp_s = span(S, n * dk * dv * sizeof(float)), sp_o = span(o, n * dv * so);
    const Span ins[] = {sp_q, sp_k, sp_v, sp_g, sp_b};
    for (const Span &s : ins)
        if (overlap(sp_o, s) || overlap(sp_s, s)) return KDA_ERR_INVALID_ARG;
    if (overlap(sp_o, sp_s)) return KDA_ERR_INVALID_ARG;

    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S = S; a.o = o;
    a.B = B; a.H = H; a.dk = dk; a.dv = dv;
    a.qkv_bf16 = qkv_dtype == KDA_BF16;
    a.gate_bf16 = gate_dtype == KDA_BF16;
    a.out_bf16 = out_dtype == KDA_BF16;
    return kda::launch_decode_step(a, (hipStream_t)stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

const char *kda_status_string(kda_status_t status)
{
    switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: null, misaligned or overlapping pointer, bad size or dtype";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: dk/dv combination not provided";
    case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH: the HIP runtime rejected the kernel launch";
    }
    return "KDA_ERR_UNKNOWN";
}

int kda_abi_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
