// Internal interface between the C ABI (kda_api.hip) and the kernel launchers.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct ChunkFwdArgs {
    const void *q, *k, *v, *g, *beta;
    const float *S0 = nullptr;        // nullable: zero initial state
    void *o = nullptr;                // nullable: outputs not written
    float *S_final = nullptr;         // nullable: final state not written
    const int *lengths = nullptr;     // nullable: per sequence, tokens from lengths[b] on are identity tokens
    const float *A_log = nullptr;     // non-null: g holds gate logits z, log-decay = -5 sigmoid(exp(A_log[h]) z)
    int B, T, H, dk, dv;
    bool qkv_bf16, gate_bf16, out_bf16;
};

struct DecodeArgs {
    const void *q, *k, *v, *g, *beta;
    float *S;
    void *o;                          // o, or y when the output epilogue is fused
    const float *A_log = nullptr;     // as in ChunkFwdArgs
    const void *z_out = nullptr;      // non-null: o -> o / rms(o) * weight * sigmoid(z_out), z_out in q's dtype
    const float *weight = nullptr;
    float eps = 0.f;
    int B, H, dk, dv;
    bool qkv_bf16, gate_bf16, out_bf16;
};

// Speculative verify (accepted == nullptr: outputs of all K drafts, S read
// only) or commit (accepted != nullptr: S advanced by accepted[b] drafts).
struct SpecArgs {
    const void *q, *k, *v, *g, *beta;
    float *S;
    void *o = nullptr;
    const int *accepted = nullptr;
    int B, K, H, dk, dv;
    bool qkv_bf16, gate_bf16, out_bf16;
};

// y = o / sqrt(mean(o^2) + eps) * weight * sigmoid(z) per row of dv channels.
struct OutputGateArgs {
    const void *o, *z;
    const float *weight;
    void *y;
    int64_t rows;
    int dv;                           // multiple of 64, at most 512
    float eps;
    bool o_bf16, z_bf16, y_bf16;
};

// Per-chunk intermediates of the backward, float32, one block per
// (sequence, head, 32-token chunk), head-major.
struct BwdWorkspace {
    float *b, *W, *dQt, *dW, *dKb;   // [chunk][32][dk]
    float *Aqk, *Akk0, *N, *dAqk;    // [chunk][32][32]
    float *U, *dU;                   // [chunk][32][dv]
    float *h, *dh;                   // [chunk][dk][dv]: state before / state gradient after the chunk
    float *dGam;                     // [chunk][dk]
};

struct ChunkBwdArgs {
    const void *q, *k, *v, *g, *beta;
    const float *S0 = nullptr;        // nullable: zero initial state
    const void *dO;
    const float *dS_final = nullptr;  // nullable: no gradient on the final state
    float *dq, *dk, *dv, *dg, *dbeta;
    float *dS0 = nullptr;             // nullable: not written
    BwdWorkspace ws;
    int B, T, H, dk_dim, dv_dim;      // (dk, dv name the gradient outputs here)
    bool qkv_bf16, gate_bf16, do_bf16;
};

hipError_t launch_chunk_fwd(const ChunkFwdArgs &a, hipStream_t stream);        // any dtypes
// Prep/state workgroups through a ring in the workspace (bfloat16 q, k, v,
// dk = 128, dv a multiple of 64 from 128 to 512, no per-sequence lengths).  `used` is
// false when the call is not taken (shape, or a workspace that is missing or
// too small): the caller then launches the other kernels.
constexpr int PS_MAX_GROUP = 128;   // heads per launch, at most
hipError_t launch_chunk_fwd_ps(const ChunkFwdArgs &a, void *workspace, size_t workspace_bytes,
                               hipStream_t stream, bool &used);
size_t chunk_ps_workspace_bytes(int B, int H, int dk, int dv);   // 0: the pair kernel does not apply
// The ring kernel's workspace inside the library (no allocation): a device
// array sized for NOALLOC_HEADS heads, its address on the stream's device.
constexpr int NOALLOC_HEADS = 64;
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(hipStream_t stream, void **out);
// Bound on every spin wait of the chunk kernels (sleeps between polls); the
// previous value is returned.  A wait that runs out marks the call failed.
unsigned set_spin_limit(unsigned limit);
unsigned spin_limit();
hipError_t launch_chunk_fwd_bf16(const ChunkFwdArgs &a, hipStream_t stream);   // bfloat16 q, k, v
// bfloat16 q, k, v, no per-sequence lengths, no logits: a.S_final <- the value
// slabs' final states from a zero start (N), M_out [B H][dk][dk] <- the chunk
// sequence's linear map on the state (S_out = M S_in + N); no outputs.
hipError_t launch_chunk_fwd_bf16_trans(const ChunkFwdArgs &a, float *M_out, hipStream_t stream);
// The forward as P segments of T / P tokens run side by side and joined
// through their linear maps (bfloat16 q, k, v, T a multiple of P, no lengths,
// no logits); the workspace holds N, M and the segments' starting states.
size_t chunk_seqpar_workspace_bytes(int B, int H, int dk, int dv, int P);
hipError_t launch_chunk_fwd_seqpar(const ChunkFwdArgs &a, int P, void *workspace, hipStream_t stream);
hipError_t launch_decode_step(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_spec_step(const SpecArgs &a, hipStream_t stream);           // dk, dv in {64, 128}
hipError_t launch_verify_tile(const SpecArgs &a, hipStream_t stream);         // K <= 16: verify, or commit if accepted is set
hipError_t launch_output_gate(const OutputGateArgs &a, hipStream_t stream);
hipError_t launch_chunk_bwd(const ChunkBwdArgs &a, hipStream_t stream);       // dk, dv in {64, 128}
size_t chunk_bwd_workspace_floats(int B, int T, int H, int dk, int dv);
BwdWorkspace chunk_bwd_workspace(float *base, int B, int T, int H, int dk, int dv);

}  // namespace kda
