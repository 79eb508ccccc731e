/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library, libkda.so.
 *
 * The layer (one head, state S with dk rows = key channels and dv columns):
 * for every token t, in order,
 *     S <- Diag(exp(g_t)) S                       fade each key channel
 *     S <- S + beta_t k_t (v_t - S^T k_t)^T       erase what k_t retrieves, write v_t
 *     o_t = S^T q_t                               read from the updated state
 * ("Review A - Sequence and depth", Free recall, the question on KDA's three
 * operations; "K3 Architecture Illustrated", section "Combining KDA and MLA",
 * FIG 21; the erase factor I - beta k k^T from the section "Under what
 * conditions are RoPE, PaTH, and KDA related?").
 *
 * kda_chunk_fwd computes this over a whole sequence in the chunkwise form:
 * sequential between 64-token chunks, parallel inside a chunk, with the
 * output split into the inter-chunk term (Gamma . Q) S and the masked
 * intra-chunk term A V~, and keys rescaled by 1/Gamma inside 16-token tiles
 * ("Kimi K3 - Lesson 3 of 14 - Sequence axis", the chunkwise diagram and the
 * paragraphs on the 1/Gamma rescale and on g_min = -5).  The result is the
 * token recurrence's, up to rounding.
 *
 * kda_decode_step advances every (sequence, head) state by one token in place
 * (the fixed-size state of "Review A", Discriminating between mechanisms).
 *
 * kda_verify_step and kda_commit_step serve speculative decoding ("K3
 * Architecture Illustrated", the section on speculative decoding: the
 * recurrent state needs rollback handling after rejected proposals): verify
 * runs K draft tokens through the current state without changing it, commit
 * then advances the state by each sequence's accepted prefix only.
 *
 * kda_chunk_fwd_gate and kda_decode_step_gate take raw gate logits z and a
 * per-head log-scale A_h instead of g, and form g = -5 sigmoid(exp(A_h) z)
 * inside the kernels ("Kimi K3 - Lesson 3 of 14 - Sequence axis", the
 * scaled-sigmoid gate with g_min = -5 and A_h a learnable per-head log-scale
 * initialised to 0).  The page shows the mapping without its formula; the
 * scale is read as acting on the logit inside the sigmoid, which keeps every
 * g in [-5, 0] for any A_h and is the plain -5 sigmoid(z) at A_h = 0.
 *
 * kda_output_gate and kda_decode_step_gated apply the module's output
 * epilogue to the read: per (token, head) row of dv channels
 *     y = o / sqrt(mean_j o_j^2 + eps) * weight * sigmoid(z_out)
 * ("Kimi K3 - Lesson 3 of 14 - Sequence axis", the output-gate paragraph: a
 * full-rank, input-dependent gate after the recurrent read decides which
 * channels pass; "K3 Architecture Illustrated", the KDA section under FIG 21:
 * the module includes normalisation and output gating).  The pages give no
 * formula; the reading is RMS normalisation over the head's dv channels with
 * a learnable per-channel weight [dv] shared by all heads, then a sigmoid
 * gate from per-token logits with o's shape.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Tensor pointers are DEVICE pointers to contiguous row-major memory, each
 *    aligned to 16 bytes.  The caller owns every buffer; the library
 *    allocates nothing, keeps no state between calls and is reentrant.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously on it; device-side faults surface at the caller's next
 *    synchronisation.
 *  - Arguments are validated on the host before any HIP call.  A non-OK
 *    status means nothing was enqueued (KDA_ERR_LAUNCH: the launch itself
 *    was rejected by the runtime).
 *  - Preconditions that are NOT checked (the data stays on the device):
 *    every g lies in [-5, 0] (the g_min = -5 floor that bounds 1/Gamma by e^80
 *    inside a 16-token tile, "Kimi K3 - Lesson 3 of 14", the g_min
 *    paragraphs); all inputs are finite.  Outside them results are undefined
 *    (typically inf/NaN), never a fault.
 *  - Keys and queries are used as given (no normalisation, no scaling).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Both enums span the whole int range (the two range members), so any int a
 * caller passes is a value of the type: out-of-set values are rejected by
 * the checks, not undefined behaviour. */
typedef enum {
    KDA_F32 = 0,   /* IEEE float32 */
    KDA_BF16 = 1,  /* bfloat16 (round-to-nearest-even when produced) */
    KDA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    KDA_DTYPE_RANGE_MAX_ = 2147483647
} kda_dtype_t;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,  /* NULL / misaligned / overlapping pointer, negative size, bad dtype */
    KDA_ERR_UNSUPPORTED = 2,  /* valid but not provided: dk or dv outside the supported set */
    KDA_ERR_LAUNCH = 3,       /* the HIP runtime rejected the kernel launch */
    KDA_ERR_SCRATCH = 4,      /* kda_chunk_fwd_noalloc: input beyond its fixed scratch */
    KDA_STATUS_RANGE_MIN_ = -2147483647 - 1,
    KDA_STATUS_RANGE_MAX_ = 2147483647
} kda_status_t;

/* ABI version of this header; bumped on any incompatible change. */
#define KDA_ABI_VERSION 6

/*
 * kda_chunk_fwd -- chunkwise forward over T tokens for B sequences x H heads.
 *
 *   q, k   [B, T, H, dk]  qkv_dtype   queries, keys
 *   v      [B, T, H, dv]  qkv_dtype   values
 *   g      [B, T, H, dk]  gate_dtype  per-key-channel log-decay, in [-5, 0]
 *   beta   [B, T, H]      gate_dtype  write strength (any real value)
 *   S0     [B, H, dk, dv] float32     initial state, or NULL for zeros
 *   o      [B, T, H, dv]  out_dtype   output (written)
 *   S_final[B, H, dk, dv] float32     state after token T-1 (written), or NULL
 *                                     to skip; may be the same pointer as S0
 *                                     (in-place continuation), must not
 *                                     overlap it otherwise.
 *
 * Supported: dk in {64, 128}; dv a positive multiple of 64, at most 512;
 * any T >= 0 (a ragged final chunk is padded internally with identity
 * tokens, which leave the state unchanged); B, H >= 0.  T == 0 copies S0
 * (or zeros) to S_final.  `o` must not overlap any input; S_final must not
 * overlap q, k, v, g, beta or o.
 *
 * Internal state is float32.  Contractions run on the matrix cores with
 * float32 accumulation: float32 operands when qkv_dtype == KDA_F32; for
 * KDA_BF16 inputs, fp16 operands (11 significant bits), with the state-update
 * operand U and the right-hand sides of the diagonal solves carried as two
 * fp16 terms, and two-term bfloat16 for the diagonal 16-token Gram tiles,
 * whose 1/decay factor reaches e^80.  The fp16 operands need |v|, |S| and
 * |o| below 65504 (true for unit-scale values and L2-normalised q and k, as
 * the method uses them); beyond that the KDA_BF16 path produces inf.
 * out_dtype == KDA_F32 keeps the output at accumulator precision; KDA_BF16
 * rounds it once (the output of a heavy-tailed workload can lose several
 * percent of its RMS to that rounding alone).
 */
kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v,
                           const void *g, const void *beta, const float *S0,
                           void *o, float *S_final,
                           int B, int T, int H, int dk, int dv,
                           kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype,
                           kda_dtype_t out_dtype, void *stream);

/*
 * kda_decode_step -- one token for every (sequence, head), state updated in place.
 *
 *   q, k   [B, H, dk]     qkv_dtype
 *   v      [B, H, dv]     qkv_dtype
 *   g      [B, H, dk]     gate_dtype  log-decay in [-5, 0]
 *   beta   [B, H]         gate_dtype
 *   S      [B, H, dk, dv] float32     read and written IN PLACE
 *   o      [B, H, dv]     out_dtype   output (written)
 *
 * Supported: dk in {64, 128}, dv in {64, 128}; B, H >= 0.  `o` must not
 * overlap any input or S; S must not overlap q, k, v, g or beta.
 * Arithmetic is float32 throughout (the step is bandwidth-bound).
 */
kda_status_t kda_decode_step(const void *q, const void *k, const void *v,
                             const void *g, const void *beta, float *S, void *o,
                             int B, int H, int dk, int dv,
                             kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype,
                             kda_dtype_t out_dtype, void *stream);

/*
 * kda_chunk_fwd_gate -- kda_chunk_fwd with the log-decay formed in the kernel.
 *
 *   z      [B, T, H, dk]  gate_dtype  gate logits (any real value)
 *   A_log  [H]            float32     per-head log-scale A_h (device pointer,
 *                                     4-byte aligned)
 *   g = -5 sigmoid(exp(A_log[h]) z), in [-5, 0] for every z.  Everything
 *   else, including supported sizes and errors, as kda_chunk_fwd; A_log must
 *   not be NULL and must not overlap o or S_final.
 */
kda_status_t kda_chunk_fwd_gate(const void *q, const void *k, const void *v,
                                const void *z, const float *A_log, const void *beta,
                                const float *S0, void *o, float *S_final,
                                int B, int T, int H, int dk, int dv,
                                kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype,
                                kda_dtype_t out_dtype, void *stream);

/*
 * kda_chunk_fwd_ws, kda_chunk_fwd_gate_ws -- kda_chunk_fwd and
 * kda_chunk_fwd_gate with a caller-owned workspace.  The workspace lets
 * bfloat16 q, k, v with dk = 128 (dv a multiple of 64 from 128 to 512) take
 * the ring kernel: a head's dv columns are split over dv / 64 workgroups,
 * which take turns computing the state-independent part of the chunks of the
 * chunkwise form ("Kimi K3 - Lesson 3 of 14 - Sequence axis", the chunkwise
 * diagram: decays, 1/Gamma-rescaled operands, intra-chunk Gram tiles, the
 * diagonal inverses), so each chunk's part is computed once per head instead
 * of once per workgroup, and hand it to one another through a four-slot ring
 * per head held in the workspace.  Other inputs run the kernels of
 * kda_chunk_fwd.  The ring pays for dv of 256 and more when the grid (B H dv
 * / 64 workgroups) fills at most half the device (at B = 1, H = 8, T = 4096:
 * 1.0x the time of kda_chunk_fwd at dv = 128, 0.84x at dv = 256, 0.79x at
 * dv = 512); a full-device grid runs faster without it (1.28x at B = 1, H =
 * 96, T = 131072, dv = 128).
 *
 *   workspace        device memory of at least kda_chunk_fwd_workspace_bytes(B,
 *                    T, H, dk, dv) bytes, 16-byte aligned, owned by the caller;
 *                    it needs no initialisation, its contents are undefined
 *                    afterwards, and it must not overlap any other argument.
 *                    NULL makes the call kda_chunk_fwd (or _gate) exactly.
 *   workspace_bytes  its size; a non-NULL workspace below the required size is
 *                    KDA_ERR_INVALID_ARG.
 *
 * Everything else (shapes, dtypes, aliasing rules, preconditions, precision,
 * errors) as kda_chunk_fwd / kda_chunk_fwd_gate; the arithmetic is the same,
 * step for step.  Calls sharing one workspace must not overlap in time (use
 * one stream, or one workspace per stream).  The kernel's workgroups wait
 * for one another (bounded waits, at most kda_debug_set_spin_limit sleeps
 * each); if a wait runs out, the call still completes and every output it
 * writes from then on (o and S_final of the affected heads) is NaN.
 */
size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv);   /* 0: no workspace is used */

kda_status_t kda_chunk_fwd_ws(const void *q, const void *k, const void *v,
                              const void *g, const void *beta, const float *S0,
                              void *o, float *S_final, void *workspace, size_t workspace_bytes,
                              int B, int T, int H, int dk, int dv,
                              kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype,
                              kda_dtype_t out_dtype, void *stream);

kda_status_t kda_chunk_fwd_gate_ws(const void *q, const void *k, const void *v,
                                   const void *z, const float *A_log, const void *beta,
                                   const float *S0, void *o, float *S_final,
                                   void *workspace, size_t workspace_bytes,
                                   int B, int T, int H, int dk, int dv,
                                   kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype,
                                   kda_dtype_t out_dtype, void *stream);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd_ws for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the ring lives in a device array inside the library
 * instead of a caller's workspace.  The call allocates nothing and calls no
 * allocating routine.
 *
 * Arguments, preconditions, results and errors as kda_chunk_fwd_ws without
 * the workspace.  The array holds the ring of 64 heads (about 15.8 MiB per
 * device, kept until the process ends): where the ring kernel applies
 * (bfloat16 q, k, v, dk = 128, dv a multiple of 64 from 128 to 512) and B * H
 * exceeds 64, the call returns KDA_ERR_SCRATCH and enqueues nothing; other
 * inputs run the kernels of kda_chunk_fwd, which use no scratch.  Every call
 * on one device shares that device's array: calls that overlap in time on one
 * device (two streams, two threads) race and give undefined results; calls
 * ordered on one stream do not.  The array's contents carry over from call to
 * call and need no clearing (each launch tags its flags with a fresh epoch).
 */
kda_status_t kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                   const void *g, const void *beta, const float *S0,
                                   void *o, float *S_final, int B, int T, int H, int dk, int dv,
                                   kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype,
                                   kda_dtype_t out_dtype, void *stream);

/*
 * kda_chunk_fwd_seqpar -- kda_chunk_fwd computed as `segments` pieces of the
 * sequence side by side, for grids too small to fill the device (few
 * sequences and heads, long T).  Between chunks the chunkwise form is a
 * sequential recurrence ("Kimi K3 - Lesson 3 of 14 - Sequence axis", the
 * chunkwise diagram), but each chunk's step is affine in the state, so a run
 * of chunks is too: S_out = M S_in + N.  The call runs every segment of
 * T / segments tokens from a zero state, also carrying dk transition columns
 * that start from the identity with zero values (giving N and M per segment),
 * forms the segments' true starting states in order (S_{p+1} = M_p S_p + N_p
 * in float32; the last one is S_final), and runs every segment again from its
 * starting state to write o.  The sequential part is T / segments tokens long
 * twice instead of T once, at (dv + dk) / dv times the first pass's columns.
 * Results equal kda_chunk_fwd's up to rounding (the chunks start at every
 * segment start, and the segments meet through the float32 products).
 *
 *   segments   1 .. KDA_SEQPAR_MAX_SEGMENTS, dividing T; it pays while
 *              B * segments * H * (dv + dk) / 64 workgroups fit the device.
 *   workspace  device memory of at least kda_chunk_fwd_seqpar_workspace_bytes
 *              bytes, 16-byte aligned, owned by the caller, not overlapping any
 *              other argument; no initialisation needed, contents undefined
 *              afterwards.  Calls sharing one workspace must not overlap in time.
 *
 * Everything else (shapes, dtypes, S0 / S_final aliasing, preconditions,
 * precision, errors) as kda_chunk_fwd, with these additions: q, k, v must be
 * bfloat16 (KDA_ERR_UNSUPPORTED otherwise); segments outside the range or not
 * dividing T, or a missing or short workspace, is KDA_ERR_INVALID_ARG.
 */
#define KDA_SEQPAR_MAX_SEGMENTS 64
size_t kda_chunk_fwd_seqpar_workspace_bytes(int B, int T, int H, int dk, int dv, int segments);   /* 0: invalid shape */

/*
 * kda_chunk_fwd_seqpar_segments -- a segment count for kda_chunk_fwd_seqpar,
 * or 1 where the plain kda_chunk_fwd is expected to be faster.  Host-only
 * arithmetic on the shape: among the divisors of T up to
 * KDA_SEQPAR_MAX_SEGMENTS, the one with the smallest estimated time (passes
 * of B * segments * H * (dv + dk) / 64 and B * segments * H * dv / 64
 * workgroups over `cus` compute units, and the combine), compared with the
 * plain forward's, from per-chunk and per-segment costs measured on MI355X.
 * cus <= 0 takes the current device's compute-unit count (1 is returned if
 * that query fails).  Invalid shapes return 1.
 */
int kda_chunk_fwd_seqpar_segments(int B, int T, int H, int dk, int dv, int cus);

kda_status_t kda_chunk_fwd_seqpar(const void *q, const void *k, const void *v,
                                  const void *g, const void *beta, const float *S0,
                                  void *o, float *S_final, void *workspace, size_t workspace_bytes,
                                  int B, int T, int H, int dk, int dv, int segments,
                                  kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype,
                                  kda_dtype_t out_dtype, void *stream);

/*
 * kda_chunk_fwd_gate_seqpar -- kda_chunk_fwd_seqpar with the log-decay formed
 * in the kernels from gate logits z and per-head A_log, as kda_chunk_fwd_gate
 * does ("Kimi K3 - Lesson 3 of 14 - Sequence axis", the scaled-sigmoid
 * mapping).  Arguments as kda_chunk_fwd_seqpar with z in place of g and A_log
 * ([H] float32, device) added; a NULL A_log is KDA_ERR_INVALID_ARG.  The
 * workspace size is kda_chunk_fwd_seqpar_workspace_bytes'.
 */
kda_status_t kda_chunk_fwd_gate_seqpar(const void *q, const void *k, const void *v,
                                       const void *z, const float *A_log, const void *beta,
                                       const float *S0, void *o, float *S_final,
                                       void *workspace, size_t workspace_bytes,
                                       int B, int T, int H, int dk, int dv, int segments,
                                       kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype,
                                       kda_dtype_t out_dtype, void *stream);

/*
 * kda_debug_set_spin_limit -- test hook: the bound (sleeps between polls) on
 * every wait inside the chunk kernels launched after the call, process-wide;
 * returns the previous bound (default 2^20).  A small bound makes the waits
 * give up, which lets a test check that a failed wait yields NaN outputs
 * rather than wrong finite ones.  Not for production use.
 */
unsigned kda_debug_set_spin_limit(unsigned limit);

/*
 * kda_decode_step_gate -- kda_decode_step with g = -5 sigmoid(exp(A_log[h]) z)
 * formed in the kernel (z [B, H, dk] gate_dtype, A_log [H] float32).
 */
kda_status_t kda_decode_step_gate(const void *q, const void *k, const void *v,
                                  const void *z, const float *A_log, const void *beta,
                                  float *S, void *o, int B, int H, int dk, int dv,
                                  kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype,
                                  kda_dtype_t out_dtype, void *stream);

/*
 * kda_verify_step -- K draft tokens per sequence through the current state,
 * outputs only.
 *
 *   q, k, g [B, K, H, dk], v [B, K, H, dv], beta [B, K, H]: the draft tokens
 *   S       [B, H, dk, dv] float32   the state before the drafts; READ ONLY
 *   o       [B, K, H, dv]  out_dtype o[:, j] is the output token j would get
 *                                    after tokens 0..j-1 of its draft
 *
 * Equivalent to kda_chunk_fwd(q, k, v, g, beta, S0 = S, o, S_final = NULL)
 * over T = K tokens; same sizes, dtypes and errors.  S must not be NULL and
 * must not overlap o.  Up to 16 drafts run as one tile of the chunkwise form
 * on the matrix cores; with KDA_BF16 drafts its two products with the state
 * take single fp16 operands (so |S| must stay below 65504, as for
 * kda_chunk_fwd), with KDA_F32 drafts float32 operands.
 */
kda_status_t kda_verify_step(const void *q, const void *k, const void *v,
                             const void *g, const void *beta, const float *S, void *o,
                             int B, int K, int H, int dk, int dv,
                             kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype,
                             kda_dtype_t out_dtype, void *stream);

/*
 * kda_commit_step -- advance S in place by the accepted prefix of each draft.
 *
 *   k, g [B, K, H, dk], v [B, K, H, dv], beta [B, K, H]: the same draft tokens
 *   accepted [B] int32 (device): tokens 0..accepted[b]-1 of sequence b are
 *                   applied, the rest are treated as identity tokens (values
 *                   are clamped to [0, K])
 *   S        [B, H, dk, dv] float32, read and written IN PLACE
 *
 * Afterwards S is the state kda_chunk_fwd would reach over the first
 * accepted[b] tokens of each sequence.  No output is written.  S must not
 * overlap k, v, g, beta or accepted.  A sequence with no accepted token
 * keeps its state bit for bit.  Up to 16 drafts run as one tile on the
 * matrix cores (S read once, updated in registers, written once; of the
 * drafts only the accepted prefix is read from memory); with
 * KDA_BF16 drafts the products take two-term fp16 operands (about 22
 * significant bits; |S| below 65504), with KDA_F32 drafts float32 operands.
 */
kda_status_t kda_commit_step(const void *k, const void *v, const void *g, const void *beta,
                             const int *accepted, float *S,
                             int B, int K, int H, int dk, int dv,
                             kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, void *stream);

/*
 * kda_output_gate -- the output epilogue over `rows` rows of dv channels
 * (rows = B * T * H for a forward's o [B, T, H, dv]).
 *
 *   o      [rows, dv] o_dtype       the reads
 *   z      [rows, dv] z_dtype       gate logits
 *   weight [dv] float32             per-channel normalisation weight
 *   eps    >= 0, finite             added to the mean square (eps = 0 makes an
 *                                   all-zero row NaN, as the formula does)
 *   y      [rows, dv] y_dtype       the result; may be o itself when
 *                                   y_dtype == o_dtype, must not overlap z or
 *                                   weight otherwise
 *
 * dv a multiple of 64 up to 512 (else KDA_ERR_UNSUPPORTED).  float32 arithmetic.
 */
kda_status_t kda_output_gate(const void *o, const void *z, const float *weight, float eps, void *y,
                             int64_t rows, int dv, kda_dtype_t o_dtype, kda_dtype_t z_dtype,
                             kda_dtype_t y_dtype, void *stream);

/*
 * kda_decode_step_gated -- a decode step whose output goes through the output
 * epilogue inside the same kernel: y = kda_output_gate(o) with o the read
 * kda_decode_step would write.
 *
 *   g       [B, H, dk] gate_dtype: the log-decay when A_log is NULL, gate
 *           logits (as kda_decode_step_gate) when A_log [H] float32 is given
 *   z_out   [B, H, dv] qkv_dtype    output-gate logits
 *   weight  [dv] float32, eps >= 0  as kda_output_gate
 *   y       [B, H, dv] out_dtype    the gated output (o itself is not stored)
 *
 * Otherwise as kda_decode_step; y must not overlap any input or S.
 */
kda_status_t kda_decode_step_gated(const void *q, const void *k, const void *v, const void *g,
                                   const float *A_log, const void *beta, float *S, const void *z_out,
                                   const float *weight, float eps, void *y, int B, int H, int dk, int dv,
                                   kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t out_dtype,
                                   void *stream);

/*
 * kda_chunk_bwd -- gradients of kda_chunk_fwd.  Given the upstream gradients
 * dO of the outputs (and dS_final of the final state), computes the
 * gradients of L = sum(o * dO) + sum(S_final * dS_final) with respect to
 * q, k, v, g, beta and S0.  The pages describe training the layer but give
 * no gradients; these are the derivatives of the recurrence above, taken
 * through the chunkwise form (32-token chunks, tile-local 1/Gamma references
 * as in the forward, float32 arithmetic throughout).
 *
 *   q, k, v, g, beta, S0   as kda_chunk_fwd (S0 NULL = zero state)
 *   dO        [B, T, H, dv]  do_dtype
 *   dS_final  [B, H, dk, dv] float32, or NULL (= zero)
 *   dq, dk, dg [B, T, H, dk], dv [B, T, H, dv], dbeta [B, T, H]: float32 outputs
 *   dS0       [B, H, dk, dv] float32 output, or NULL (not written)
 *   workspace device memory of at least kda_chunk_bwd_workspace_bytes(B, T,
 *             H, dk, dv) bytes, owned by the caller, contents undefined
 *             before and after; it must not overlap any argument
 *
 * dk, dv in {64, 128} (else KDA_ERR_UNSUPPORTED).  No output may overlap an
 * input, another output or the workspace.  Preconditions as the forward.
 */
size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv);

kda_status_t kda_chunk_bwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                           const float *S0, const void *dO, const float *dS_final,
                           float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dS0,
                           void *workspace, size_t workspace_bytes,
                           int B, int T, int H, int dk_dim, int dv_dim,
                           kda_dtype_t qkv_dtype, kda_dtype_t gate_dtype, kda_dtype_t do_dtype,
                           void *stream);

/* Static, human-readable name of a status code (never NULL). */
const char *kda_status_string(kda_status_t status);   /* codes outside the set: "KDA_ERR_UNKNOWN" */

/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
