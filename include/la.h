/*
 * la.h -- C ABI of the causal linear-attention library for AMD MI355X (gfx950).
 *
 * The operator replaces softmax attention with a fixed-size matrix state that
 * is updated once per token.  Three variants are provided:
 *
 *   LA_NORMALIZED   normalized kernel linear attention with phi(x) = elu(x)+1:
 *                   S_t = S_{t-1} + v_t phi(k_t)^T,  z_t = z_{t-1} + phi(k_t),
 *                   o_t = S_t phi(q_t) / (z_t . phi(q_t)).
 *                   Page "Beyond -- Linear attention and recurrent memory",
 *                   section "The big idea"; page "Linear Attention",
 *                   normalized kernel formulation.
 *   LA_GATED        gated linear attention with a per-step, per-key-channel
 *                   decay gamma_t in (0,1]^{d_k} and no normalizer:
 *                   S_t = S_{t-1} diag(gamma_t) + v_t phi(k_t)^T,
 *                   o_t = S_t phi(q_t).
 *                   Page "Ch. 11 Linear attention and Hyena", section 11.3
 *                   (GLA gate, cumulative log-gate rescaling) and the solution
 *                   to Exercise 11.5.
 *   LA_GATED_DELTA  gated delta rule with unit-norm keys, scalar gate g_t and
 *                   write strength beta_t:
 *                   S_t = g_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *                   o_t = S_t q_t.
 *                   Page "Module 18 Beyond attention", section 18.2; page
 *                   "Linear Attention", gated-delta-rule formulation.
 *   LA_KDA          the gated delta rule with a per-key-channel (diagonal)
 *                   decay alpha_t in (0,1]^{d_k}, decay first:
 *                   S_t = S_{t-1} diag(alpha_t) (I - beta_t k_t k_t^T)
 *                         + beta_t v_t k_t^T,  o_t = S_t q_t.
 *                   Page "Beyond -- Linear attention and recurrent memory",
 *                   section "From fixed decay to KDA's gated delta write".
 *   LA_RETENTION    linear attention with a fixed per-head decay gamma_h and
 *                   no normalizer (the constant gate):
 *                   S_t = gamma_h S_{t-1} + v_t phi(k_t)^T,  o_t = S_t phi(q_t).
 *                   Page "Ch. 11 Linear attention and Hyena", section 11.3
 *                   (RetNet bullet).
 *
 * LA_NORMALIZED optionally takes the same fixed per-head decay, applied to
 * both accumulators (page "Beyond -- Linear attention and recurrent memory",
 * section "Fixed decay versus an input-dependent gate"):
 *   S_t = gamma_h S_{t-1} + v_t phi(k_t)^T,  z_t = gamma_h z_{t-1} + phi(k_t).
 *
 * Every token is "update first, then read": a token attends to itself
 * (page "Beyond -- Linear attention and recurrent memory", section
 * "Pitfalls to expect").
 *
 * CONVENTIONS (all entry points)
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or retains memory, and keeps no global
 *     state except the scratch array of la_chunk_fwd_noalloc.  Calls are
 *     thread-safe (la_chunk_fwd_noalloc: see its note on overlapping calls).
 *   - Tensors are dense, row-major (C order), 16-byte aligned.
 *   - Per-token tensors are (B, H, T, d).  The state S of every variant is
 *     (B, H, d_v, d_k) float32 (row = value channel, column = key channel);
 *     the normalizer z is (B, H, d_k) float32.
 *   - q, k, v and out have the element type `dtype` (LA_F32 or LA_BF16);
 *     gates, beta and the state are always float32.  Arithmetic is float32;
 *     matrix products of bf16 inputs run on bf16 matrix cores with float32
 *     accumulation.
 *   - Arguments are validated synchronously on the host BEFORE any HIP call;
 *     a failing call launches nothing and returns LA_EINVAL or
 *     LA_EUNSUPPORTED; la_last_error() then describes the failed check.
 *   - Execution is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  No host synchronization happens inside a call.  A launch
 *     failure returns LA_EHIP.
 *   - Documented preconditions that are NOT checked (values live on the
 *     device): gate entries in (0, 1]; beta in [0, 1]; keys of
 *     LA_GATED_DELTA of unit length; z0 >= 0 for LA_NORMALIZED.  Any gate in
 *     (0, 1] is handled, however strong the decay: decay factors are only
 *     ever formed as products or exponentials that do not exceed 1.
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_ABI_VERSION 3

typedef enum {
    LA_OK = 0,
    LA_EINVAL = 1,        /* bad argument: null pointer, bad size, bad combination, misalignment, aliasing */
    LA_EUNSUPPORTED = 2,  /* valid request the library has no kernel for (head size, chunk size) */
    LA_EHIP = 3           /* the HIP runtime reported an error at launch */
} la_status;

typedef enum { LA_NORMALIZED = 0, LA_GATED = 1, LA_GATED_DELTA = 2, LA_RETENTION = 3, LA_KDA = 4 } la_variant;
typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;
typedef enum { LA_PHI_IDENTITY = 0, LA_PHI_ELU1 = 1 } la_phi;

/*
 * Problem descriptor.
 *   variant  la_variant.
 *   dtype    la_dtype of q, k, v, out.
 *   phi      feature map on q and k.  LA_NORMALIZED requires LA_PHI_ELU1 (the
 *            normalizer needs positive features); LA_GATED and LA_RETENTION
 *            accept either; LA_GATED_DELTA and LA_KDA require
 *            LA_PHI_IDENTITY.
 *   B, H     batch size and heads, >= 0.
 *   T        tokens per sequence, >= 0 (ignored by la_decode_step).
 *   d_k      key/query head size; d_v value head size.  Supported:
 *            d_k in {16, 32, 64, 128}, d_v in {16, 32, 64, 128}.
 *   chunk    chunk length of la_chunk_fwd: 0 (= 64), 16, 32, 64 or 128.
 *            The result does not depend on it beyond floating-point
 *            rounding; a length whose tiles do not fit a compute unit's LDS
 *            runs as the largest one that does (128 runs as 64).
 */
typedef struct {
    int32_t variant;
    int32_t dtype;
    int32_t phi;
    int32_t B, H, T;
    int32_t d_k, d_v;
    int32_t chunk;
} la_desc;

/*
 * Bytes of device workspace la_chunk_fwd needs for `desc` (0 when none).
 * LA_KDA with T > 0 needs one record per chunk of every head, holding the
 * chunk's state-independent tiles (Q and K scaled by their decays, W, U' and
 * the scores; about 72.5 KiB per 64-token chunk at d_k = d_v = 128 in bf16).
 * LA_NORMALIZED and LA_RETENTION with T > 0 use one as follows.  When its heads alone cannot occupy
 * the GPU its state is a plain sum over the tokens, so the sequence runs as
 * concurrent segments whose state increments are staged in the workspace
 * (one d_v x d_k + d_k float32 slot per head and segment); otherwise the
 * workspace holds a copy of z0 (B*H*d_k float32) when z_T is z0, since the
 * workgroups of a head's value blocks all read z0 and one writes z_T.  The
 * size depends on the descriptor only.  Returns 0 for an invalid descriptor
 * as well; la_chunk_fwd reports it.
 */
size_t la_chunk_fwd_workspace(const la_desc *desc);

/*
 * Chunkwise-parallel forward over whole sequences.
 *
 * The sequence is cut into chunks of `chunk` tokens (the last may be
 * ragged).  Inside a chunk, tokens interact through masked score matrices on
 * the matrix cores; across chunks only the fixed-size state is carried.
 * This is the parallel/recurrent equivalence of page "Ch. 11 Linear
 * attention and Hyena", sections 11.2-11.3, applied per chunk; the gated
 * delta rule folds its in-chunk dependencies into one unit-lower-triangular
 * solve per chunk.
 *
 *   q     (B,H,T,d_k) dtype.            k (B,H,T,d_k) dtype.
 *   v     (B,H,T,d_v) dtype.
 *   gate  LA_GATED: gamma (B,H,T,d_k) f32, 16-byte aligned;
 *         LA_KDA: alpha (B,H,T,d_k) f32, 16-byte aligned;
 *         LA_GATED_DELTA: g (B,H,T) f32;
 *         LA_NORMALIZED, LA_RETENTION: the fixed decay gamma_h (H,) f32,
 *         shared by the batch, or NULL for none (gamma_h = 1).
 *   beta  LA_GATED_DELTA, LA_KDA: (B,H,T) f32; otherwise must be NULL.
 *   S0    initial state (B,H,d_v,d_k) f32, or NULL for zeros.
 *   z0    LA_NORMALIZED: initial normalizer (B,H,d_k) f32 or NULL for
 *         zeros; otherwise must be NULL.
 *   out   (B,H,T,d_v) dtype, written.  Must not overlap any other argument.
 *   S_T   final state (B,H,d_v,d_k) f32, written, or NULL.  May be the same
 *         pointer as S0 (in-place carry); must not partially overlap it.
 *   z_T   LA_NORMALIZED: final normalizer (B,H,d_k) f32 or NULL; may equal
 *         z0.  Otherwise must be NULL.
 *   workspace, workspace_bytes
 *         caller-owned device scratch of at least la_chunk_fwd_workspace()
 *         bytes, 16-byte aligned, overlapping no other argument (may be NULL
 *         when that is 0).  Its contents on entry do not matter; calls that
 *         share one workspace must not run concurrently.
 *   stream  hipStream_t to run on.
 */
la_status la_chunk_fwd(const la_desc *desc,
                       const void *q, const void *k, const void *v,
                       const float *gate, const float *beta,
                       const float *S0, const float *z0,
                       void *out, float *S_T, float *z_T,
                       void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * Bytes of device workspace la_chunk_bwd needs for `desc` (0 for an invalid
 * descriptor): the state entering and the cotangent leaving every chunk of
 * every head, float32 (d_k d_v values, plus d_k for LA_NORMALIZED's
 * normalizer), one float per chunk and, for LA_NORMALIZED, two floats per
 * token; about 2 x 64.5 KiB per 64-token chunk at d_k = d_v = 128.  The
 * backward picks its own chunk length (64, or 32 where float32 tiles at
 * head size 128 do not fit a compute unit's LDS); desc->chunk is ignored.
 */
size_t la_chunk_bwd_workspace(const la_desc *desc);

/*
 * Chunked backward pass (training) of LA_NORMALIZED and LA_RETENTION, with
 * or without the fixed per-head decay: the gradients of a loss L with
 * respect to every input of la_chunk_fwd, given its gradients with respect
 * to the outputs.  The pages name chunkwise training without giving an
 * algorithm (page "Linear Attention", question on sequential training; page
 * "Beyond -- Linear attention and recurrent memory", section "The big
 * idea"); the chunk equations are derived from the recurrence at the top of
 * this file.  The forward pass is recomputed from the inputs, so nothing of
 * it needs to be kept: the state entering every chunk (a scan over the
 * chunks), for LA_NORMALIZED every token's output and denominator in float32
 * from float32 features (its gradient nearly cancels between the value and
 * normalizer parts, so the forward's rounded output would not do), then the
 * cotangent leaving every chunk (a reverse scan), and finally every chunk's
 * gradients on the matrix cores.  Other variants return LA_EUNSUPPORTED.
 *
 *   q, k, v, gate, S0, z0   the forward's inputs, as for la_chunk_fwd (there
 *         is no beta in these variants).
 *   dout  dL/dout (B,H,T,d_v) dtype.
 *   dS_T  dL/dS_T (B,H,d_v,d_k) f32, or NULL for zero.
 *   dz_T  LA_NORMALIZED: dL/dz_T (B,H,d_k) f32 or NULL for zero; otherwise
 *         NULL.
 *   dq, dk (B,H,T,d_k) dtype and dv (B,H,T,d_v) dtype, written.
 *   dgate dL/dgamma (H,) f32 summed over the batch, written, or NULL; must
 *         be NULL when gate is NULL.
 *   dS0   dL/dS0 (B,H,d_v,d_k) f32, written, or NULL.
 *   dz0   LA_NORMALIZED: dL/dz0 (B,H,d_k) f32, written, or NULL; otherwise
 *         NULL.
 *   workspace, workspace_bytes   at least la_chunk_bwd_workspace() bytes of
 *         caller-owned device memory, 16-byte aligned; contents on entry do
 *         not matter.
 * Outputs must not overlap each other, the inputs or the workspace.
 * Arithmetic is float32 (bf16 operands on the matrix cores for bf16 data,
 * except where a product feeds a cancellation, as above).
 */
la_status la_chunk_bwd(const la_desc *desc,
                       const void *q, const void *k, const void *v,
                       const float *gate, const float *S0, const float *z0,
                       const void *dout, const float *dS_T, const float *dz_T,
                       void *dq, void *dk, void *dv,
                       float *dgate, float *dS0, float *dz0,
                       void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * la_chunk_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  It
 * takes no workspace: the scratch la_chunk_fwd would need comes from a
 * device array the library holds, LA_NOALLOC_SCRATCH_BYTES on each GPU it
 * runs on, kept until the process ends.  The entry point itself allocates
 * nothing (no hipMalloc, no allocating library call); the caller passes every
 * input and output as for la_chunk_fwd.  A call whose la_chunk_fwd_workspace()
 * exceeds LA_NOALLOC_SCRATCH_BYTES is rejected with LA_EINVAL before any HIP
 * call.  Every call on one GPU shares that GPU's array (its contents on entry
 * do not matter), so calls that overlap in time on one GPU race: serialize
 * them, e.g. on one stream.  Otherwise the same arguments, checks and results
 * as la_chunk_fwd.
 */
#define LA_NOALLOC_SCRATCH_BYTES (32u << 20)
la_status la_chunk_fwd_noalloc(const la_desc *desc,
                               const void *q, const void *k, const void *v,
                               const float *gate, const float *beta,
                               const float *S0, const float *z0,
                               void *out, float *S_T, float *z_T,
                               void *stream);

/*
 * One recurrent decode step for every (b, h): reads one token, updates the
 * state in place, writes one output.  The per-token arithmetic is the
 * recurrence of the variant (see the top of this file), with the state
 * streamed through registers once.  desc->T and desc->chunk are ignored.
 *
 *   q, k  (B,H,d_k) dtype.   v (B,H,d_v) dtype.
 *   gate  LA_GATED: gamma (B,H,d_k) f32; LA_KDA: alpha (B,H,d_k) f32;
 *         LA_GATED_DELTA: g (B,H) f32; LA_NORMALIZED, LA_RETENTION:
 *         gamma_h (H,) f32 or NULL.
 *   beta  LA_GATED_DELTA, LA_KDA: (B,H) f32; otherwise must be NULL.
 *   S     (B,H,d_v,d_k) f32, read and overwritten with the new state.
 *   z     LA_NORMALIZED: (B,H,d_k) f32, read and overwritten; otherwise NULL.
 *   out   (B,H,d_v) dtype, written; must not overlap any other argument.
 */
la_status la_decode_step(const la_desc *desc,
                         const void *q, const void *k, const void *v,
                         const float *gate, const float *beta,
                         float *S, float *z, void *out,
                         void *stream);

/*
 * Speculative decoding by checkpoint plus input replay (page "Beyond --
 * Linear attention and recurrent memory", section "What we don't cover":
 * a fixed state has no token rows to truncate after rejected drafts).
 *
 * la_verify runs T draft tokens per sequence (desc->T) from the checkpointed
 * state S (and z) and writes the output of every token, leaving S and z
 * untouched: the same outputs as T consecutive la_decode_step calls.
 *   q, k  (B,H,T,d_k) dtype.   v (B,H,T,d_v) dtype.
 *   gate  LA_GATED: (B,H,T,d_k) f32; LA_GATED_DELTA: (B,H,T) f32;
 *         LA_NORMALIZED, LA_RETENTION: gamma_h (H,) f32 or NULL.
 *   beta  LA_GATED_DELTA: (B,H,T) f32; otherwise NULL.
 *   S, z  the checkpoint, (B,H,d_v,d_k) and (LA_NORMALIZED) (B,H,d_k) f32,
 *         read only.
 *   out   (B,H,T,d_v) dtype, written; overlaps nothing else.
 *
 * la_commit then applies the first accepted[b] tokens of each sequence b to
 * S (and z) in place, replaying the same inputs (q is not needed): the state
 * that accepted[b] la_decode_step calls would have left.  accepted is (B,)
 * int32 in device memory; values are clamped to [0, T] (0 leaves the
 * sequence's state as it is).  Both calls read the state once; la_commit
 * writes it once.  Argument checks and errors as la_decode_step.
 */
la_status la_verify(const la_desc *desc,
                    const void *q, const void *k, const void *v,
                    const float *gate, const float *beta,
                    const float *S, const float *z, void *out,
                    void *stream);
la_status la_commit(const la_desc *desc,
                    const void *k, const void *v,
                    const float *gate, const float *beta,
                    const int32_t *accepted,
                    float *S, float *z,
                    void *stream);

/* Static description of a status code. */
const char *la_status_str(la_status status);

/* Description of the last failed check on the calling thread ("" if none). */
const char *la_last_error(void);

/* LA_ABI_VERSION of the loaded library. */
int la_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LA_H */
