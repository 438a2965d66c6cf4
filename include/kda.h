/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward library
 * (libkda.so).
 *
 * What is computed.  For every batch entry b and head h independently, with
 * state S in R^{dk x dv} (rows = key channels, columns = value channels):
 *
 *   g_t     = g_min * sigmoid(exp(A[h]) * z_t)     per key channel   (Eq. 5)
 *   alpha_t = exp(g_t)
 *   S_t     = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T   (Eq. 1)
 *   o_t     = scale * S_t^T q_t                    (read AFTER the update)
 *
 * Sources: Eq. 1 and the read-after-update order -- "Kimi K3: the paper and
 * proofs side by side", section 2.1.1 (Equation 1) and its Lean `step`; the
 * bounded gate with g_min = -5 -- "Kimi K3 reading notes", section 2 (Hybrid
 * Attention); carrying the state across a split of the sequence -- the
 * paper-and-proofs page, "Streaming, full sequences, and chunk boundaries"
 * (run_append); heads packed and independent -- the same page, updateTerm.
 * Eq. 1 has no output scale; pass scale = 1 for the equation as written.
 *
 * Conventions shared by every entry point.
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent),
 *    owned by the caller.  The library never allocates, frees or retains them.
 *  - Layouts are contiguous row-major, token-major:
 *      q, k, z, G : [B, T, H, dk]     v, o : [B, T, H, dv]     beta : [B, T, H]
 *      A          : [H, dk] fp32      state: [B, H, dk, dv] fp32
 *    (decode uses N sequences in place of B and no T axis).
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously; the call returns after enqueue without synchronising.
 *  - Arguments are validated on the host before anything is launched.  On any
 *    error the call launches nothing and writes no output or state.  A launch
 *    failure reported by the runtime returns KDA_ERR_HIP.  Nothing throws.
 *  - Supported: dk, dv in {16, 32, 64, 128}; chunk in {16, 64}; any T >= 0
 *    (the last chunk may be partial); input dtype KDA_F32 or KDA_BF16 (q, k,
 *    v, z, beta share it); output dtype KDA_F32 or KDA_BF16.  Anything else
 *    returns KDA_ERR_UNSUPPORTED.  Sizes are limited so that every element
 *    index fits in 63 bits and B*H, N*H fit in 31 bits; T (and n_draft) is at
 *    most 2^31 - 65.  Larger sizes return KDA_ERR_SHAPE.
 *  - Alignment: tensor base pointers 16-byte aligned (beta: its element
 *    size).  Allocator pointers and token slices of contiguous tensors with
 *    d >= 16 satisfy this.  Otherwise KDA_ERR_ALIGN.
 *  - Calls on one stream run in order; concurrent calls on different streams
 *    must not write the same state or output buffers.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes: zero on success, negative on error.  The first six keep the
 * numbering of the boundary's contract sketch; KDA_ERR_ALIAS and KDA_ERR_ALIGN
 * are this library's additions. */
typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_NULL = -1,        /* a required pointer is NULL                    */
  KDA_ERR_SHAPE = -2,       /* a size is negative, zero where it must be at
                               least 1 (H, N, dk, dv), or too large          */
  KDA_ERR_DTYPE = -3,       /* dtype enum out of range                       */
  KDA_ERR_WORKSPACE = -4,   /* the caller's workspace is smaller than needed */
  KDA_ERR_UNSUPPORTED = -5, /* valid but not provided (dk, dv, chunk, ...)   */
  KDA_ERR_HIP = -6,         /* the HIP runtime reported an error at launch   */
  KDA_ERR_ALIAS = -7,       /* outputs overlap inputs in a forbidden way     */
  KDA_ERR_ALIGN = -8        /* a pointer is not aligned as required          */
} kda_status;

typedef enum kda_dtype { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Human-readable name of a status code (static storage; never NULL). */
const char* kda_status_string(int status);

/* Library ABI version (major * 100 + minor): 200 since the chunked prefill
 * takes a workspace and the status codes are negative. */
int kda_version(void);

/* 1 when kda_chunk_fwd / kda_chunk_fwd_z run the bf16 matrix-core kernel
 * (bf16 matrix products with fp32 accumulation) for these arguments, 0 when
 * they run the fp32 matrix-core tile kernel (fp32 products throughout).  Pure
 * query: touches no device. */
int kda_chunk_uses_mfma(kda_dtype in_dtype, int dk, int dv, int chunk);

/*
 * kda_gate -- bounded decay gate and chunk-local log-decay sums.
 *
 * G[b,t,h,c] = sum over u from the start of t's chunk up to t of
 *              g_min * sigmoid(exp(A[h,c]) * z[b,u,h,c]),
 * chunks being consecutive runs of `chunk` tokens starting at t = 0
 * (chunk = 1 returns g itself).  Natural-log units, fp32 output.
 * Source: "Kimi K3 reading notes", section 2 (g and alpha = exp(g)); the
 * chunk-local sums are the cumulative log-decay whose 16-token range
 * (-80, 0) the same section states.
 *
 *   z      [B,T,H,dk] in z_dtype (device)     A [H,dk] fp32 (device)
 *   g_min  lower bound of g (the pages fix -5), in [-5, 0]: the range the
 *          chunked prefill accepts (KDA_ERR_UNSUPPORTED otherwise)
 *   chunk  1, 16 or 64
 *   G      [B,T,H,dk] fp32 (device, written); must not overlap z or A
 */
kda_status kda_gate(const void* z, kda_dtype z_dtype, const float* A,
                    float g_min, int B, int T, int H, int dk, int chunk,
                    float* G, void* stream);

/*
 * kda_chunk_fwd_workspace_bytes -- device scratch memory that kda_chunk_fwd,
 * kda_chunk_fwd_z and kda_chunk_fwd_z_prologue need for these sizes (any
 * input dtype).  0 means the call needs none (workspace may then be NULL).
 * Pure host computation; negative or zero-sized arguments give 0.
 *
 * The library picks the launch form from the sizes alone: one pass over the
 * sequence when B*H alone fills the GPU, otherwise (few, long sequences) the
 * segment-parallel form of "Kimi K3 reading notes", section 7, whose
 * per-segment end states, transitions and entry states live in the workspace.
 * Both forms give the same result within the stated tolerance.
 */
size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk);

/*
 * kda_chunk_fwd -- chunked prefill with state in and out, from precomputed
 * chunk-local log-decay sums G (the output of kda_gate with the same chunk).
 *
 * Computes, for t = 0..T-1 of every (b, h), o_t and the final state S_T of
 * the recurrence above, starting from S_in (or zero).  The chunked algorithm
 * regroups the token updates inside each chunk of `chunk` tokens (the
 * chunkwise form named on "Kimi K3: architecture, derivations and a
 * pinned-source audit", section 4.5) and carries the state between chunks;
 * results equal the token recurrence up to rounding.
 *
 *   q, k   [B,T,H,dk] in_dtype     v [B,T,H,dv] in_dtype     beta [B,T,H] in_dtype
 *   G      [B,T,H,dk] fp32 chunk-local sums (chunk must match kda_gate's).
 *          Every channel's log-decay over any aligned 16-token tile (both
 *          kernels anchor their decay factors per tile), G at the tile's last
 *          token minus G before its first, must be at least -80: the
 *          tile's decay and its reciprocal must be normal fp32 numbers,
 *          and so must a query or key component times that decay.  G from
 *          kda_gate (g_min >= -5, the bounded gate of the pages) always is.
 *   S_in   [B,H,dk,dv] fp32 or NULL (zero state)
 *   o      [B,T,H,dv] in o_dtype (written)
 *   S_out  [B,H,dk,dv] fp32 or NULL (not written); may equal S_in exactly
 *          (in-place state update) but must not partially overlap it
 *   scale  output scale (1 for Eq. 1 as written)
 *   workspace, workspace_bytes
 *          caller-owned device memory, 16-byte aligned, of at least
 *          kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk) bytes
 *          (KDA_ERR_WORKSPACE otherwise; NULL when that is 0).  It must not
 *          overlap any argument; its contents on entry do not matter and are
 *          overwritten.  Calls that run concurrently need separate workspaces.
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v,
                         const void* beta, kda_dtype in_dtype, const float* G,
                         const float* S_in, void* o, kda_dtype o_dtype,
                         float* S_out, int B, int T, int H, int dk, int dv,
                         int chunk, float scale, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd_z -- the same chunked prefill with the gate fused: takes the
 * decay logits z [B,T,H,dk] (in_dtype), A [H,dk] fp32 and g_min instead of G.
 * Equal to kda_gate followed by kda_chunk_fwd up to rounding; this is the
 * path that avoids the fp32 round trip of G through memory.  g_min must lie
 * in [-5, 0] (16 g_min >= -80 keeps every 16-token tile's decay, its
 * reciprocal and a query or key component times that decay normal fp32
 * numbers); other values return KDA_ERR_UNSUPPORTED.
 * Workspace: as kda_chunk_fwd.
 */
kda_status kda_chunk_fwd_z(const void* q, const void* k, const void* v,
                           const void* beta, const void* z, kda_dtype in_dtype,
                           const float* A, float g_min, const float* S_in,
                           void* o, kda_dtype o_dtype, float* S_out, int B,
                           int T, int H, int dk, int dv, int chunk, float scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd_z_noalloc -- kda_chunk_fwd_z for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, result and validation as
 * kda_chunk_fwd_z, without the workspace: where the call needs scratch memory
 * (kda_chunk_fwd_workspace_bytes > 0) it uses a static array of the library's
 * on the current device, of KDA_NOALLOC_SCRATCH_BYTES (24 MiB), which each
 * device holds until the process ends.  A need beyond that returns
 * KDA_ERR_WORKSPACE (the automatic launch form never needs more: it makes at
 * most 128 (b, h, segment) units of three 128 x 128 fp32 matrices each).  The
 * call allocates nothing.  Every call on one device
 * shares that device's array, whose contents the call overwrites before
 * reading: calls that overlap in time on one device (different streams, or
 * threads) race and must not be issued; calls in order on one stream are safe.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)24 << 20)
kda_status kda_chunk_fwd_z_noalloc(const void* q, const void* k, const void* v,
                                   const void* beta, const void* z, kda_dtype in_dtype,
                                   const float* A, float g_min, const float* S_in,
                                   void* o, kda_dtype o_dtype, float* S_out, int B,
                                   int T, int H, int dk, int dv, int chunk, float scale,
                                   void* stream);

/*
 * kda_decode_step -- one token per sequence, state updated IN PLACE.
 *
 * For n < N, h < H: gate from z and A, S[n,h] <- (I - beta k k^T)
 * Diag(alpha) S[n,h] + beta k v^T, o[n,h] = scale * S[n,h]^T q.
 * The state is fixed-size per sequence; a caller that must keep the old
 * state (a cached prefix) copies it before calling ("Kimi K3: architecture,
 * derivations and a pinned-source audit", section 9.3: copy before mutation).
 *
 *   q, k, z [N,H,dk] in_dtype    v [N,H,dv] in_dtype    beta [N,H] in_dtype
 *   A       [H,dk] fp32          S [N,H,dk,dv] fp32 (read and written)
 *   o       [N,H,dv] in o_dtype (written; must not overlap S)
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v,
                           const void* z, const void* beta, kda_dtype in_dtype,
                           const float* A, float g_min, float* S, void* o,
                           kda_dtype o_dtype, int N, int H, int dk, int dv,
                           float scale, void* stream);

/*
 * Fused prologue ("Kimi K3: the paper and proofs side by side", section 2.1.1,
 * Equations 2-6, "Preparing the queries, keys, values, and decay"; write
 * strength in (0, 1): "Kimi K3: architecture, derivations and a
 * pinned-source audit", section 4.2).
 *
 * kda_chunk_fwd_z_prologue and kda_decode_step_prologue take the same
 * arguments as kda_chunk_fwd_z (workspace included: its size is
 * kda_chunk_fwd_workspace_bytes) and kda_decode_step, but q and k arrive
 * un-normalised and beta as a logit.  Inside the kernels, per token:
 *   q^ = q / sqrt(|q|^2 + 1e-6),  k^ = k / sqrt(|k|^2 + 1e-6)   (fp32 sums)
 *   beta = 1 / (1 + e^(-beta_logit))
 * and the step then runs on (q^, k^, beta).  A zero q or k stays zero.  The
 * short convolution, the activation and the projections that produce these
 * inputs are not part of the library (they need trained weights).
 * Shapes, dtypes, layouts, validation and errors: as the plain entry points.
 */
kda_status kda_chunk_fwd_z_prologue(const void* q, const void* k, const void* v, const void* beta_logit,
                                    const void* z, kda_dtype in_dtype, const float* A, float g_min,
                                    const float* S_in, void* o, kda_dtype o_dtype, float* S_out, int B, int T,
                                    int H, int dk, int dv, int chunk, float scale, void* workspace,
                                    size_t workspace_bytes, void* stream);
kda_status kda_decode_step_prologue(const void* q, const void* k, const void* v, const void* z,
                                    const void* beta_logit, kda_dtype in_dtype, const float* A, float g_min,
                                    float* S, void* o, kda_dtype o_dtype, int N, int H, int dk, int dv,
                                    float scale, void* stream);

/*
 * kda_chunk_bwd_z -- backward pass of kda_chunk_fwd_z (training).
 *
 * Given the forward's inputs and dL/do (d_o [B,T,H,dv], dtype do_dtype) and
 * optionally dL/dS_out (dS_out [B,H,dk,dv] fp32, NULL = the final state does not
 * enter the loss), writes the gradients of L with respect to every input, in
 * fp32, in the layouts of the inputs: dq, dk, dz [B,T,H,dk]; dv [B,T,H,dv];
 * dbeta [B,T,H]; dA [H,dk] (summed over batch and tokens); dS_in [B,H,dk,dv]
 * (may be NULL).  S_in may be NULL (zero state), as in the forward.
 *
 * The derivative is the chain rule of the forward recurrence ("Kimi K3: the
 * paper and proofs side by side", section 2.1.1, Equation 1, and the bounded
 * gate of "Kimi K3 reading notes", section 2), computed chunkwise: a forward
 * pass keeps the state entering every 64-token block in the workspace, then
 * one workgroup per (b, h), or per (b, h, half of the value columns) when that
 * leaves compute units idle, walks the blocks backwards in 16-token sub-chunks:
 * matrix-core products with fp32 accumulation, fp32 operands for fp32 inputs and
 * bf16 operands on the larger products for bf16 inputs.  Deterministic: two
 * calls on the same inputs give the same bits.
 *
 * Supported: dk, dv in {16, 32, 64, 128}; in_dtype, do_dtype in {f32, bf16};
 * g_min in [-5, 0] (16 g_min >= -80 keeps every in-sub-chunk decay ratio in
 * the fp32 range).  workspace: caller-owned device memory, 16-byte aligned, of
 * kda_chunk_bwd_z_workspace_bytes(B, T, H, dk, dv) bytes; contents on entry do
 * not matter.  No output may overlap an input, another output or the workspace.
 */
size_t kda_chunk_bwd_z_workspace_bytes(int B, int T, int H, int dk, int dv);
kda_status kda_chunk_bwd_z(const void* q, const void* k, const void* v, const void* beta, const void* z,
                           kda_dtype in_dtype, const float* A, float g_min, const float* S_in,
                           const void* d_o, kda_dtype do_dtype, const float* dS_out, float* dq, float* dk,
                           float* dv, float* dbeta, float* dz, float* dA, float* dS_in, int B, int T, int H,
                           int dk_dim, int dv_dim, float scale, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * kda_chunk_fwd_z_segmented -- kda_chunk_fwd_z for few, long sequences.
 *
 * Same inputs, outputs and result as kda_chunk_fwd_z (within the stated
 * tolerance of the input dtype: the arithmetic is regrouped).  The sequence is cut into
 * `segments` chunk-aligned segments that run in parallel, using the fragment
 * decomposition of "Kimi K3 reading notes", section 7: each segment from the
 * zero state gives its end state S~_p; from the identity with zero values, its
 * transition M_p (a dk x dk map); a scan gives the true entry states
 * E_{p+1} = M_p E_p + S~_p (E_0 = S_in); each segment then runs from E_p and
 * writes its outputs, the last one S_out.  About three times the work of one
 * pass, for `segments` times the parallelism: the form for small B*H and long
 * T (a million tokens on 8 heads), where one pass leaves most of the GPU idle.
 *
 * Applies to every supported shape and dtype.  segments == 1, or T within
 * one segment's length, runs the plain kda_chunk_fwd_z (no workspace needed).
 *
 * workspace: caller-owned device memory, 16-byte aligned, at least
 * kda_chunk_fwd_z_segmented_workspace_bytes(B, H, dk, dv, segments) bytes
 * (KDA_ERR_WORKSPACE otherwise), overlapping no argument; its contents on
 * entry do not matter and are overwritten.  S_out may equal S_in.
 */
size_t kda_chunk_fwd_z_segmented_workspace_bytes(int B, int H, int dk, int dv, int segments);
kda_status kda_chunk_fwd_z_segmented(const void* q, const void* k, const void* v,
                                     const void* beta, const void* z, kda_dtype in_dtype,
                                     const float* A, float g_min, const float* S_in,
                                     void* o, kda_dtype o_dtype, float* S_out, int B,
                                     int T, int H, int dk, int dv, int chunk, float scale,
                                     int segments, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * kda_decode_replay -- speculative-decoding state replay in one launch
 * ("Kimi K3: architecture, derivations and a pinned-source audit", section
 * 10.3: the drafted tokens' inputs are cached and the accepted prefix is
 * replayed on chip instead of rolling the state back).
 *
 * For n < N, h < H the drafted tokens t = 0 .. n_draft-1 run one at a time
 * from S_snapshot[n,h], each step the update of kda_decode_step; o[t,n,h]
 * is written for every drafted token, and S_commit[n,h] receives the state
 * after the first accepted[n] of them (a copy of S_snapshot[n,h] when
 * accepted[n] == 0).  S_snapshot is only read.
 *
 *   q, k, z  [n_draft,N,H,dk] in_dtype     v [n_draft,N,H,dv] in_dtype
 *   beta     [n_draft,N,H] in_dtype        A [H,dk] fp32
 *   S_snapshot [N,H,dk,dv] fp32 (read)     accepted [N] int32, device memory,
 *                                          values clamped to [0, n_draft]
 *   o        [n_draft,N,H,dv] o_dtype (written)
 *   S_commit [N,H,dk,dv] fp32 (written)
 * n_draft >= 0 (0: the snapshot is copied to S_commit).  o and S_commit must
 * not overlap any input or each other (KDA_ERR_ALIAS).  Alignment: 16 bytes
 * for q, k, v, z, A, S_snapshot, o, S_commit; 4 bytes for accepted; beta
 * element-aligned.
 */
kda_status kda_decode_replay(const void* q, const void* k, const void* v,
                             const void* z, const void* beta, kda_dtype in_dtype,
                             const float* A, float g_min, const float* S_snapshot,
                             const int* accepted, void* o, kda_dtype o_dtype,
                             float* S_commit, int n_draft, int N, int H, int dk,
                             int dv, float scale, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
