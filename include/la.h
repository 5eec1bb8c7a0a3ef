/*
 * la.h -- C ABI of liblachunk: chunkwise gated-delta linear attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes causal linear attention generalised to the gated
 * delta rule.  For one (batch b, head h) with a dk x dv state S:
 *
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                      (state after token t's update)
 *
 * with alpha_t = exp(log_alpha_t).  The rule combines the delta rule's
 * erase-then-write with a scalar decay of the whole state ("Gated DeltaNet"
 * and "Fast Weight Programmers与DeltaNet" in the hybrid-attention notes
 * "混合注意力学习(1): 线性注意力"; "继续改进：GDN" in the lecture notes
 * "【CS336】lecture4 线性注意力|Mamba|GDN|DSA").  Four modes:
 *
 *   LA_MODE_LINEAR        S_t = S_{t-1} + k_t v_t^T  (no feature map, no
 *                         normaliser -- the numerator-only form of
 *                         "线性注意力" in the hybrid-attention notes and of
 *                         "The Devil in Linear Transformer" in
 *                         "LinearAttention 概述")
 *   LA_MODE_DELTA         alpha_t = 1
 *   LA_MODE_GATED_DELTA   the full rule
 *   LA_MODE_GATED_LINEAR  S_t = alpha_t S_{t-1} + k_t v_t^T: linear
 *                         attention with the scalar state decay and no
 *                         erase (the weight decay attributed to Mamba2 in
 *                         "Gated DeltaNet" of the hybrid-attention notes;
 *                         the gated state update of "继续改进：Mamba" in the
 *                         lecture notes)
 *
 * No scaling, activation, feature map, denominator or output norm is applied
 * inside the op; the caller prepares q, k, beta and log_alpha.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer into memory the caller owns;
 *   tensors are dense, row-major (C order), with no padding, and at least
 *   16-byte aligned.
 * - Per-token tensors are laid out [B, H, L, d]; gates [B, H, L]; states
 *   [B, H, dk, dv].  The decode step drops the L axis.
 * - `dtype` selects the element types of q, k, v and out (la_dtype_t):
 *   float32 throughout, bfloat16 throughout (output rounded to nearest
 *   even), or bfloat16 inputs with a float32 output.  Gates and states are
 *   always float32; products accumulate in float32 and the state is carried
 *   in float32.  With bf16 inputs every float intermediate that feeds a
 *   bf16 matrix product is split into two bf16 terms, so the only roundings
 *   beyond float are the bf16 inputs themselves, one bf16 copy of each
 *   chunk's triangular factor T = (I + A)^-1, and the output (when it is
 *   bf16).
 * - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *   enqueued asynchronously; the call returns without synchronising.
 * - Return value: LA_OK or an la_status_t error code.  Argument errors are
 *   detected before anything is enqueued and leave all outputs untouched.
 *   A failed launch returns LA_ERR_HIP.  Faults during
 *   execution surface at the caller's next synchronisation.
 *   la_last_error() returns a message for the last non-OK return on the
 *   calling thread.
 * - The library allocates no memory and keeps no pointer after a call
 *   returns.  Scratch space, where a call needs any, is a caller-provided
 *   device workspace whose size la_chunk_workspace_bytes() reports; calls
 *   that run concurrently need separate workspaces.
 */
#ifndef LA_H_
#define LA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LA_MODE_LINEAR = 0,
  LA_MODE_DELTA = 1,
  LA_MODE_GATED_DELTA = 2,
  LA_MODE_GATED_LINEAR = 3
} la_mode_t;

/* Element types of (q, k, v) and of out.  LA_DTYPE_BF16_F32OUT takes bf16
 * inputs and writes a float32 output (no output rounding to bf16). */
typedef enum {
  LA_DTYPE_F32 = 0,         /* q, k, v float32; out float32 */
  LA_DTYPE_BF16 = 1,        /* q, k, v bf16;    out bf16    */
  LA_DTYPE_BF16_F32OUT = 2  /* q, k, v bf16;    out float32 */
} la_dtype_t;

/* Steps in front of and behind the op that the fused entry points
 * (la_chunk_fwd_fused, la_decode_step_fused) take inside; flags, OR-ed.
 * LA_PRO_GATES: the gate arguments are raw scores a, b and the op uses
 *   beta = sigmoid(b) and log_alpha = -gate_scale * softplus(a), with
 *   softplus(a) = log(1 + e^a) -- a write strength in (0, 1) from an
 *   activation, as for the delta rule's learning-rate network ("Fast Weight
 *   Programmers与DeltaNet" in the hybrid-attention notes), and a decay in
 *   (0, 1) from a non-negative rate, the Mamba2-style gate ("Gated DeltaNet"
 *   there; "继续改进：Mamba" in the lecture notes).
 * LA_PRO_QK_L2NORM: q and k are used as x / sqrt(|x|^2 + 1e-6) per token:
 *   the delta rule replaces a stored value exactly only for unit keys
 *   ("Fast Weight Programmers与DeltaNet").
 * LA_EPI_DSKIP: o_t += D * v_t per channel, D [H, dv] float32 -- the term in
 *   v that Mamba adds to the output next to the state's read-out, a
 *   residual path around the state ("继续改进：Mamba" in the lecture notes).
 * LA_EPI_OUT_NORM: then o_t = o_t / sqrt(mean over dv of o_t^2 + norm_eps)
 *   * w per (token, head), w [H, dv] float32 (NULL: ones) -- the output
 *   normalisation that replaces linear attention's denominator ("The Devil
 *   in Linear Transformer" in "LinearAttention 概述").  In the chunkwise
 *   forward it is a second pass over out (the chain kernels own 16 columns
 *   of a row each); a bf16 out is normalised from its rounded values. */
typedef enum {
  LA_PRO_GATES = 1,
  LA_PRO_QK_L2NORM = 2,
  LA_EPI_DSKIP = 4,
  LA_EPI_OUT_NORM = 8
} la_fused_flag_t;

/* Options of the fused entry points; a NULL pointer to it means none. */
typedef struct {
  int flags;                 /* la_fused_flag_t bits                       */
  float gate_scale;          /* LA_PRO_GATES in a decayed mode: > 0        */
  const float* dskip;        /* LA_EPI_DSKIP: D [H, dv], DEVICE            */
  const float* norm_weight;  /* LA_EPI_OUT_NORM: w [H, dv], DEVICE, or NULL */
  float norm_eps;            /* LA_EPI_OUT_NORM: > 0                       */
} la_fused_opts_t;

/* Longest sequence (L) or packed batch (T), in tokens, that any entry point
 * takes: 2^31 - 1025, so that a length rounded up to the largest row block
 * the kernels walk (1024 tokens) still fits a 32-bit signed index. */
#define LA_MAX_TOKENS 2147482623

typedef enum {
  LA_OK = 0,
  LA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  LA_ERR_SHAPE = 2,       /* non-positive size, sizes past the grid limit,
                             or a length above LA_MAX_TOKENS             */
  LA_ERR_UNSUPPORTED = 3, /* (dk, dv, C, dtype, mode) outside the built set  */
  LA_ERR_ALIAS = 4,       /* an output overlaps an input (see each call)     */
  LA_ERR_HIP = 5,         /* HIP launch failure                              */
  LA_ERR_WORKSPACE = 6    /* workspace missing, too small or misaligned      */
} la_status_t;

/*
 * la_chunk_fwd -- chunkwise-parallel forward over whole sequences (prefill /
 * training form).
 *
 * Computes o[b,h,t,:] = S_t^T q_t for t = 0..L-1 and the final state S_L for
 * every (b, h), starting from S0.  The sequence is cut into chunks of C
 * tokens; inside a chunk the masked products are used, across chunks the
 * state is carried.  The chunkwise form is exact -- C changes rounding only,
 * not the result ("FLASH" in "LinearAttention 概述"; "FWP分块并行机制" in
 * the hybrid-attention notes).  The delta modes use the inductive
 * redefinition of the per-token update vectors (WY/UT representation,
 * "重新定义降低内存占用" and "HouseHolder变换和WY表示" in the hybrid-attention
 * notes) so no intermediate state is stored per token.
 *
 *   q          [B, H, L, dk]  dtype          queries
 *   k          [B, H, L, dk]  dtype          keys
 *   v          [B, H, L, dv]  dtype          values
 *   log_alpha  [B, H, L]      float32        log of the decay (<= 0);
 *                                            required for GATED_DELTA and
 *                                            GATED_LINEAR, ignored (may be
 *                                            NULL) otherwise
 *   beta       [B, H, L]      float32        write strength; required for
 *                                            DELTA and GATED_DELTA, ignored
 *                                            (may be NULL) for LINEAR and
 *                                            GATED_LINEAR
 *   S0         [B, H, dk, dv] float32        initial state; NULL = zeros
 *   out        [B, H, L, dv]  dtype          output (written)
 *   S_final    [B, H, dk, dv] float32        final state (written); may be
 *                                            NULL; may equal S0 (in-place)
 *   B, H, L, dk, dv, C        sizes; L need not be a multiple of C: the
 *                             last chunk then holds L mod C tokens
 *   mode       la_mode_t;  dtype  la_dtype_t
 *   workspace  device scratch of workspace_bytes bytes, 16-byte aligned,
 *              at least what la_chunk_workspace_bytes() reports for the same
 *              arguments; may be NULL when that is 0.  Its contents on entry
 *              are ignored and on return are unspecified.  The bf16 delta
 *              modes keep each chunk's T factor there (B*H*ceil(L/C) *
 *              6 KiB: T as bf16 operand fragments); float inputs need none,
 *              nor do the modes without erase (LINEAR, GATED_LINEAR)
 *              unless the call runs sequence-parallel (below).
 *   stream     hipStream_t
 *
 * With bf16 inputs and few long sequences -- too few (b, h, 16-column)
 * state tiles to occupy every compute unit -- the call runs each sequence
 * as P segments in parallel (la_chunk_fwd_segmented), P chosen from the
 * sizes alone (la_chunk_segments); the workspace then also holds three
 * float arrays of B*H*P*dk*dv.  The result differs from the P = 1 walk by
 * rounding only.
 *
 * Supported: dk = dv in {64, 128}, C = 64, all dtypes, all modes.
 * Aliasing: S_final == S0 is allowed; any other overlap of out or S_final
 * with an input, or of out with S_final, returns LA_ERR_ALIAS, as does a
 * workspace that overlaps any tensor argument.  A missing, short or
 * misaligned workspace returns LA_ERR_WORKSPACE.
 */
int la_chunk_fwd(const void* q, const void* k, const void* v,
                 const float* log_alpha, const float* beta, const float* S0,
                 void* out, float* S_final, int B, int H, int L, int dk,
                 int dv, int C, int mode, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * la_chunk_fwd_noalloc -- la_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments without the
 * workspace, the same kernels and results.  The scratch la_chunk_fwd keeps
 * in its workspace lives instead in a static device array of the library,
 * LA_NOALLOC_SCRATCH_BYTES (128 MiB) per GPU, held from the library's first
 * use on that GPU until the process ends; its address is looked up once per
 * device (hipGetSymbolAddress) on the first call there.  Nothing is
 * allocated: no hipMalloc / hipFree / torch allocation in the call.
 *
 * Limit: a call whose la_chunk_workspace_bytes() exceeds
 * LA_NOALLOC_SCRATCH_BYTES returns LA_ERR_WORKSPACE before anything is
 * enqueued (e.g. B*H*ceil(L/C) above 21,845 chunk-heads in the bf16 delta
 * modes); use la_chunk_fwd with a workspace for those.
 *
 * Every call on one GPU shares that GPU's array, and the array keeps the
 * last call's contents: each call writes every scratch byte it reads before
 * reading it, so nothing needs clearing, but calls that overlap in time on
 * one GPU (two streams, two host threads) race on it -- serialise them.
 * Errors as la_chunk_fwd, plus LA_ERR_HIP if the array's address cannot be
 * obtained.
 */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int la_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                         const float* log_alpha, const float* beta, const float* S0,
                         void* out, float* S_final, int B, int H, int L, int dk,
                         int dv, int C, int mode, int dtype, void* stream);

/*
 * la_chunk_workspace_bytes -- size of the workspace la_chunk_fwd needs for
 * these sizes, mode and dtype, written to *bytes (0 if it needs none).
 * Validates the same shape, mode and dtype rules as la_chunk_fwd and
 * returns the same error codes; LA_ERR_NULL for a NULL bytes.
 */
int la_chunk_workspace_bytes(int B, int H, int L, int dk, int dv, int C,
                             int mode, int dtype, size_t* bytes);

/*
 * la_chunk_fwd_fused -- la_chunk_fwd with the steps in front of and behind
 * the op done inside it (la_fused_flag_t in opts->flags): raw gate scores
 * (LA_PRO_GATES), unnormalised q and k (LA_PRO_QK_L2NORM), the residual in
 * v (LA_EPI_DSKIP) and the output norm (LA_EPI_OUT_NORM).  The result is
 * la_chunk_fwd's on the prepared inputs followed by the epilogue, except
 * that q and k are normalised in float32 and never rounded to bf16 after
 * normalisation.
 *
 *   a_raw      [B, H, L] float32  log_alpha as in la_chunk_fwd, or with
 *                                 LA_PRO_GATES the raw decay score a
 *   b_raw      [B, H, L] float32  beta, or with LA_PRO_GATES the raw score b
 *   opts       la_fused_opts_t or NULL; LA_PRO_GATES is ignored in LINEAR
 *              mode (no gates); NULL or flags = 0 is exactly la_chunk_fwd
 *   workspace  at least la_chunk_fused_workspace_bytes() for the same
 *              arguments: la_chunk_fwd's, then with a prologue flag four
 *              float32 arrays of B*H*L (the gates and the logs of the
 *              inverse norms of q and k, written by the T-solve kernel and
 *              read by the chain)
 *   everything else as in la_chunk_fwd (sequence-parallel plan included);
 *              dskip and norm_weight count as inputs for the alias rules
 *
 * Supported: bf16 inputs (LA_DTYPE_BF16, LA_DTYPE_BF16_F32OUT) when any
 * flag is set, else LA_ERR_UNSUPPORTED; unknown flags, a bad gate_scale or
 * norm_eps: LA_ERR_UNSUPPORTED; LA_EPI_DSKIP with a NULL dskip:
 * LA_ERR_NULL.  With LA_PRO_QK_L2NORM the inverse norms ride in the decay
 * tables of the chain kernels (LINEAR and DELTA run their decayed kernels
 * with log alpha = 0): no extra pass over q or k.
 */
int la_chunk_fwd_fused(const void* q, const void* k, const void* v,
                       const float* a_raw, const float* b_raw, const float* S0,
                       void* out, float* S_final, int B, int H, int L, int dk,
                       int dv, int C, int mode, int dtype,
                       const la_fused_opts_t* opts, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * la_chunk_fused_workspace_bytes -- workspace size for la_chunk_fwd_fused
 * with these sizes, mode, dtype and options, written to *bytes.  Same checks
 * and error codes; LA_ERR_NULL for a NULL bytes.
 */
int la_chunk_fused_workspace_bytes(int B, int H, int L, int dk, int dv, int C,
                                   int mode, int dtype,
                                   const la_fused_opts_t* opts, size_t* bytes);

/*
 * la_chunk_fwd_segmented -- la_chunk_fwd with each (b, h) sequence cut into
 * `segments` chunk-aligned pieces that run in parallel (sequence-parallel
 * forward).
 *
 * The state after any run of chunks is an affine function of the state
 * before it, S_end = M S_start + X, because every token's update is linear
 * in the state; the chunkwise form is exact for any cut of the sequence
 * ("FLASH" and "Lightning Attention" in "LinearAttention 概述": the output
 * splits into an intra-block part and an inter-block part carried by the
 * state).  The call therefore runs three steps on `stream`:
 *   1. every segment but the last from its local start (S0 for the first,
 *      zero otherwise) to its end state X_p, and, in the delta modes, every
 *      inner segment's transition M_p (dk x dk, the same walk with V = 0
 *      from the identity); without erase M_p is exp(sum of log_alpha over
 *      the segment) times the identity;
 *   2. a scan over the segments: S_in(0) = S0, S_in(1) = X_0, S_in(p+1) =
 *      M_p S_in(p) + X_p, in float32;
 *   3. every segment from S_in(p), writing its outputs; the last segment
 *      writes S_final.
 * The segments are balanced: segment p holds chunks floor(p n / P) ..
 * floor((p+1) n / P) - 1 of the n = ceil(L/C) chunks.  The work grows (step
 * 1 is extra), the serial depth shrinks from n to about 2 n / P chunk steps.
 *
 *   segments   P, 1 <= P <= min(ceil(L/C), 1024); P = 1 is la_chunk_fwd's
 *              whole-sequence walk; P > 1 needs bf16 inputs (dtype
 *              LA_DTYPE_BF16 or LA_DTYPE_BF16_F32OUT), else
 *              LA_ERR_UNSUPPORTED; out of range: LA_ERR_SHAPE
 *   workspace  at least la_chunk_segmented_workspace_bytes() for the same
 *              arguments: the T factors as in la_chunk_fwd, then X, M and
 *              S_in (3 * B*H*P*dk*dv float32) when P > 1
 *   everything else as in la_chunk_fwd, including the aliasing rules
 *              (S_final == S0 is allowed: S0 is read only by steps 1 and 2)
 */
int la_chunk_fwd_segmented(const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta,
                           const float* S0, void* out, float* S_final, int B,
                           int H, int L, int dk, int dv, int C, int mode,
                           int dtype, int segments, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * la_chunk_segmented_workspace_bytes -- workspace size for
 * la_chunk_fwd_segmented with these arguments, written to *bytes.  Same
 * checks and error codes; LA_ERR_NULL for a NULL bytes.
 */
int la_chunk_segmented_workspace_bytes(int B, int H, int L, int dk, int dv,
                                       int C, int mode, int dtype,
                                       int segments, size_t* bytes);

/*
 * la_chunk_segments -- the segment count la_chunk_fwd uses for these sizes,
 * mode and dtype, written to *segments (1: the whole-sequence walk).  It
 * depends on the arguments only, never on the data or the device.  Same
 * checks and error codes as la_chunk_workspace_bytes; LA_ERR_NULL for a
 * NULL segments.
 */
int la_chunk_segments(int B, int H, int L, int dk, int dv, int C, int mode,
                      int dtype, int* segments);

/*
 * la_chunk_fwd_varlen -- la_chunk_fwd over a packed batch of N independent
 * sequences of different lengths (the same method per sequence: each has its
 * own initial and final state, and no token sees another sequence's).
 *
 * The sequences are concatenated along one token axis of T tokens;
 * sequence s holds tokens cu_seqlens[s] .. cu_seqlens[s+1] - 1.  Every
 * sequence is cut into chunks of C from its own start, so its last chunk may
 * be partial; an empty sequence leaves its state unchanged
 * (S_final = S0).
 *
 *   q          [H, T, dk]     dtype          queries (per head, tokens of all
 *                                            sequences back to back)
 *   k          [H, T, dk]     dtype
 *   v          [H, T, dv]     dtype
 *   log_alpha  [H, T]         float32        as in la_chunk_fwd
 *   beta       [H, T]         float32        as in la_chunk_fwd
 *   S0         [N, H, dk, dv] float32        initial states; NULL = zeros
 *   out        [H, T, dv]     dtype          output (written)
 *   S_final    [N, H, dk, dv] float32        final states (written); may be
 *                                            NULL; may equal S0
 *   cu_seqlens [N + 1]        int32 DEVICE   offsets: 0 = cu_seqlens[0] <=
 *                                            ... <= cu_seqlens[N] = T
 *   N, H, T, dk, dv, C        N >= 1, T >= 0; sizes as in la_chunk_fwd
 *   mode, dtype, workspace, workspace_bytes, stream   as in la_chunk_fwd;
 *              the workspace size comes from la_chunk_varlen_workspace_bytes
 *              (bf16 delta modes: H * (ceil(T/C) + N) * 6 KiB, whatever the
 *              offsets)
 *
 * The offsets are read on the device and cannot be validated before the
 * launch: offsets that are not nondecreasing within [0, T] give unspecified
 * results, but every access stays inside the tensors (they are clamped).
 * Aliasing: as in la_chunk_fwd, with cu_seqlens counted as an input.
 */
int la_chunk_fwd_varlen(const void* q, const void* k, const void* v,
                        const float* log_alpha, const float* beta,
                        const float* S0, void* out, float* S_final,
                        const int* cu_seqlens, int N, int H, int T, int dk,
                        int dv, int C, int mode, int dtype, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * la_chunk_varlen_workspace_bytes -- workspace size for la_chunk_fwd_varlen
 * with these sizes, mode and dtype, written to *bytes.  Same checks and
 * error codes; LA_ERR_NULL for a NULL bytes.
 */
int la_chunk_varlen_workspace_bytes(int N, int H, int T, int dk, int dv, int C,
                                    int mode, int dtype, size_t* bytes);

/*
 * la_noncausal_fwd -- the bidirectional (non-causal) form of linear
 * attention: every token reads the state after the whole sequence,
 *     S = S0 + sum_t k_t v_t^T,   o_t = S^T q_t   (O = Q (K^T V)),
 * by the associativity of the matrix products: two products in linear time
 * with no causal mask ("快速预览" in "LinearAttention 概述": enough for
 * bidirectional models, no kernel needed).  S is accumulated by the LINEAR-mode chain kernel
 * over parallel segments of the sequence, the segments' partial states are
 * summed in a fixed order, then O = Q S on MFMA with S split into bf16
 * hi + lo operands.
 *
 *   q, k, v    [B, H, L, d]   bf16 (dtype LA_DTYPE_BF16 or _BF16_F32OUT)
 *   S0         [B, H, d, d]   float32 or NULL (zeros)
 *   out        [B, H, L, d]   bf16 / float32 (written)
 *   S_final    [B, H, d, d]   float32 (written: S) or NULL; may equal S0
 *   B, H, L, dk, dv  dk = dv in {64, 128}, L >= 1
 *   workspace  at least la_noncausal_workspace_bytes() bytes, 16-byte
 *              aligned (the segments' partial states and S)
 * Errors as la_chunk_fwd; float inputs return LA_ERR_UNSUPPORTED.
 */
int la_noncausal_fwd(const void* q, const void* k, const void* v,
                     const float* S0, void* out, float* S_final, int B, int H,
                     int L, int dk, int dv, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/* la_noncausal_workspace_bytes -- workspace size for la_noncausal_fwd with
 * these sizes and dtype, written to *bytes; same checks. */
int la_noncausal_workspace_bytes(int B, int H, int L, int dk, int dv,
                                 int dtype, size_t* bytes);

/*
 * la_chunk_bwd -- gradients of la_chunk_fwd (training): for upstream
 * gradients grad_out of the outputs and grad_S_final of the final state,
 * the gradients of sum(grad_out * out) + sum(grad_S_final * S_final) with
 * respect to q, k, v, log_alpha, beta and S0.
 *
 * The pages print no gradient formulas; training runs the chunked form and
 * keeps the state entering every chunk for the backward ("FWP分块并行机制"
 * in the hybrid-attention notes; train with the parallel form: "朴素线性注意力"
 * in the lecture notes).  The call differentiates the forward's chunk step
 * (WY/UT form, "HouseHolder变换和WY表示"; scalar decay, "Gated DeltaNet"):
 * a per-chunk prep kernel (decays, T, and the two products that do not
 * depend on the state gradient, P^T dO and Q^T diag(gam) dO), a forward walk
 * storing each chunk's entry state and U = T R, a reverse walk over chunks
 * carrying the state gradient (dU = P^T dO + diag(f) K dS', dR = T^T dU,
 * dS = gam_C dS' + Q^T diag(gam) dO - K^T diag(beta gam) dR), and a
 * parallel per-chunk kernel for dq, dk, dbeta and dlog_alpha.
 *
 *   q, k, v         [B, H, L, d]   dtype (LA_DTYPE_F32 or LA_DTYPE_BF16)
 *   log_alpha, beta [B, H, L]      float32, as in la_chunk_fwd (NULL where
 *                                  the mode does not read them)
 *   S0              [B, H, d, d]   float32 or NULL (zeros)
 *   grad_out        [B, H, L, d]   dtype (the type of la_chunk_fwd's out)
 *   grad_S_final    [B, H, d, d]   float32 or NULL (zeros)
 *   grad_q, grad_k, grad_v [B, H, L, d]  float32 (written)
 *   grad_log_alpha  [B, H, L]      float32 (written; required in the gated
 *                                  modes, else ignored and may be NULL)
 *   grad_beta       [B, H, L]      float32 (written; required in the delta
 *                                  modes, else ignored and may be NULL)
 *   grad_S0         [B, H, d, d]   float32 (written) or NULL
 *   B, H, L, dk, dv, C   dk = dv in {64, 128}, C = 64, any L >= 1 (the
 *                        last chunk may be partial)
 *   workspace       at least la_chunk_bwd_workspace_bytes() bytes, 16-byte
 *                   aligned: per chunk the entry state, the gradient of the
 *                   leaving state and Q^T diag(gam) dO (3 d^2 floats) and
 *                   T^T (C^2 floats); per token U, dR and P^T dO (3 d floats)
 *                   and g
 * Errors as la_chunk_fwd: missing required pointers LA_ERR_NULL; shapes
 * LA_ERR_SHAPE / LA_ERR_UNSUPPORTED (also LA_DTYPE_BF16_F32OUT); any overlap
 * between an output and an input, another output or the workspace
 * LA_ERR_ALIAS.  Gradients of bf16 inputs are accumulated in float32 with
 * float operands split into bf16 hi + lo parts.
 */
int la_chunk_bwd(const void* q, const void* k, const void* v,
                 const float* log_alpha, const float* beta, const float* S0,
                 const void* grad_out, const float* grad_S_final, float* grad_q,
                 float* grad_k, float* grad_v, float* grad_log_alpha,
                 float* grad_beta, float* grad_S0, int B, int H, int L, int dk,
                 int dv, int C, int mode, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream);

/* la_chunk_bwd_workspace_bytes -- workspace size for la_chunk_bwd with these
 * sizes, mode and dtype, written to *bytes; same shape checks. */
int la_chunk_bwd_workspace_bytes(int B, int H, int L, int dk, int dv, int C,
                                 int mode, int dtype, size_t* bytes);

/*
 * la_chunk_bwd_varlen -- la_chunk_bwd for a packed batch of N variable-length
 * sequences, the gradients of la_chunk_fwd_varlen: tokens laid out as there
 * (q, k, v, grad_out and the token gradients [H, T, d]; gates and their
 * gradients [H, T]; S0, grad_S_final, grad_S0 [N, H, d, d]), with
 * cu_seqlens [N + 1] int32 on the device (sequence s is tokens
 * cu_seqlens[s] .. cu_seqlens[s+1] - 1; the kernels clamp the offsets as
 * la_chunk_fwd_varlen does).  Each sequence's gradients equal those of
 * la_chunk_bwd on that sequence alone; an empty sequence passes grad_S_final
 * to grad_S0.  Workspace: la_chunk_bwd_varlen_workspace_bytes(), the
 * per-chunk arrays sized for H (ceil(T / C) + N) chunk slots.  Errors as
 * la_chunk_bwd, plus LA_ERR_NULL for a NULL cu_seqlens.
 */
int la_chunk_bwd_varlen(const void* q, const void* k, const void* v,
                        const float* log_alpha, const float* beta, const float* S0,
                        const void* grad_out, const float* grad_S_final,
                        const int* cu_seqlens, float* grad_q, float* grad_k,
                        float* grad_v, float* grad_log_alpha, float* grad_beta,
                        float* grad_S0, int N, int H, int T, int dk, int dv, int C,
                        int mode, int dtype, void* workspace, size_t workspace_bytes,
                        void* stream);

/* la_chunk_bwd_varlen_workspace_bytes -- workspace size for la_chunk_bwd_varlen
 * with these sizes, mode and dtype (whatever the offsets), written to *bytes. */
int la_chunk_bwd_varlen_workspace_bytes(int N, int H, int T, int dk, int dv, int C,
                                        int mode, int dtype, size_t* bytes);

/*
 * la_chunk_bwd_fused -- the gradients of la_chunk_fwd_fused with respect to
 * its raw inputs, for the prologue's flags: with LA_PRO_QK_L2NORM q and k are
 * the unnormalised vectors and grad_q, grad_k their gradients; with
 * LA_PRO_GATES a_raw and b_raw are the raw gate scores and grad_a, grad_b
 * their gradients (da = -gate_scale sigmoid(a) dlog_alpha, db = sigmoid(b)
 * (1 - sigmoid(b)) dbeta; for x_hat = x / sqrt(|x|^2 + 1e-6), dx = (dx_hat -
 * x_hat (x_hat . dx_hat)) / sqrt(|x|^2 + 1e-6)).  A prologue kernel writes the
 * inverse norms and the activated gates into the workspace, the backward's
 * kernels read the raw q and k with the norms as per-row factors (the
 * normalised rows are never rounded to bf16), and a last kernel applies the
 * chain rule in place.  Arguments, layouts and errors as
 * la_chunk_bwd (a_raw, b_raw in place of log_alpha, beta; grad_a, grad_b in
 * place of their gradients); opts as la_chunk_fwd_fused, where the epilogue
 * flags (LA_EPI_DSKIP, LA_EPI_OUT_NORM) return LA_ERR_UNSUPPORTED: their
 * backward is not built.  NULL opts or flags = 0 is la_chunk_bwd.
 *   workspace  at least la_chunk_bwd_fused_workspace_bytes() bytes, 16-byte
 *              aligned: the inverse norms of q and k, the activated
 *              gates, then la_chunk_bwd's workspace
 */
int la_chunk_bwd_fused(const void* q, const void* k, const void* v,
                       const float* a_raw, const float* b_raw, const float* S0,
                       const void* grad_out, const float* grad_S_final, float* grad_q,
                       float* grad_k, float* grad_v, float* grad_a, float* grad_b,
                       float* grad_S0, int B, int H, int L, int dk, int dv, int C,
                       int mode, int dtype, const la_fused_opts_t* opts, void* workspace,
                       size_t workspace_bytes, void* stream);

/* la_chunk_bwd_fused_workspace_bytes -- workspace size for la_chunk_bwd_fused
 * with these sizes, mode, dtype and options, written to *bytes. */
int la_chunk_bwd_fused_workspace_bytes(int B, int H, int L, int dk, int dv, int C,
                                       int mode, int dtype, const la_fused_opts_t* opts,
                                       size_t* bytes);

/*
 * la_decode_step -- one token of the recurrence for B*H independent states
 * (decode / inference form), updating the state in place.
 *
 * For every (b, h): reads S, applies the mode's update with this token's
 * (q, k, v, beta, log_alpha) and writes S back, then o = S_new^T q.  The
 * erase term is evaluated as k (k^T S) -- the read k^T S first -- so a step
 * costs O(dk dv), not O(dk^2 dv) ("继续改进：GDN" in the lecture notes).  The
 * recurrent form is the inference path of the same method ("朴素线性注意力"
 * in the lecture notes; "Prefill、Decode与KVCache" in the hybrid-attention
 * notes): S after la_chunk_fwd is the S of the first decode step.
 *
 *   q, k       [B, H, dk]     dtype
 *   v          [B, H, dv]     dtype
 *   log_alpha  [B, H]         float32  (GATED_DELTA, GATED_LINEAR; else
 *                                       may be NULL)
 *   beta       [B, H]         float32  (DELTA, GATED_DELTA; else may be NULL)
 *   S          [B, H, dk, dv] float32  state, read and overwritten in place
 *   out        [B, H, dv]     dtype    output (written)
 *
 * Supported: dk, dv in {64, 128} (independently), both dtypes, all modes.
 * Aliasing: out must not overlap S or any input; S must not overlap q, k,
 * v or the gates (LA_ERR_ALIAS).
 */
int la_decode_step(const void* q, const void* k, const void* v,
                   const float* log_alpha, const float* beta, float* S,
                   void* out, int B, int H, int dk, int dv, int mode,
                   int dtype, void* stream);

/*
 * la_decode_step_fused -- la_decode_step with the fused steps of
 * la_chunk_fwd_fused (opts as there): a_raw and b_raw [B, H] are the raw
 * gate scores with LA_PRO_GATES; q, k are normalised inside with
 * LA_PRO_QK_L2NORM (their inverse norms folded into the step's dot products
 * and update); LA_EPI_DSKIP and LA_EPI_OUT_NORM act on the step's output
 * inside the kernel.  Both dtypes; NULL opts or flags = 0 is exactly
 * la_decode_step.  Errors as la_decode_step, plus those of the options.
 */
int la_decode_step_fused(const void* q, const void* k, const void* v,
                         const float* a_raw, const float* b_raw, float* S,
                         void* out, int B, int H, int dk, int dv, int mode,
                         int dtype, const la_fused_opts_t* opts,
                         void* stream);

/*
 * Kernel timing with HIP events (profiling aid).
 *
 * Between la_profile_begin() and la_profile_end(), every kernel the library
 * launches (from any thread) is bracketed by two HIP events recorded on the
 * stream it is launched on.  la_profile_end() waits for the recorded events,
 * then reports, per kernel name ("la_tsolve", "la_chunk", "la_decode"), the
 * number of launches and the summed event-to-event time in milliseconds,
 * and stops recording.  `out` is a host array of `capacity` entries; the
 * number of distinct kernels is written to *count (entries beyond capacity
 * are dropped).  Returns LA_ERR_HIP if an event call fails, LA_ERR_NULL for
 * a NULL count.  Timing adds one event record per launch and no host
 * synchronisation until la_profile_end().
 */
typedef struct {
  char name[32];
  int launches;
  double total_ms;
} la_kernel_time_t;

int la_profile_begin(void);
int la_profile_end(la_kernel_time_t* out, int capacity, int* count);

/* Message for the last non-OK return on the calling thread ("" if none).
 * The pointer stays valid until the next call on the same thread. */
const char* la_last_error(void);

/* Library version string, e.g. "lachunk 0.4.0 gfx950". */
const char* la_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LA_H_ */
