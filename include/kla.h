/*
 * kla.h -- C ABI of libkla.so: Kaczmarz Linear Attention (KLA) prefill and
 * decode on AMD Instinct MI355X (gfx950).
 *
 * The operation (per sequence and per head, state S in R^{dk x dv}) is the
 * gated delta rule with the Kaczmarz step size from the KLA technical
 * summary ("Resumo Tecnico: Atencao Linear Kaczmarz (KLA)",
 * gist.science/pt/paper/2605.08587), sections "Derivacao Teorica" and
 * "A Regra de Atualizacao KLA":
 *
 *     beta_t = eta_t / (k_t^T k_t + eps)
 *     S~     = alpha_t S_{t-1}
 *     e_t    = v_t - S~^T k_t
 *     S_t    = S~ + beta_t k_t e_t^T
 *     o_t    = S_t^T q_t            (read after the write)
 *
 * alpha_t is the scalar decay gate and eta_t the relaxation gate; both are
 * per (token, head).  No scaling is applied to q (callers pre-scale).
 *
 * The *_ex entry points also run the two gate variants the same kernels
 * cover: beta_t = eta_t directly (KLA_BETA_DIRECT), the learned scalar step
 * of Gated DeltaNet that KLA replaces (KLA summary, introduction), and, with
 * alpha = NULL, no decay (alpha_t = 1): with the direct step this is
 * DeltaNet ("Linear Attention Architectures: Mechanisms, Trade-offs, and
 * Cross-Layer Routing", gist.science/pt/paper/2607.07953, section "Notacao
 * Unificada", DeltaNet and Gated DeltaNet).
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers (HIP device memory) except where
 *     noted; the caller owns every buffer.  The library never allocates or
 *     frees memory and keeps no state between calls, apart from the static
 *     scratch array of kla_fwd_chunked_split_noalloc.
 *   - Tensors are dense, row-major, with the innermost dimension contiguous.
 *     Pointers to q, k, v, o and states must be 16-byte aligned.
 *   - q, k, v share one element type (kla_dtype).  alpha, eta, o and all
 *     states are fp32.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous and ordered on that stream; nothing synchronises the host.
 *   - Arguments are checked on the host before any launch.  On an error
 *     nothing is launched and no output is written.  Launch failures are
 *     reported as KLA_ERR_HIP.
 *   - Results are deterministic: repeated calls with the same inputs give
 *     bitwise identical outputs (no atomics, fixed reduction order).
 *   - Supported shapes: dk = dv in {64, 128}, chunk = 64.
 */
#ifndef KLA_H
#define KLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every enum below also names the int32 bounds (the *_RANGE_ members, never
 * valid arguments), so any int32 a C caller passes is a value of the type:
 * an unknown value reaches the library's argument checks and is rejected,
 * instead of being undefined behaviour in the C++ implementation. */
typedef enum {
    KLA_OK = 0,
    KLA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, aliasing */
    KLA_ERR_UNSUPPORTED = -2, /* valid but not implemented (dk, dv, chunk, dtype) */
    KLA_ERR_WORKSPACE = -3,   /* workspace smaller than the query returned */
    KLA_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
    KLA_STATUS_RANGE_MIN = -2147483647 - 1,
    KLA_STATUS_RANGE_MAX = 2147483647
} kla_status;

typedef enum {
    KLA_F32 = 0,  /* IEEE binary32 */
    KLA_BF16 = 1, /* bfloat16 (8-bit exponent, 7-bit mantissa) */
    KLA_DTYPE_RANGE_MIN = -2147483647 - 1,
    KLA_DTYPE_RANGE_MAX = 2147483647
} kla_dtype;

typedef enum {
    KLA_BETA_KACZMARZ = 0, /* beta_t = eta_t / (k_t^T k_t + eps)   (KLA) */
    KLA_BETA_DIRECT = 1,   /* beta_t = eta_t; eps is unused       (Gated DeltaNet) */
    KLA_BETA_RANGE_MIN = -2147483647 - 1,
    KLA_BETA_RANGE_MAX = 2147483647
} kla_beta_mode;

/*
 * Bytes of device workspace kla_fwd_chunked (and kla_fwd_chunked_ex) needs
 * for these sizes: with cu_seqlens, the order in which the sequences are
 * scheduled (longest first, one int32 per sequence, rounded up to 256 bytes)
 * for 2 .. 1024 sequences; 0 otherwise.  A dense batch (cu_seqlens NULL)
 * needs none, but callers may always pass the queried size.
 */
size_t kla_fwd_chunked_workspace_size(int32_t n_seqs, int64_t total_tok, int32_t H,
                                      int32_t dk, int32_t dv, int32_t chunk);

/*
 * Chunkwise-parallel prefill over packed sequences.
 *
 * The chunked form computes the same result as the token recurrence above
 * (up to rounding).  The KLA summary, section "Implementacao", keeps Gated
 * DeltaNet's chunk-parallel algorithm and changes only the diagonal
 * coefficient matrix B = Diag(beta_1..beta_C) of the chunk solver.
 *
 *   q, k        [total_tok, H, dk]   element type `dtype`
 *   v           [total_tok, H, dv]   element type `dtype`
 *   alpha, eta  [total_tok, H]       fp32; alpha in (0, 1], eta in [0, 1].
 *               alpha may be NULL: alpha_t = 1 for every token (no decay).
 *   cu_seqlens  device int32 [n_seqs + 1] with 0 = cu[0] <= cu[1] <= ... <=
 *               cu[n_seqs] = total_tok: sequence s is tokens [cu[s], cu[s+1]).
 *               NULL means n_seqs equal sequences of total_tok / n_seqs tokens
 *               (a dense [B, T, H, d] batch).  The contents are NOT checked on
 *               the host (that would need a synchronisation); violating the
 *               ordering above is undefined behaviour.
 *   chunk       must be 64.
 *   eps         the stabiliser in beta; eps >= 0.  With eps = 0 a zero key
 *               gives a non-finite result.
 *   initial_state [n_seqs, H, dk, dv] fp32 start state of each sequence, or
 *               NULL for zeros.
 *   o           [total_tok, H, dv] fp32, written: o_t = S_t^T q_t.
 *   final_state [n_seqs, H, dk, dv] fp32, written with each sequence's last
 *               state, or NULL.  It may be the same buffer as initial_state
 *               (in-place update); any other overlap is an error.
 *   workspace   device buffer of workspace_bytes >= the size query (may be
 *               NULL when the query returns 0, or when cu_seqlens is NULL),
 *               16-byte aligned, not overlapping any argument; contents on
 *               entry ignored, on return unspecified.  With cu_seqlens, a
 *               first launch writes the sequences' longest-first order
 *               into it and the prefill takes (sequence, head) pairs in
 *               that order, so long sequences do not start last.
 *
 * Errors: KLA_ERR_INVALID_ARG for null required pointers, misalignment,
 * n_seqs <= 0, H <= 0, total_tok < 0, total_tok not divisible by n_seqs when
 * cu_seqlens is NULL, eps < 0 or not finite, or `o` overlapping an input;
 * KLA_ERR_UNSUPPORTED for other dk/dv/chunk/dtype values; KLA_ERR_WORKSPACE
 * for a short workspace; KLA_ERR_HIP if the launch fails.
 */
kla_status kla_fwd_chunked(const void *q, const void *k, const void *v,
                           const float *alpha, const float *eta,
                           const int32_t *cu_seqlens, int32_t n_seqs, int64_t total_tok,
                           int32_t H, int32_t dk, int32_t dv, int32_t chunk, float eps,
                           kla_dtype dtype, const float *initial_state, float *o,
                           float *final_state, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * kla_fwd_chunked with the step-size rule chosen by beta_mode (arguments in
 * the same order, beta_mode after dtype).  KLA_BETA_KACZMARZ is exactly
 * kla_fwd_chunked; KLA_BETA_DIRECT uses beta_t = eta_t (eta in [0, 1] as
 * Gated DeltaNet's writing strength; eps is still range-checked but unused).
 * The chunk algorithm is unchanged: only B = Diag(beta) differs (KLA summary,
 * section "Implementacao").  Errors: as kla_fwd_chunked, plus
 * KLA_ERR_INVALID_ARG for an unknown beta_mode.
 */
kla_status kla_fwd_chunked_ex(const void *q, const void *k, const void *v,
                              const float *alpha, const float *eta,
                              const int32_t *cu_seqlens, int32_t n_seqs, int64_t total_tok,
                              int32_t H, int32_t dk, int32_t dv, int32_t chunk, float eps,
                              kla_dtype dtype, kla_beta_mode beta_mode,
                              const float *initial_state, float *o, float *final_state,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace kla_fwd_chunked_split needs: for every
 * (sequence, head), the maps (A, B) of segments 0..n_splits-2 and the start
 * states of all n_splits segments, each dk x dv fp32 (dk = dv):
 * n_seqs * H * dk * dv * 4 * (3 n_splits - 2) bytes.  0 for n_splits <= 1.
 */
size_t kla_fwd_chunked_split_workspace_size(int32_t n_seqs, int32_t H, int32_t dk, int32_t dv,
                                            int32_t n_splits);

/*
 * kla_fwd_chunked_ex with every sequence cut into n_splits segments on chunk
 * boundaries (segment p = chunks [p*c, (p+1)*c) of the sequence, c =
 * ceil(chunks / n_splits); trailing segments of short sequences may be
 * empty), for batches with too few (sequence, head) pairs to fill the GPU.
 *
 * The state map of a segment is affine, S_end = A S_start + B (the chunk
 * form of the KLA summary, section "Implementacao", is linear in the
 * chunk-start state).  Four launches on the stream:
 *   0. the A slots of the workspace are set to the identity;
 *   1. for segments 0..n_splits-2: A from the start I with V read as 0, and
 *      B from a zero start, by the prefill kernel (no output);
 *   2. a scan: S_0 = initial state (or 0), S_{p+1} = A_p S_p + B_p;
 *   3. every segment from its start state, writing o; the last segment
 *      writes final_state.
 * The result equals kla_fwd_chunked_ex up to rounding; the work is about
 * (3 - 2/n_splits) times that of one pass, spread over n_splits times as
 * many workgroups.
 *
 *   n_splits    1 .. 1024; 1 is exactly kla_fwd_chunked_ex.
 *   workspace   device buffer of at least
 *               kla_fwd_chunked_split_workspace_size(...) bytes, 16-byte
 *               aligned, not overlapping any argument.  Its contents on
 *               entry are ignored and on return are unspecified.
 * Other arguments as kla_fwd_chunked_ex.  Errors: as kla_fwd_chunked_ex,
 * plus KLA_ERR_INVALID_ARG for n_splits out of range or a workspace that
 * overlaps an argument, KLA_ERR_WORKSPACE for a short workspace.
 */
kla_status kla_fwd_chunked_split(const void *q, const void *k, const void *v,
                                 const float *alpha, const float *eta,
                                 const int32_t *cu_seqlens, int32_t n_seqs, int64_t total_tok,
                                 int32_t H, int32_t dk, int32_t dv, int32_t chunk, float eps,
                                 kla_dtype dtype, kla_beta_mode beta_mode, int32_t n_splits,
                                 const float *initial_state, float *o, float *final_state,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * Size in bytes of the device scratch array that kla_fwd_chunked_split_noalloc
 * uses in place of a caller workspace (32 MiB per GPU).
 */
#define KLA_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)

/*
 * kla_fwd_chunked_split for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operation, arguments and result, without the
 * workspace arguments.  The segment maps and start states live in a static
 * device array of KLA_NOALLOC_SCRATCH_BYTES inside the library, one copy per
 * GPU, held until the process ends.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); on its first call on a
 * device it looks up that device's copy of the array once.
 *
 *   Limit: kla_fwd_chunked_split_workspace_size(n_seqs, H, dk, dv, n_splits)
 *          must not exceed KLA_NOALLOC_SCRATCH_BYTES, else KLA_ERR_WORKSPACE
 *          and nothing is launched (for example, at dk = dv = 128 the long
 *          dense batch of 2 sequences x 16 heads allows n_splits <= 6).
 *   Sharing: every call on one GPU uses the same array, whose contents are
 *          the last call's (no call needs them cleared: each call writes
 *          every part it reads).  Calls that overlap in time on one GPU
 *          (concurrent streams, or threads) race on it and give wrong
 *          results; order them on one stream.
 * Other arguments and errors as kla_fwd_chunked_split (KLA_ERR_HIP also when
 * the array's device address cannot be obtained).
 */
kla_status kla_fwd_chunked_split_noalloc(const void *q, const void *k, const void *v,
                                         const float *alpha, const float *eta,
                                         const int32_t *cu_seqlens, int32_t n_seqs,
                                         int64_t total_tok, int32_t H, int32_t dk, int32_t dv,
                                         int32_t chunk, float eps, kla_dtype dtype,
                                         kla_beta_mode beta_mode, int32_t n_splits,
                                         const float *initial_state, float *o,
                                         float *final_state, void *stream);

/*
 * One recurrent decode step for n_seqs independent sequences: every
 * (sequence, head) state advances by one token IN PLACE, and o receives the
 * read of the new state.  It is the token recurrence above applied once,
 * written as a single pass over the state:
 *   x = S^T k, y = S^T q, e = v - alpha x, o = alpha y + beta (k^T q) e,
 *   S <- alpha S + beta k e^T.
 *
 *   q, k        [n_seqs, H, dk]      element type `dtype`
 *   v           [n_seqs, H, dv]      element type `dtype`
 *   alpha, eta  [n_seqs, H]          fp32 (alpha may be NULL: alpha = 1)
 *   state       [n_seqs, H, dk, dv]  fp32, read and updated in place
 *   o           [n_seqs, H, dv]      fp32, written
 *
 * Errors: as kla_fwd_chunked (o must not overlap state or the inputs).
 */
kla_status kla_decode_step(const void *q, const void *k, const void *v,
                           const float *alpha, const float *eta, float *state, float *o,
                           int32_t n_seqs, int32_t H, int32_t dk, int32_t dv, float eps,
                           kla_dtype dtype, void *stream);

/*
 * kla_decode_step with the step-size rule chosen by beta_mode (as in
 * kla_fwd_chunked_ex).  Errors: as kla_decode_step, plus KLA_ERR_INVALID_ARG
 * for an unknown beta_mode.
 */
kla_status kla_decode_step_ex(const void *q, const void *k, const void *v,
                              const float *alpha, const float *eta, float *state, float *o,
                              int32_t n_seqs, int32_t H, int32_t dk, int32_t dv, float eps,
                              kla_dtype dtype, kla_beta_mode beta_mode, void *stream);

/*
 * Per-channel decay (Kimi Delta Attention's gate; linear-attention survey
 * page, "Linear Attention Architectures: Mechanisms, Trade-offs, and
 * Cross-Layer Routing", section "Metodologia e Estrutura": one decay rate per
 * feature channel).  The state's rows are the key channels, so the token
 * step becomes
 *   S~ = Diag(a_t) S_{t-1},  e_t = v_t - S~^T k_t,  S_t = S~ + beta_t k_t e_t^T,
 *   o_t = S_t^T q_t,
 * with beta_t from beta_mode as in kla_fwd_chunked_ex.
 *
 *   alpha       [total_tok, H, dk] fp32, required, 16-byte aligned; every
 *               rate in (0, 1], however small.  (A chunk in which one
 *               channel's rates multiply below 2^-100 inside an aligned
 *               block of 16 tokens, or, with bf16 inputs, below 2^-200 over
 *               the chunk, takes a slower exact path.)
 * Other arguments and errors as kla_fwd_chunked_ex (whole sequences only; no
 * workspace is needed).  fp32 inputs run on the fp32 MFMA; bf16 inputs on
 * the bf16 MFMA, every fp32 factor entering as a hi/lo pair of bf16 values
 * (each product to about 2^-16 of its size), with fp32 accumulation.
 */
kla_status kla_fwd_chunked_kda(const void *q, const void *k, const void *v,
                               const float *alpha, const float *eta,
                               const int32_t *cu_seqlens, int32_t n_seqs, int64_t total_tok,
                               int32_t H, int32_t dk, int32_t dv, int32_t chunk, float eps,
                               kla_dtype dtype, kla_beta_mode beta_mode,
                               const float *initial_state, float *o, float *final_state,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step with the per-channel decay (the step above, once):
 *   x = S^T (a o k), y = S^T (a o q), e = v - x, o = y + beta (k^T q) e,
 *   S <- Diag(a) S + beta k e^T.
 *   alpha       [n_seqs, H, dk] fp32, required, 16-byte aligned.
 * Other arguments and errors as kla_decode_step_ex.
 */
kla_status kla_decode_step_kda(const void *q, const void *k, const void *v,
                               const float *alpha, const float *eta, float *state, float *o,
                               int32_t n_seqs, int32_t H, int32_t dk, int32_t dv, float eps,
                               kla_dtype dtype, kla_beta_mode beta_mode, void *stream);

/*
 * Curvature-conditioned read ("Don't Read Everything: A Curvature-Conditioned
 * Query for Linear Attention", sections "Derivacao Teorica", "O Mecanismo"
 * and "Integracao").  Only the read changes: with Sigma_t the covariance of
 * the keys j <= t of the sequence, weighted uniformly (the Hessian at q = 0
 * of log sum_j exp(k_j^T q)),
 *   q_clean_t = q_t - lambda_t Sigma_t q_t,   o_t = S_t^T q_clean_t,
 *   Sigma_t q = P_t q / n_t - m_t (m_t . q) / n_t^2,
 *   P_t = sum_{j<=t} k_j k_j^T,  m_t = sum_{j<=t} k_j,  n_t = number of keys.
 * The running sums are the extra state per (sequence, head): one record of
 * kla_ccq_state_floats(dk) = dk*dk + dk + 4 fp32, [P row-major | m | n | pad].
 * n is held in fp32 (exact up to 2^24 keys).
 */
size_t kla_ccq_state_floats(int32_t dk);

/* Workspace bytes of kla_fwd_chunked_ccq: the cleaned queries (bf16 inputs:
 * a bf16 hi and lo pair, plus total_tok x H x dv fp32 of scratch for the
 * cleaning pass; fp32 inputs: fp32), 256-byte rounded parts.  0 when
 * total_tok <= 0. */
size_t kla_fwd_chunked_ccq_workspace_size(int64_t total_tok, int32_t H, int32_t dk, int32_t dv,
                                          kla_dtype dtype);

/*
 * Prefill with the curvature-conditioned read.  Launches on the stream:
 *   1. the query cleaning for every token (chunked: Q P + lower(Q K^T) K,
 *      the running sums carried over chunks) into the workspace;
 *      For bf16 inputs the cleaned query is written as a bf16 hi and lo
 *      pair, and sequences of at least ceil((dk*dk + dk + 4) / dk) tokens
 *      are cleaned as two halves in parallel: a first launch leaves the
 *      running sums of the first halves in the scratch part of the
 *      workspace (each sequence in its own token rows), a second cleans
 *      both halves;
 *   2. bf16 inputs: one bf16 prefill reading with both parts of the
 *      cleaned query, o = S^T (q_hi + q_lo), which writes the end state;
 *      fp32 inputs: the fp32 prefill reading with the fp32 cleaned query.
 *   lambda      [total_tok, H] fp32, the contraction gate (any real value).
 *   ccq_in      [n_seqs, H, kla_ccq_state_floats(dk)] fp32 start sums, or NULL
 *               for zero (a sequence that starts here).
 *   ccq_out     same shape, written with the end sums, or NULL.  It must not
 *               overlap any other argument (ccq_in included).
 *   workspace   >= kla_fwd_chunked_ccq_workspace_size(...) bytes, 16-byte
 *               aligned, overlapping nothing; contents unspecified on return.
 * Other arguments as kla_fwd_chunked_ex.  Errors: as kla_fwd_chunked_ex,
 * plus KLA_ERR_INVALID_ARG for a null lambda or an overlapping ccq_out,
 * KLA_ERR_WORKSPACE for a short workspace.
 */
kla_status kla_fwd_chunked_ccq(const void *q, const void *k, const void *v,
                               const float *alpha, const float *eta, const float *lambda,
                               const int32_t *cu_seqlens, int32_t n_seqs, int64_t total_tok,
                               int32_t H, int32_t dk, int32_t dv, int32_t chunk, float eps,
                               kla_dtype dtype, kla_beta_mode beta_mode,
                               const float *initial_state, const float *ccq_in, float *o,
                               float *final_state, float *ccq_out, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Workspace bytes of kla_decode_step_ccq: the fp32 cleaned query per
 * (sequence, head), rounded to 256. */
size_t kla_decode_step_ccq_workspace_size(int32_t n_seqs, int32_t H, int32_t dk);

/*
 * One decode step with the curvature-conditioned read: ccq_state [n_seqs, H,
 * kla_ccq_state_floats(dk)] takes the new key (in place), the cleaned query
 * goes to the workspace, and the decode step reads with it (state updated
 * in place as kla_decode_step_ex).  lambda [n_seqs, H] fp32.  Errors: as
 * kla_decode_step_ex, plus KLA_ERR_INVALID_ARG for a null lambda, ccq_state
 * or workspace or any overlap, KLA_ERR_WORKSPACE for a short workspace.
 */
kla_status kla_decode_step_ccq(const void *q, const void *k, const void *v,
                               const float *alpha, const float *eta, const float *lambda,
                               float *state, float *ccq_state, float *o, int32_t n_seqs,
                               int32_t H, int32_t dk, int32_t dv, float eps, kla_dtype dtype,
                               kla_beta_mode beta_mode, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Backward of the prefill: the gradients of a loss with respect to q, k, v,
 * alpha, eta and the initial state, given the loss's gradients with respect
 * to o (d_o) and to the final state (d_final).  The KLA summary ("Resumo
 * Tecnico: Atencao Linear Kaczmarz (KLA)", section "Implementacao") keeps
 * Gated DeltaNet's chunk algorithm, training included, and changes only
 * the step size; this is the derivative of the recurrence above, computed
 * chunkwise: a forward sweep stores each chunk-start state in the
 * workspace, a reverse sweep carries the state's gradient from the last
 * chunk to the first, and a second launch adds the column slices'
 * contributions in a fixed order (bitwise deterministic).  With bf16
 * inputs the large products run on the bf16 MFMA with the fp32 factors split
 * into hi/lo bf16 pairs (each product to about 2^-16 of its size), with fp32
 * accumulation; fp32 inputs run on the fp32 MFMA.
 *
 *   q, k, v, alpha, eta, cu_seqlens, n_seqs, total_tok, H, dk, dv, chunk,
 *   eps, dtype, beta_mode, initial_state
 *               exactly as the kla_fwd_chunked_ex call being differentiated.
 *   d_o         [total_tok, H, dv] fp32, required when total_tok > 0.
 *   d_final     [n_seqs, H, dk, dv] fp32, or NULL (the final state does not
 *               reach the loss).
 *   dq, dk_out  [total_tok, H, dk] fp32, written.
 *   dv_out      [total_tok, H, dv] fp32, written.
 *   d_alpha     [total_tok, H] fp32, written; required when alpha is set,
 *               ignored when alpha is NULL.
 *   d_eta       [total_tok, H] fp32, written.
 *   d_initial   [n_seqs, H, dk, dv] fp32, or NULL; written with the
 *               gradient of the initial state (of a zero start when
 *               initial_state is NULL).
 *   workspace   device buffer of at least kla_bwd_chunked_workspace_size
 *               bytes, 16-byte aligned, not overlapping any argument;
 *               contents on entry ignored, on return unspecified.
 * Outputs must not overlap each other or any input.  Errors: as
 * kla_fwd_chunked_ex, plus KLA_ERR_INVALID_ARG for a missing required
 * pointer or an overlap, KLA_ERR_WORKSPACE for a short workspace.
 */
size_t kla_bwd_chunked_workspace_size(int32_t n_seqs, int64_t total_tok, int32_t H, int32_t dk,
                                      int32_t dv, int32_t chunk);
kla_status kla_bwd_chunked(const void *q, const void *k, const void *v, const float *alpha,
                           const float *eta, const int32_t *cu_seqlens, int32_t n_seqs,
                           int64_t total_tok, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                           float eps, kla_dtype dtype, kla_beta_mode beta_mode,
                           const float *initial_state, const float *d_o, const float *d_final,
                           float *dq, float *dk_out, float *dv_out, float *d_alpha, float *d_eta,
                           float *d_initial, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Static description of a status code (never NULL). */
const char *kla_status_string(kla_status s);

/* Library version string, e.g. "0.1.0 gfx950". */
const char *kla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KLA_H */
