/*
 * libgdn — Gated DeltaNet token mixer for AMD Instinct MI355X (gfx950).
 *
 * C ABI. Every pointer argument is DEVICE memory unless stated otherwise; the
 * caller owns every buffer, the library allocates nothing, keeps no pointer
 * after a call returns and never synchronises: work is enqueued on `stream`
 * (a hipStream_t passed as void*, NULL = the null stream) and completes in
 * stream order. Errors found by argument validation are returned before any
 * work is enqueued, so an error means nothing was written. Faults inside a
 * kernel surface at the caller's next synchronisation on that stream.
 * Results are bitwise deterministic for a given input and launch shape (no
 * atomics). Calls are reentrant; the only library state is the thread-local
 * error detail behind gdn_last_error().
 *
 * Notation (page "NLP——技术报告解读-Qwen3.8-Flash-Next", section
 * "Gated DeltaNet 核心机制"): per head, q_t, k_t in R^dk, v_t in R^dv, state
 * S in R^{dk x dv}, decay gate alpha_t in (0,1) (passed as log alpha_t) and
 * write gate beta_t in (0,1). One token updates the state as
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 * equivalently: decay S by alpha_t, take the error e_t = v_t - S^T k_t
 * against the decayed state, add beta_t k_t e_t^T; then y_t = S_t^T q_t
 * (the post-update state, no 1/sqrt(dk) scale).
 *
 * Layouts (row-major, contiguous, token-major):
 *   q, k           [rows, H, dk]
 *   v, y           [rows, H, dv]
 *   log_alpha, beta [rows, H]          float32
 *   S0, S_T, S     [N, H, dk, dv]      float32
 * where rows = N*T for equal-length batches (sequence n owns rows
 * n*T .. n*T+T-1) or the packed total for varlen batches.
 *
 * Supported: dk, dv in {64, 128}; q/k/v and y dtypes GDN_F32, GDN_BF16 or
 * GDN_F16. With 16-bit inputs the matrix products run on 16-bit MFMA
 * (bf16 inputs: the key-side products on bf16, the rest on fp16) with fp32
 * accumulation and an fp32 state; with fp32 inputs every product runs on
 * fp32 MFMA. Gates must satisfy log_alpha finite and <= 0,
 * 0 <= beta <= 1; outside that domain the kernels still terminate and stay in
 * bounds but the accuracy is not specified. With bf16 inputs the internal
 * fp16 operands assume |v|, |S| and the intermediate errors stay below
 * about 6e4.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_API __attribute__((visibility("default")))

/* element types */
enum gdn_dtype_e {
  GDN_F32 = 0,
  GDN_BF16 = 1,
  GDN_F16 = 2,
};

/* return codes */
enum gdn_status_e {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = -1, /* null pointer, bad size, aliasing */
  GDN_ERR_UNSUPPORTED = -2, /* head size or dtype combination not built */
  GDN_ERR_MISALIGNED = -3,  /* a pointer lacks its required alignment */
  GDN_ERR_HIP = -4,         /* a HIP runtime call failed (see gdn_last_error) */
};

/*
 * Chunked parallel prefill: runs the recurrence above over whole sequences
 * and returns every y_t and the final state S_T.
 *
 *   q, k, v      inputs, dtype in_dtype, layouts above.
 *   log_alpha    float32 [rows, H], log of the decay gate.
 *   beta         float32 [rows, H], write gate.
 *   S0           float32 [N, H, dk, dv] initial states, or NULL for zeros.
 *   y            output [rows, H, dv], dtype out_dtype.
 *   S_T          float32 [N, H, dk, dv] final states, or NULL to skip. May
 *                equal S0 (in-place update); must not overlap anything else.
 *   cu_seqlens   int32 [N+1] device array of sequence starts (cu_seqlens[0]
 *                = 0, non-decreasing, cu_seqlens[N] = rows), or NULL for N
 *                sequences of T tokens each.
 *   N            number of sequences (>= 0).
 *   T            tokens per sequence when cu_seqlens is NULL; otherwise the
 *                total row count `rows` of the packed batch. Kernels clamp
 *                every sequence to [0, rows) so bad offsets cannot address
 *                memory outside the buffers.
 *   H, dk, dv    heads and head sizes.
 *
 * Empty sequences (length 0) copy S0 to S_T. Inputs must not alias outputs.
 * q, k, v, y, S0 and S_T must be 16-byte aligned; log_alpha, beta and
 * cu_seqlens 4-byte aligned. With 16-bit inputs and dk = 128, the number of
 * state columns per workgroup (16, 32, 64 or 128) follows from N * H * dv;
 * results do not depend on it (each column's arithmetic is the same). The
 * environment variable GDN_PREFILL_NS (1, 2, 4 or 8 state waves of 16
 * columns) sets it instead: a test hook.
 */
GDN_API int gdn_chunk_fwd(const void *q, const void *k, const void *v,
                          const float *log_alpha, const float *beta,
                          const float *S0, void *y, float *S_T,
                          const int32_t *cu_seqlens, int32_t N, int32_t T,
                          int32_t H, int32_t dk, int32_t dv, int32_t in_dtype,
                          int32_t out_dtype, void *stream);

/*
 * Single-token decode step, in place: for every (sequence n, head h) applies
 * one token of the recurrence above to S[n, h] and writes y[n, h].
 * The fixed-size state replaces a growing cache (page "NLP——技术报告解读-
 * Qwen3.8-Flash-Next", section "Gated DeltaNet 核心机制").
 *
 *   q, k [N, H, dk]; v, y [N, H, dv]; log_alpha, beta float32 [N, H];
 *   S float32 [N, H, dk, dv], read and overwritten.
 * S must not overlap any other argument. q, k, v, y and S must be 16-byte
 * aligned, the gates 4-byte aligned.
 */
GDN_API int gdn_decode_step(const void *q, const void *k, const void *v,
                            const float *log_alpha, const float *beta,
                            float *S, void *y, int32_t N, int32_t H,
                            int32_t dk, int32_t dv, int32_t in_dtype,
                            int32_t out_dtype, void *stream);

/*
 * Gates from raw pre-activations (page "NLP——技术报告解读-Qwen3.8-Flash-Next",
 * section "GDN 参数化细节", gate display): with per-head parameters A and
 * b_alpha, the gates of a token-head with pre-activations a (decay) and b
 * (write) are
 *     log alpha = -exp(A_h) * softplus(a + b_alpha_h),   beta = sigmoid(b).
 * The two calls below take a and b in place of log_alpha and beta and
 * compute the gates inside the kernels, in fp32, so no separate elementwise
 * pass over the gates is needed.
 *
 *   a, b       float32 [rows, H] (prefill) or [N, H] (decode), raw
 *              pre-activations; any finite values.
 *   A          float32 [H], required (log of the per-head decay rate).
 *   b_alpha    float32 [H], or NULL for zeros.
 * All three are 4-byte aligned inputs and must not overlap an output.
 */

/* Chunked prefill with raw gates; every other argument as gdn_chunk_fwd. */
GDN_API int gdn_chunk_fwd_gated(const void *q, const void *k, const void *v,
                                const float *a, const float *b, const float *A,
                                const float *b_alpha, const float *S0, void *y,
                                float *S_T, const int32_t *cu_seqlens,
                                int32_t N, int32_t T, int32_t H, int32_t dk,
                                int32_t dv, int32_t in_dtype,
                                int32_t out_dtype, void *stream);

/*
 * Segment-parallel chunked prefill. The recurrence of the page
 * "NLP——技术报告解读-Qwen3.8-Flash-Next", section "Gated DeltaNet 核心机制",
 * is affine in the state, so over a stretch of tokens S_out = M S_in + N
 * (M: the product of the per-token factors alpha_t (I - beta_t k_t k_t^T);
 * N: the stretch run from a zero state). Each sequence is cut into
 * `segments` pieces of whole 32-token chunks; the summaries (M, N) of the
 * pieces are computed independently, chained into each piece's true initial
 * state, and every piece after the first is run again from it for y. This
 * is the one-GPU form of splitting a long sequence over several GPUs. It
 * does about three times the work of gdn_chunk_fwd over 1/segments of the
 * chain, with each launch's workgroups holding whole heads. On one GPU it
 * beats gdn_chunk_fwd when N * H is small: best near segments =
 * 256 / (N * H) + 1, where each launch fills the 256 CUs once (B1 H32
 * T65536: 9 segments, 0.75x the time of gdn_chunk_fwd).
 *
 *   segments   2 .. 64.
 *   workspace  device memory of at least
 *              gdn_chunk_fwd_segmented_workspace_size(...) bytes, 256-byte
 *              aligned, not overlapping any argument; its contents on entry
 *              do not matter and are overwritten.
 * Every other argument as gdn_chunk_fwd (y and S_T equal gdn_chunk_fwd's up
 * to rounding). Errors as gdn_chunk_fwd, plus GDN_ERR_INVALID_ARG for a bad
 * segment count or a workspace that is missing or too small.
 */
GDN_API int gdn_chunk_fwd_segmented(const void *q, const void *k, const void *v,
                                    const float *log_alpha, const float *beta,
                                    const float *S0, void *y, float *S_T,
                                    const int32_t *cu_seqlens, int32_t N, int32_t T,
                                    int32_t H, int32_t dk, int32_t dv,
                                    int32_t segments, void *workspace,
                                    size_t workspace_bytes, int32_t in_dtype,
                                    int32_t out_dtype, void *stream);

/*
 * gdn_chunk_fwd_segmented for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and results, with the workspace taken from
 * a fixed scratch array of GDN_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends. The call allocates nothing and
 * rejects, with GDN_ERR_INVALID_ARG and nothing enqueued, a problem whose
 * workspace (gdn_chunk_fwd_segmented_workspace_size) exceeds that size. Every
 * call on one GPU shares that GPU's scratch, which keeps the last call's
 * contents (every byte a call reads it first writes, so nothing needs
 * clearing): calls that overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller. Arguments and errors as
 * gdn_chunk_fwd_segmented without the workspace.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
GDN_API int gdn_chunk_fwd_segmented_noalloc(const void *q, const void *k, const void *v,
                                            const float *log_alpha, const float *beta,
                                            const float *S0, void *y, float *S_T,
                                            const int32_t *cu_seqlens, int32_t N, int32_t T,
                                            int32_t H, int32_t dk, int32_t dv,
                                            int32_t segments, int32_t in_dtype,
                                            int32_t out_dtype, void *stream);

/*
 * Bytes of workspace gdn_chunk_fwd_segmented needs (0 for invalid sizes):
 * segment bounds and per-segment states of all N sequences, in fp32:
 * N * H * (2 (P - 1) dk dv + (P - 2) dk dk) * 4 bytes plus the bounds,
 * independent of the row count. `rows` as for gdn_chunk_fwd (N * T, or T
 * with cu_seqlens) is validated but does not enter the size.
 */
GDN_API size_t gdn_chunk_fwd_segmented_workspace_size(int64_t rows, int32_t N, int32_t H,
                                                      int32_t dk, int32_t dv,
                                                      int32_t segments, int32_t in_dtype);

/*
 * Decode step with raw gates and, for serving, an optional pool of state
 * slots (the fixed-size state per sequence of the same section makes a slot
 * pool the natural cache).
 *
 *   S          float32 state(s), updated in place. With state_idx NULL, S is
 *              [N, H, dk, dv] as in gdn_decode_step and n_slots is ignored.
 *              Otherwise S is a pool [n_slots, H, dk, dv].
 *   state_idx  int32 [N] device array or NULL: sequence n reads and writes
 *              slot state_idx[n]. A slot outside [0, n_slots) marks a
 *              padding entry: the pool is left untouched and y[n] = 0. Two
 *              sequences must not name the same slot (their updates would
 *              race; the result is unspecified but stays in bounds).
 *   n_slots    number of states in the pool (>= 0) when state_idx is given.
 * Every other argument as gdn_decode_step.
 */
GDN_API int gdn_decode_step_gated(const void *q, const void *k, const void *v,
                                  const float *a, const float *b,
                                  const float *A, const float *b_alpha,
                                  float *S, const int32_t *state_idx,
                                  int32_t n_slots, void *y, int32_t N,
                                  int32_t H, int32_t dk, int32_t dv,
                                  int32_t in_dtype, int32_t out_dtype,
                                  void *stream);

/*
 * Multi-token decode: applies n_tok consecutive tokens (1 <= n_tok <= 8) of
 * every sequence to its state in one pass over the state, e.g. the verify
 * step of speculative decoding with several drafted tokens. The result
 * equals n_tok calls of gdn_decode_step; the state is read and written once
 * instead of n_tok times.
 *
 *   q, k       [N, n_tok, H, dk]; v, y [N, n_tok, H, dv] (token-major within
 *              each sequence).
 *   g_a, g_b   float32 [N, n_tok, H]: log_alpha and beta when A is NULL,
 *              otherwise the raw pre-activations a and b of the gate map
 *              above (A [H], b_alpha [H] or NULL).
 *   S          float32 states, updated in place.
 *   state_idx  NULL: S is [N, H, dk, dv] and each sequence's final state is
 *              written back in place (n_slots ignored). Otherwise an int32
 *              device table [N, 1 + n_tok] over a pool S [n_slots, H, dk,
 *              dv]: column 0 is the slot the sequence starts from, column
 *              1 + j the slot that receives the state after token j (a value
 *              outside [0, n_slots) skips that write). Writing each
 *              intermediate state lets a caller roll back to any accepted
 *              prefix. A start slot outside [0, n_slots) marks a padding
 *              entry: nothing is written and its y rows are zero. Slots
 *              written by one sequence must not be read or written by
 *              another in the same call.
 * Alignment and aliasing rules as gdn_decode_step; the index table is
 * 4-byte aligned.
 */
GDN_API int gdn_decode_multi(const void *q, const void *k, const void *v,
                             const float *g_a, const float *g_b,
                             const float *A, const float *b_alpha, float *S,
                             const int32_t *state_idx, int32_t n_slots,
                             void *y, int32_t N, int32_t n_tok, int32_t H,
                             int32_t dk, int32_t dv, int32_t in_dtype,
                             int32_t out_dtype, void *stream);

/*
 * Front end of the mixer (page "NLP——技术报告解读-Qwen3.8-Flash-Next",
 * section "GDN 参数化细节", first display; the convolution is short and causal
 * per the pwwt.cn page's Fig. 2 caption): for the three projected streams
 * x_q, x_k, x_v and each channel c = h*d + i,
 *     u_t[c] = sum_{j=0..3} w[c][j] * x_{t-3+j}[c]   (no bias; rows before the
 *              start of the token's sequence count as zero)
 *     a_t = SiLU(u_t) = u_t / (1 + exp(-u_t))
 *     q_t = a_t / sqrt(sum_i a_t[i]^2 + l2_eps) over the head's d channels,
 *     k_t likewise, v_t = a_t (no normalisation).
 *
 *   q_raw, k_raw, v_raw  [rows, H, d] in in_dtype.
 *   conv_w               float32 [3][H*d][4]: q taps, then k, then v; tap 3
 *                        multiplies the current token, tap 0 the one three
 *                        rows back.
 *   cu_seqlens, N, T     as for gdn_chunk_fwd (sequence boundaries).
 *   q, k, v              outputs [rows, H, d] in out_dtype.
 * Requires dk == dv == d in {64, 128}. q, k, v, the raw inputs and conv_w
 * 16-byte aligned; outputs must not overlap inputs.
 */
GDN_API int gdn_frontend_qkv(const void *q_raw, const void *k_raw,
                             const void *v_raw, const float *conv_w,
                             const int32_t *cu_seqlens, int32_t N, int32_t T,
                             int32_t H, int32_t d, float l2_eps, void *q,
                             void *k, void *v, int32_t in_dtype,
                             int32_t out_dtype, void *stream);

/*
 * Output gate (same section, third display; the RMSNorm is the zero-centred
 * one of the pwwt.cn page, section 2.1.1, whose gain is 1 + w): for each row
 * of d values (one token of one head)
 *     o = sigmoid(z) * y / sqrt(mean(y^2) + rms_eps) * (1 + norm_w).
 *
 *   y       [rows, d] in y_dtype (a [tokens, H, d] tensor is rows = tokens*H).
 *   z       [rows, d] in z_dtype.
 *   norm_w  float32 [d], shared by all heads, or NULL for w = 0.
 *   o       [rows, d] in out_dtype; must not overlap y or z.
 * d in {64, 128}; y, z, o 16-byte aligned.
 */
GDN_API int gdn_output_gate(const void *y, const void *z, const float *norm_w,
                            float rms_eps, void *o, int64_t rows, int32_t d,
                            int32_t y_dtype, int32_t z_dtype, int32_t out_dtype,
                            void *stream);

/*
 * Bytes of device workspace gdn_chunk_fwd_fused needs for `rows` packed rows
 * of H heads of size d (0 if rows == 0): the normalised q, k, v and y in
 * fp16, each padded to 256 bytes. Returns 0 for invalid sizes.
 */
GDN_API size_t gdn_fused_workspace_size(int64_t rows, int32_t H, int32_t d);

/*
 * The whole mixer prefill in one call (page "NLP——技术报告解读-Qwen3.8-
 * Flash-Next", section "GDN 参数化细节": front end, recurrence, output gate):
 *     q, k, v = gdn_frontend_qkv(q_raw, k_raw, v_raw, conv_w, l2_eps)
 *     y, S_T  = gdn_chunk_fwd(q, k, v, log_alpha, beta, S0)
 *     o       = gdn_output_gate(y, z, norm_w, rms_eps)
 * enqueued back to back on `stream`. The intermediates live in `workspace`
 * (device memory, 256-byte aligned, at least
 * gdn_fused_workspace_size(rows, H, d) bytes, overwritten by the call):
 * q, k, v and y are kept in fp16, so the result equals the three separate
 * calls made with those intermediate dtypes. in_dtype must be GDN_BF16 or
 * GDN_F16 (GDN_F32 returns GDN_ERR_UNSUPPORTED: fp32 inputs take the three
 * separate calls, which keep their precision). Range: q and k leave the front
 * end L2-normalised, but v = SiLU(conv) and y are held in fp16, so |v|, |y|
 * must stay below 65504; larger values overflow to inf (and NaN in the gate).
 *
 *   q_raw, k_raw, v_raw, z  [rows, H, d] in in_dtype (bf16 or fp16).
 *   conv_w                  float32 [3][H*d][4] (as gdn_frontend_qkv).
 *   log_alpha, beta         float32 [rows, H].
 *   S0, S_T                 float32 [N, H, d, d]; S0 NULL = zeros, S_T NULL =
 *                           not written (S_T may equal S0).
 *   norm_w                  float32 [d] or NULL (w = 0).
 *   o                       [rows, H, d] in out_dtype.
 *   cu_seqlens, N, T        as for gdn_chunk_fwd.
 * Requires dk == dv == d in {64, 128}. Inputs must not overlap o, S_T or the
 * workspace. All arguments are validated before anything is enqueued; a
 * GDN_ERR_HIP return from a later stage can leave earlier stages' writes in
 * the workspace (never in o or S_T before the stage that writes them).
 */
GDN_API int gdn_chunk_fwd_fused(const void *q_raw, const void *k_raw,
                                const void *v_raw, const float *conv_w,
                                const float *log_alpha, const float *beta,
                                const float *S0, const void *z,
                                const float *norm_w, float l2_eps,
                                float rms_eps, void *o, float *S_T,
                                const int32_t *cu_seqlens, int32_t N,
                                int32_t T, int32_t H, int32_t dk, int32_t dv,
                                int32_t in_dtype, int32_t out_dtype,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * Serving decode of the whole mixer in one kernel (page "NLP——技术报告解读-
 * Qwen3.8-Flash-Next", section "GDN 参数化细节": front end, recurrence,
 * output gate), n_tok tokens per sequence as gdn_decode_multi:
 *     q, k, v = front end of q_raw, k_raw, v_raw with the cached history
 *     y       = the recurrence of gdn_decode_multi
 *     o       = sigmoid(z) * y / sqrt(mean(y^2) + rms_eps) * (1 + norm_w)
 * The front end is that of gdn_frontend_qkv (short causal convolution with
 * conv_w, SiLU, L2 norm of q and k with l2_eps), with the convolution's
 * three previous rows taken from conv_state instead of zeros; the
 * intermediates stay in fp32 inside the kernel.
 *
 *   q_raw, k_raw, v_raw, z   [N, n_tok, H, d] in in_dtype (raw projections).
 *   conv_w       float32 [3][H*d][4] (as gdn_frontend_qkv).
 *   conv_state   in_dtype [slots, H, 3, 3, d]: per slot and head, for q, k
 *                and v in turn, the three raw rows before the call's first
 *                token, oldest first (zeros for a fresh sequence). Read from
 *                the start slot; the rows before the next token are written
 *                wherever the state is written (see state_idx of
 *                gdn_decode_multi).
 *   g_a, g_b, A, b_alpha, S, state_idx, n_slots   as gdn_decode_multi.
 *   norm_w       float32 [d] or NULL (w = 0).
 *   o            [N, n_tok, H, d] in out_dtype.
 * Requires dk == dv == d in {64, 128}. q_raw, k_raw, v_raw, z, conv_w,
 * conv_state, S and o are 16-byte aligned; the rest 4-byte aligned. Inputs
 * must not overlap S, conv_state or o.
 */
GDN_API int gdn_decode_fused(const void *q_raw, const void *k_raw,
                             const void *v_raw, const float *conv_w,
                             void *conv_state, const float *g_a,
                             const float *g_b, const float *A,
                             const float *b_alpha, float *S,
                             const int32_t *state_idx, int32_t n_slots,
                             const void *z, const float *norm_w, float l2_eps,
                             float rms_eps, void *o, int32_t N, int32_t n_tok,
                             int32_t H, int32_t d, int32_t in_dtype,
                             int32_t out_dtype, void *stream);

/*
 * Backward pass of the chunked prefill: the gradients of
 *     L = <dy, y> + <dS_T, S_T>
 * (y and S_T as gdn_chunk_fwd computes them from the same inputs) with
 * respect to q, k, v, log_alpha, beta and S0. The pages report backward
 * kernels for this mixer (page "NLP——技术报告解读-Qwen3.8-Flash-Next",
 * section "Gated DeltaNet 核心机制" for the recurrence; the pwwt.cn page,
 * section 2.1.1, "内核效率", for the kernels); these are the derivatives of
 * that recurrence, computed chunk by chunk.
 *
 *   q, k, v, log_alpha, beta, S0, cu_seqlens, N, T, H, dk, dv
 *                 the forward's inputs, as gdn_chunk_fwd (S0 NULL = zeros).
 *   dy            [rows, H, dv] in grad_dtype: gradient of y.
 *   dS_T          float32 [N, H, dk, dv] or NULL (zeros): gradient of S_T.
 *   dq, dk_out    [rows, H, dk] in grad_dtype; dv_out [rows, H, dv].
 *   dlog_alpha, dbeta   float32 [rows, H].
 *   dS0           float32 [N, H, dk, dv] or NULL (not written).
 *   workspace     device memory, 256-byte aligned, at least
 *                 gdn_chunk_bwd_workspace_size(rows, N, H, dk, dv, in_dtype)
 *                 bytes, overwritten. It holds the state at every chunk start
 *                 ((rows / 32 + N) * H * dk * dv values: fp32 for fp32
 *                 inputs, fp16 for 16-bit inputs, whose products round the
 *                 state to fp16 in any case), the per-column-
 *                 tile partial sums of dq, dk, dbeta and dlog_alpha for the
 *                 rows of one run (dv / 32 * H * (2 dk + 2) * 4 bytes per
 *                 row, about 128 MiB at most: longer problems run the
 *                 backward sweep several times, the last chunks first,
 *                 each run taking the same share of every sequence's chunks
 *                 while 64 N rows fit in the bound, else consecutive rows)
 *                 and, with more than one run, the state gradient carried
 *                 between runs (N * H * dk * dv * 4 bytes) and a table of
 *                 the runs' sequence offsets (runs * (N + 1) * 4 bytes).
 *                 The environment variables GDN_BWD_RUNS (that many
 *                 proportional runs) and GDN_BWD_SEGMENT_ROWS (runs of that
 *                 many rows) set the runs instead: test hooks, to be set
 *                 before both calls.
 * The states are recomputed from S0 (the forward's outputs are not needed).
 * Precision: with fp32 inputs every product runs in fp32 (fp32 MFMA) and the
 * gradients meet the fp32 bar (relative L2 1e-5); with bf16/fp16 inputs the
 * operands are rounded to fp16 for the 16-bit MFMA (fp32 accumulation, fp32
 * state) and the chunk-start states come from the 16-bit prefill kernel, so
 * the 16-bit bar (2e-3) applies. Rows must be covered by the sequences
 * (cu_seqlens[N] = rows). Inputs must not overlap outputs or the workspace.
 * Tensors are 16-byte aligned, the gates and cu_seqlens 4-byte aligned.
 * Results are deterministic (partial sums are added in a fixed order).
 */
GDN_API size_t gdn_chunk_bwd_workspace_size(int64_t rows, int32_t N, int32_t H,
                                            int32_t dk, int32_t dv, int32_t in_dtype);
GDN_API int gdn_chunk_bwd(const void *q, const void *k, const void *v,
                          const float *log_alpha, const float *beta,
                          const float *S0, const void *dy, const float *dS_T,
                          const int32_t *cu_seqlens, int32_t N, int32_t T,
                          int32_t H, int32_t dk, int32_t dv, void *dq,
                          void *dk_out, void *dv_out, float *dlog_alpha,
                          float *dbeta, float *dS0, int32_t in_dtype,
                          int32_t grad_dtype, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Backward pass with the gates given as raw pre-activations (as
 * gdn_chunk_fwd_gated): a, b [rows, H] replace log_alpha and beta, A [H]
 * (required) and b_alpha [H] (or NULL) are the per-head parameters, and the
 * gate gradients come back through the gate map: da, db [rows, H] float32
 * and dA, db_alpha [H] float32 (sums over all rows; written even when
 * b_alpha is NULL). Every other argument as gdn_chunk_bwd.
 */
GDN_API int gdn_chunk_bwd_gated(const void *q, const void *k, const void *v,
                                const float *a, const float *b, const float *A,
                                const float *b_alpha, const float *S0,
                                const void *dy, const float *dS_T,
                                const int32_t *cu_seqlens, int32_t N, int32_t T,
                                int32_t H, int32_t dk, int32_t dv, void *dq,
                                void *dk_out, void *dv_out, float *da, float *db,
                                float *dA, float *db_alpha, float *dS0,
                                int32_t in_dtype, int32_t grad_dtype,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * Convolution cache of gdn_decode_fused after a prefill: for every sequence
 * of a prefill batch (layout as gdn_frontend_qkv's raw inputs) and head,
 * writes the last three raw rows of q_raw, k_raw and v_raw, oldest first,
 * with zeros in place of rows before the sequence start, into
 * conv_state [slots, H, 3, 3, d] (dtype as the raw rows) at slot
 * slot_idx[n] (int32 device array, or NULL for slot n with slots = N;
 * entries outside [0, n_slots) are skipped). A pure copy: the rows the
 * short causal convolution of the next decode token needs.
 */
GDN_API int gdn_conv_state_from_prefill(const void *q_raw, const void *k_raw,
                                        const void *v_raw,
                                        const int32_t *cu_seqlens, int32_t N,
                                        int32_t T, int32_t H, int32_t d,
                                        const int32_t *slot_idx, int32_t n_slots,
                                        void *conv_state, int32_t dtype,
                                        void *stream);

/* Human-readable name of a return code (static string, never NULL). */
GDN_API const char *gdn_status_string(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
GDN_API const char *gdn_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
GDN_API int gdn_version(void);

/*
 * State columns per workgroup that gdn_chunk_fwd (and the chunk-start
 * states of gdn_chunk_bwd) would use for a batch of N sequences, H heads and
 * head sizes dk, dv with the given input dtype: 16, 32, 64 or 128 (32 for
 * fp32 inputs, dk = 64 and the segmented form). A query for profiling and
 * tests; it launches nothing. Results never depend on it. Returns 0 for
 * invalid sizes or dtypes.
 */
GDN_API int32_t gdn_prefill_state_columns(int32_t N, int32_t H, int32_t dk, int32_t dv,
                                          int32_t in_dtype);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
