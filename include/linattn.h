/*
 * linattn.h - C ABI of liblinattn.so: causal linear attention and the gated
 * delta rule on AMD Instinct MI355X (gfx950).
 *
 * Operations are defined on the page "Linear attention and hybrids"
 * (ai.flicky.cc, stage 5, module 5.5, lesson 03); each entry point below names
 * the section and equation it computes.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates or frees device memory, and keeps no mutable
 *    global state; calls on different streams are independent.  The one
 *    exception is gdn_prefill_noalloc, which uses a fixed array in the
 *    library's own device memory (see there).
 *  - Tensors are dense row-major (C order) with the shapes given, and every
 *    pointer must be 16-byte aligned.
 *  - Activations (q, k, v, o) are float32 (LA_F32) or bfloat16 (LA_BF16), as
 *    chosen by `dtype`.  Gates (alpha, beta), states (S, z) and all
 *    accumulation are float32 whatever `dtype` is.
 *  - Layouts: q, k [B,H,T,dk]; v, o [B,H,T,dv]; alpha, beta [B,H,T];
 *    S [B,H,dv,dk] (row i of S belongs to value channel i); z [B,H,dk].
 *  - No 1/sqrt(d) scale is applied anywhere (the equations have none).
 *  - Arguments are validated on the host before anything is enqueued.  On an
 *    error nothing is launched and no output is written.  Work is enqueued
 *    asynchronously on `stream` (a hipStream_t passed as void*; NULL is the
 *    null stream); there is no host synchronisation.  A launch failure
 *    returns LA_ERR_HIP; faults inside kernels surface at the caller's next
 *    synchronisation.  No C++ exception crosses this interface.
 *  - Results are deterministic: two identical calls give bitwise-equal
 *    outputs (no atomics in any reduction).
 *  - Supported: dk, dv in {16, 32, 64, 128}; chunk in {16, 32, 64, 128};
 *    B, H, N >= 0 and T >= 0 (a zero-sized call copies the carried state to
 *    the output state and returns LA_OK).  Combinations that are valid but
 *    not implemented return LA_ERR_UNSUPPORTED.
 *  - Chunk length.  The chunked form gives the same result for every block
 *    length up to rounding, so `chunk` is a performance choice.  bf16 with
 *    dk = dv = 128 runs on the matrix-core kernels, which always use 64-token
 *    blocks, whatever valid chunk is asked for.  Every other shape runs on
 *    fp32 kernels with the requested block length and ONE workgroup per head;
 *    they suit small heads and few tokens, and are slow at large head sizes:
 *    measured on MI355X for B=2, H=16, T=8192, dk = dv = 128, those kernels
 *    (fp32 activations, chunk 32) take about 180 ms for
 *    gdn_prefill and 97 ms for lin_attn_prefill, against 0.15 ms and 0.12 ms
 *    on the matrix cores and 4 ms for the gated delta rule's recurrent form.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_ABI_VERSION 1

typedef int la_status;

enum {
    LA_OK = 0,
    LA_ERR_NULL = 1,        /* a required pointer is NULL                         */
    LA_ERR_SHAPE = 2,       /* a size is negative, out of range or too large
                               (also: a grid of 2^32 or more work-items, which
                               one launch cannot hold, e.g. a decode step over
                               2^24 heads of d = 16)                             */
    LA_ERR_DTYPE = 3,       /* dtype is not LA_F32 / LA_BF16                      */
    LA_ERR_UNSUPPORTED = 4, /* valid arguments, combination not implemented       */
    LA_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                   */
    LA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required         */
    LA_ERR_HIP = 7,         /* the HIP runtime reported an error                  */
    LA_ERR_ARG = 8          /* bad enum value (form, kind, fn) or overlap         */
};

enum { LA_F32 = 0, LA_BF16 = 1 };
enum { LA_FORM_CHUNKED = 0, LA_FORM_RECURRENT = 1, LA_FORM_PARALLEL = 2 };
enum { LA_KIND_NORMALIZED = 0, LA_KIND_GATED_DELTA = 1, LA_KIND_GATED = 2, LA_KIND_KDA = 3 };
enum {
    LA_FN_LIN_ATTN_PREFILL = 0,
    LA_FN_GDN_PREFILL = 1,
    LA_FN_DECODE_STEP = 2,
    LA_FN_GLA_PREFILL = 3,
    LA_FN_KDA_PREFILL = 4,
    LA_FN_GDN_VARLEN = 5,  /* B = number of sequences, T = total tokens */
    LA_FN_PREFILL_VARLEN = 6  /* lin_attn_prefill_varlen; sizes as for 5 */
};

/*
 * lin_attn_prefill - normalised causal linear attention over T tokens.
 *
 * Computes, per head and token t (section "The kernel trick: removing
 * softmax", the rewritten o_i equation; section "Three forms of one
 * computation", recurrent form):
 *     phi(x) = x + 1 for x > 0, exp(x) otherwise (elu + 1)
 *     S_t = S_{t-1} + v_t phi(k_t)^T,  z_t = z_{t-1} + phi(k_t)
 *     o_t = S_t phi(q_t) / (z_t . phi(q_t))        (token t included)
 * with S_0 = S0 and z_0 = z0 (zeros when NULL).  `form` picks how it is
 * evaluated (same section: masked parallel form, recurrent form, or the
 * chunked form with block size `chunk`, the last block possibly shorter):
 *   LA_FORM_PARALLEL  - masked T x T form; S0 and z0 must be NULL; T <= 8192.
 *   LA_FORM_RECURRENT - token by token, state in registers.
 *   LA_FORM_CHUNKED   - block-parallel form; `chunk` is the block size.
 * Outputs: o [B,H,T,dv]; S_out [B,H,dv,dk] and z_out [B,H,dk] receive the
 * final state when not NULL.  S_out may be the same pointer as S0 and z_out
 * the same as z0 (in-place update); any other overlap is an error.
 * workspace/ws_bytes: device scratch of at least
 * la_workspace_bytes(LA_FN_LIN_ATTN_PREFILL, ...) bytes (may be NULL when that
 * is 0); its contents on entry and exit are unspecified, and it must not
 * overlap any tensor argument (LA_ERR_ARG).
 */
la_status lin_attn_prefill(int dtype, int B, int H, int T, int dk, int dv,
                           const void* q, const void* k, const void* v,
                           const float* S0, const float* z0,
                           void* o, float* S_out, float* z_out,
                           int form, int chunk,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * gla_prefill - scalar-gated (unnormalised) linear attention over T tokens.
 *
 * Section "Memory must forget: decay and gates": the decay equation
 * S_t = gamma S_{t-1} + v_t k_t^T with the constant gamma replaced by an
 * input-dependent gate alpha_t, no feature map and no normaliser:
 *     S_t = alpha_t S_{t-1} + v_t k_t^T,   o_t = S_t q_t   (token t included)
 * alpha [B,H,T] float32 holds gate values (a constant alpha is the decay
 * equation itself).  S_0 = S0 (zeros when NULL).  form:
 *   LA_FORM_RECURRENT - token by token, any supported dtype and sizes;
 *   LA_FORM_CHUNKED   - block form, bf16 with dk = dv = 128 (64-token
 *                       blocks for any valid chunk; other shapes:
 *                       LA_ERR_UNSUPPORTED).
 * Outputs o [B,H,T,dv] and, when not NULL, S_out [B,H,dv,dk] (may be the
 * same pointer as S0).  workspace/ws_bytes: at least
 * la_workspace_bytes(LA_FN_GLA_PREFILL, ...) bytes, not overlapping any
 * tensor argument.
 */
la_status gla_prefill(int dtype, int B, int H, int T, int dk, int dv,
                      const void* q, const void* k, const void* v,
                      const float* alpha, const float* S0,
                      void* o, float* S_out,
                      int form, int chunk,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * gdn_prefill - the gated delta rule (Gated DeltaNet) over T tokens.
 *
 * Computes, per head and token t (section "Delta rule and Gated DeltaNet",
 * Gated DeltaNet equation; no feature map and no denominator, as the page
 * writes k for phi(k) and drops the normaliser from the decay section on):
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 * with S_0 = S0 (zeros when NULL).  alpha, beta [B,H,T] are gate VALUES
 * (alpha in (0,1], beta in [0,1]), float32.
 *   LA_FORM_RECURRENT - token by token, state in registers.
 *   LA_FORM_CHUNKED   - chunkwise form with chunk length `chunk`: per chunk
 *     a state-independent pass (chunk-local cumulative log-gates, K K^T, the
 *     unit lower-triangular solve of the WY/UT representation, Q K^T) and a
 *     sequential scan that carries S between chunks in float32.
 * Outputs: o [B,H,T,dv]; S_out [B,H,dv,dk] (final state) when not NULL; it
 * may be the same pointer as S0.  workspace: at least
 * la_workspace_bytes(LA_FN_GDN_PREFILL, ...) bytes.
 */
la_status gdn_prefill(int dtype, int B, int H, int T, int dk, int dv,
                      const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta,
                      const float* S0, void* o, float* S_out,
                      int form, int chunk,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * gdn_prefill_noalloc - gdn_prefill with no workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).
 *
 * Same operation, arguments, layouts and errors as gdn_prefill (workspace and
 * ws_bytes omitted).  Where gdn_prefill needs a workspace, this call uses one
 * array in the library's own device memory instead: 72 MiB per device
 * (la_workspace_bytes(LA_FN_GDN_PREFILL, ...) never exceeds it for the
 * supported shapes; a call that would need more returns LA_ERR_WORKSPACE),
 * held by every device the library runs on until the process ends.  The call
 * itself allocates nothing and frees nothing.  Every call on one device
 * shares that array and it keeps the last call's contents (nothing in it is
 * read before the same call writes it): calls that overlap in time on one
 * device - on different streams, or from different threads - race and give
 * wrong results; order them on one stream.  The array's address is looked up
 * on the first call on each device (with that device current); a failure
 * there returns LA_ERR_HIP.
 */
la_status gdn_prefill_noalloc(int dtype, int B, int H, int T, int dk, int dv,
                              const void* q, const void* k, const void* v,
                              const float* alpha, const float* beta,
                              const float* S0, void* o, float* S_out,
                              int form, int chunk, void* stream);

/*
 * gdn_prefill_prep / gdn_prefill_scan - the two halves of gdn_prefill with
 * LA_FORM_CHUNKED on the matrix-core path (dtype LA_BF16, dk = dv = 128,
 * any valid chunk (64-token blocks); other shapes return
 * LA_ERR_UNSUPPORTED).  Same equation and
 * section as gdn_prefill.  The library cuts each head's sequence into
 * segments of whole chunks (so that the chip is filled even with few heads);
 * over a segment the recurrence is an affine map of the entering state.
 *   prep: state-independent; for every segment but the last of every head,
 *     the segment's map (from k, v, alpha, beta), all segments in parallel;
 *     writes `workspace`.
 *   scan: composes the maps with S0 into each segment's entering state, then
 *     computes o and S_out for all segments in parallel; reads q, k, v,
 *     alpha, beta and the workspace written by prep for the same B, H, T.
 * gdn_prefill(..., LA_FORM_CHUNKED, 64, ...) computes the same result; it may
 * cut the sequence differently (its first segment runs beside the maps, which
 * needs S0 and o, so only the one-call form can do it), so the two agree to
 * rounding, not bit for bit.  Callers that split them must order scan after
 * prep (e.g. with an event) and must not reuse the workspace before scan has
 * finished.
 * The workspace layout is private to the library; when a single segment
 * covers the sequence the workspace size is 0 and prep does nothing.
 */
la_status gdn_prefill_prep(int dtype, int B, int H, int T, int dk, int dv,
                           const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, int chunk,
                           void* workspace, size_t ws_bytes, void* stream);
la_status gdn_prefill_scan(int dtype, int B, int H, int T, int dk, int dv,
                           const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta,
                           const float* S0, void* o, float* S_out,
                           int chunk, void* workspace, size_t ws_bytes,
                           void* stream);

/*
 * lin_attn_decode_step - one generation step for N sequences x H heads,
 * updating the carried state IN PLACE.
 *   LA_KIND_GATED_DELTA (section "Delta rule and Gated DeltaNet"):
 *       S <- alpha S (I - beta k k^T) + beta v k^T,   o = S q
 *     alpha, beta [N,H] float32 are required; z must be NULL.
 *   LA_KIND_GATED (section "Memory must forget: decay and gates", the decay
 *   equation with the input-dependent gate alpha_t):
 *       S <- alpha S + v k^T,   o = S q
 *     alpha [N,H] float32 is required; beta and z must be NULL.
 *   LA_KIND_KDA (same section as the gated delta kind, Kimi Delta Attention):
 *       S <- S Diag(alpha) (I - beta k k^T) + beta v k^T,   o = S q
 *     alpha [N,H,dk] float32 (one decay per key channel) and beta [N,H]
 *     float32 are required; z must be NULL.
 *   LA_KIND_NORMALIZED (section "Three forms of one computation", recurrent
 *   form, applied to one token):
 *       S <- S + v phi(k)^T,  z <- z + phi(k),  o = S phi(q) / (z . phi(q))
 *     z [N,H,dk] float32 is required; alpha and beta must be NULL.
 * q, k [N,H,dk]; v, o [N,H,dv]; S [N,H,dv,dk] float32, read once and written
 * once.  Each head's state is read and rewritten by one pass over HBM.
 */
la_status lin_attn_decode_step(int kind, int dtype, int N, int H, int dk, int dv,
                               const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta,
                               float* S, float* z, void* o, void* stream);

/*
 * gdn_prefill_varlen - the gated delta rule over a packed batch of N
 * sequences of different lengths, with state snapshots for prefix reuse.
 *
 * Every sequence is the recurrence of gdn_prefill (section "Delta rule and
 * Gated DeltaNet", Gated DeltaNet equation) on its own tokens, from its own
 * state.  Section "Honest talk: why MiniMax went back to full attention"
 * names prefix caching (reusing the work done for a shared beginning of
 * different requests) as missing from many implementations; for this layer
 * the reusable part of a prefix is its state, which this call can save at
 * regular positions.
 * Layout (device pointers, 16-byte aligned unless stated):
 *   cu_seqlens [N+1] int32, 4-byte aligned: sequence n is tokens
 *     cu_seqlens[n] .. cu_seqlens[n+1] (non-decreasing from 0 to T_total;
 *     values outside [0, T_total] are clamped, so a bad table gives wrong
 *     results but no access outside the buffers);
 *   q, k [H, T_total, dk]; v, o [H, T_total, dv] (every head holds all the
 *     sequences back to back); alpha, beta [H, T_total] float32;
 *   S0, S_out [N, H, dv, dk] float32 (S0 NULL = zeros; S_out may be S0);
 *   snapshots: when snap_interval > 0 and S_snap is not NULL, the state of
 *     sequence n after p tokens, for every positive multiple p of
 *     snap_interval up to its length, is written to
 *     S_snap[base_n + p / snap_interval - 1] ([snap_count, H, dv, dk]
 *     float32), base_n = sum over m < n of len_m / snap_interval; slots at or
 *     past snap_count are not written.
 * form: LA_FORM_CHUNKED (bf16, dk = dv = 128, any valid chunk: 64-token
 * blocks; snap_interval a multiple of 64) or LA_FORM_RECURRENT (any
 * supported dtype and size, snapshots at any interval).
 * workspace/ws_bytes: at least la_workspace_bytes(LA_FN_GDN_VARLEN, dtype, N,
 * H, T_total, dk, dv, form, chunk) bytes (the segment table is built on the
 * device, so the host never reads cu_seqlens); it must not overlap any
 * other argument.  Errors as for gdn_prefill.
 */
la_status gdn_prefill_varlen(int dtype, int N, int H, int T_total, int dk, int dv,
                             const int* cu_seqlens,
                             const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta, const float* S0,
                             void* o, float* S_out,
                             int snap_interval, int snap_count, float* S_snap,
                             int form, int chunk,
                             void* workspace, size_t ws_bytes, void* stream);

/*
 * lin_attn_prefill_varlen - a packed batch of N sequences of different
 * lengths, with state snapshots for prefix reuse, for every kind of
 * recurrence in this library.
 *
 * kind picks the recurrence each sequence runs on its own tokens from its own
 * state, the same equations as the uniform entry points:
 *   LA_KIND_NORMALIZED  - lin_attn_prefill (section "Three forms of one
 *                         computation"); state (S, z); alpha, beta NULL;
 *   LA_KIND_GATED       - gla_prefill (section "Memory must forget: decay and
 *                         gates"); alpha [H, T_total] float32; beta NULL;
 *   LA_KIND_KDA         - kda_prefill (section "Delta rule and Gated
 *                         DeltaNet", KDA); alpha [H, T_total, dk] and beta
 *                         [H, T_total] float32;
 *   LA_KIND_GATED_DELTA - forwards to gdn_prefill_varlen (same arguments;
 *                         z0, z_out and z_snap must be NULL).
 * Section "Honest talk: why MiniMax went back to full attention" names prefix
 * caching (reusing the work done for a shared beginning of different
 * requests) as missing from many implementations; for these layers the
 * reusable part of a prefix is the state (S, and z for the normalised kind),
 * which this call can save at regular positions.
 * Layout (device pointers, 16-byte aligned unless stated):
 *   cu_seqlens [N+1] int32, 4-byte aligned: sequence n is tokens
 *     cu_seqlens[n] .. cu_seqlens[n+1] (non-decreasing from 0 to T_total;
 *     values outside [0, T_total] are clamped, so a bad table gives wrong
 *     results but no access outside the buffers);
 *   q, k [H, T_total, dk]; v, o [H, T_total, dv] (every head holds all the
 *     sequences back to back);
 *   S0, S_out [N, H, dv, dk] and (normalised kind) z0, z_out [N, H, dk]
 *     float32; S0/z0 NULL = zeros; S_out may be S0 and z_out may be z0;
 *     other kinds: z0, z_out, z_snap must be NULL (LA_ERR_ARG);
 *   snapshots: when snap_interval > 0 and S_snap is not NULL, the state of
 *     sequence n after p tokens, for every positive multiple p of
 *     snap_interval up to its length, is written to
 *     S_snap[base_n + p / snap_interval - 1] ([snap_count, H, dv, dk]
 *     float32) and, for the normalised kind, z_snap[same slot]
 *     ([snap_count, H, dk] float32, then required), with base_n = sum over
 *     m < n of len_m / snap_interval; slots at or past snap_count are not
 *     written.
 * form: LA_FORM_RECURRENT (token by token, state in registers; any supported
 * dtype and size; snapshots at any interval) or LA_FORM_CHUNKED, the block
 * form on the matrix cores for every kind (bf16, dk = dv = 128, any valid
 * chunk: 64-token blocks; snap_interval a multiple of 64; other dtypes and
 * sizes return LA_ERR_UNSUPPORTED).  The recurrent form is token-serial
 * within each sequence: on 16 sequences of mixed lengths (16 384 tokens, the
 * longest 3551, H = 16, d = 128) it takes 1.9-2.8 ms, against 0.13 ms
 * (normalised), 0.12 ms (scalar-gated), 0.36 ms (KDA) and 0.18 ms (gated
 * delta) for the block form.
 * workspace/ws_bytes: at least la_workspace_bytes(LA_FN_PREFILL_VARLEN,
 * dtype, N, H, T_total, dk, dv, form, chunk) bytes (one size for every kind;
 * the sequence and snapshot tables are built on the device, so the host
 * never reads cu_seqlens); it must not overlap any other argument.  Any overlap between outputs, or between an
 * output and an input other than the in-place state pairs, is LA_ERR_ARG.
 */
la_status lin_attn_prefill_varlen(int kind, int dtype, int N, int H, int T_total, int dk, int dv,
                                  const int* cu_seqlens,
                                  const void* q, const void* k, const void* v,
                                  const float* alpha, const float* beta,
                                  const float* S0, const float* z0,
                                  void* o, float* S_out, float* z_out,
                                  int snap_interval, int snap_count,
                                  float* S_snap, float* z_snap,
                                  int form, int chunk,
                                  void* workspace, size_t ws_bytes, void* stream);

/*
 * kda_prefill - Kimi Delta Attention over T tokens: the gated delta rule with
 * a per-channel decay.
 *
 * Section "Delta rule and Gated DeltaNet": KDA replaces the scalar gate of the
 * Gated DeltaNet equation by a diagonal matrix Diag(alpha_t), one decay rate
 * per memory channel.  The diagonal acts on the key side of S (d_v x d_k),
 * where the scalar stands:
 *     S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t                                   (token t included)
 * alpha [B,H,T,dk] float32 holds decay values per key channel (all equal: the
 * Gated DeltaNet equation); beta [B,H,T] float32.  S_0 = S0 (zeros when NULL).
 * form:
 *   LA_FORM_RECURRENT - token by token, any supported dtype and sizes;
 *   LA_FORM_CHUNKED   - block form on the matrix cores, bf16 with
 *                       dk = dv = 128 (64-token blocks for any valid
 *                       chunk; other shapes: LA_ERR_UNSUPPORTED).  alpha
 *                       must lie in (0, 1].
 * Outputs o [B,H,T,dv] and, when not NULL, S_out [B,H,dv,dk] (may be the
 * same pointer as S0; any other overlap is LA_ERR_ARG).  workspace/ws_bytes:
 * at least la_workspace_bytes(LA_FN_KDA_PREFILL, ...) bytes (0 for the
 * recurrent form; 74 240 bytes per head and chunk of 64 tokens for the block
 * form), not overlapping any tensor argument.
 */
la_status kda_prefill(int dtype, int B, int H, int T, int dk, int dv,
                      const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta, const float* S0,
                      void* o, float* S_out,
                      int form, int chunk,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * gdn_preprocess - the cheap per-token operations in front of a Gated
 * DeltaNet layer, fused into one pass that also turns the token-major
 * projections into the head-major rows gdn_prefill reads.
 *
 * Page "Linear attention and hybrids": section "2025 hybrids: Qwen3-Next and
 * Kimi Linear" (a causal depthwise convolution over time with kernel 4 in
 * front of q, k and v), section "Delta rule and Gated DeltaNet" (unit-length
 * keys), section "Memory must forget: decay and gates" (sigmoid gates).  Per
 * sequence b, token t and channel c (C = H*(2dk+dv) channels):
 *     y_t[c] = sum_{i=0..3} conv_w[c][i] x_{t-3+i}[c]     (no bias)
 * where the three tokens before t = 0 are conv_state (zeros when NULL).  The
 * channels are q (H*dk), then k (H*dk), then v (H*dv), each head's block
 * contiguous.  Then, per head h:
 *     q[b,h,t] = y_t[q block h] / |y_t[q block h]|   (a zero row stays zero)
 *     k[b,h,t] = y_t[k block h] / |y_t[k block h]|
 *     v[b,h,t] = y_t[v block h]
 *     alpha[b,h,t] = sigmoid(a_logit[b,t,h]),  beta[b,h,t] = sigmoid(b_logit[b,t,h])
 * Arguments (device pointers, 16-byte aligned, element type `dtype` unless
 * stated):
 *   x [B,T,C]; conv_w [C,4] float32 (tap 3 multiplies the current token);
 *   a_logit, b_logit [B,T,H] float32; conv_state [B,3,C] or NULL (row 0 is
 *   token t-3); conv_state_out [B,3,C] or NULL receives the last three tokens
 *   of [conv_state; x], ready for the next call on the same sequences; it must
 *   not overlap conv_state or any other argument (LA_ERR_ARG);
 *   q, k [B,H,T,dk]; v [B,H,T,dv]; alpha, beta [B,H,T] float32.
 * dk, dv in {16, 32, 64, 128}.  T = 0 only copies conv_state to
 * conv_state_out.  Errors: LA_ERR_DTYPE, LA_ERR_SHAPE, LA_ERR_NULL,
 * LA_ERR_ALIGN, LA_ERR_ARG (overlap), LA_ERR_HIP; nothing is launched on
 * error.  Works asynchronously on `stream`; the caller owns every buffer.
 */
la_status gdn_preprocess(int dtype, int B, int T, int H, int dk, int dv,
                         const void* x, const float* conv_w,
                         const float* a_logit, const float* b_logit,
                         const void* conv_state, void* conv_state_out,
                         void* q, void* k, void* v, float* alpha, float* beta,
                         void* stream);

/*
 * gdn_preprocess_varlen - gdn_preprocess over a packed batch of N sequences
 * of different lengths, producing the layout gdn_prefill_varlen reads.
 *
 * Same operations and sources as gdn_preprocess, per sequence: the
 * convolution of sequence n never reaches into another sequence; its three
 * tokens before the first come from conv_state[n] (zeros when conv_state is
 * NULL), and conv_state_out[n] receives the last three tokens of
 * [conv_state[n]; its tokens].  Layout (device pointers):
 *   cu_seqlens [N+1] int32 (4-byte aligned): sequence n is tokens
 *     cu_seqlens[n] .. cu_seqlens[n+1] (non-decreasing from 0 to T_total;
 *     out-of-range values are clamped, never read past a buffer);
 *   x [T_total, C], a_logit, b_logit [T_total, H] float32, conv_w [C, 4]
 *   float32, conv_state / conv_state_out [N, 3, C] (dtype; NULL allowed, not
 *   the same memory);
 *   q, k [H, T_total, dk], v [H, T_total, dv], alpha, beta [H, T_total]
 *   float32.
 * Errors as for gdn_preprocess; nothing is launched on error.
 */
la_status gdn_preprocess_varlen(int dtype, int N, int T_total, int H, int dk, int dv,
                                const int* cu_seqlens, const void* x, const float* conv_w,
                                const float* a_logit, const float* b_logit,
                                const void* conv_state, void* conv_state_out,
                                void* q, void* k, void* v, float* alpha, float* beta,
                                void* stream);

/*
 * la_workspace_bytes - device workspace needed by one call of `fn` with the
 * given arguments (0 when none is needed).  Returns (size_t)-1 when the
 * arguments are invalid or the combination is not supported.
 */
size_t la_workspace_bytes(int fn, int dtype, int B, int H, int T, int dk, int dv,
                          int form, int chunk);

/* la_status_str - a static, human-readable name for a status code. */
const char* la_status_str(la_status s);

/* la_abi_version - LA_ABI_VERSION of the built library. */
int la_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
