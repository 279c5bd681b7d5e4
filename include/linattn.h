/*
 * linattn.h -- C ABI of liblinattn.so: causal linear attention with a fixed
 * d_k x d_v state on one AMD Instinct MI355X (gfx950).
 *
 * The operations are those of the article "From GPT-2 to Kimi K3, explained"
 * (Chinese mirror on transcrab.onev.cat, German mirror on youmind.com):
 *   - ELU+1 linear attention with a running normaliser (section "Linear
 *     Attention", cached forward: S += phi(k)^T v, z += phi(k),
 *     o = phi(q) S / phi(q).z);
 *   - the DeltaNet delta rule (sections "DeltaNet (Fast Weight Programmers)"
 *     and "DeltaNet (Parallelizing Linear Transformers with Delta Rule)":
 *     read r = k S, u = beta (v - r), write S += k^T u, output o = q S), whose
 *     prefill runs in the chunkwise UT/WY form of the latter section;
 *   - its gated variants (sections "Gated Delta Net" and "KDA / Kimi
 *     Linear"): before each read the state decays, S <- diag(a_t) S, with a
 *     separate decay a_t[i] per key channel i (KDA), or one scalar a_t per
 *     token (Gated DeltaNet);
 *   - gated linear attention, the first step of section "Gated Delta Net"
 *     (the additive cache with a forgetting factor credited to Mamba-2):
 *     S <- a_t S + k^T v, o = q S.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.   All tensors are dense, row-major, last index fastest:
 *           q, k [B,H,T,dk]; v, o [B,H,T,dv]; beta [B,H,T];
 *           g [B,H,T,dk] (per key channel) or [B,H,T] (per token);
 *           S [B,H,dk,dv] (row i = key channel i); z [B,H,dk].
 *           Decode entry points use the same layout with T = 1 dropped:
 *           q, k [N,H,dk]; v, o [N,H,dv]; beta [N,H]; g [N,H,dk] or [N,H].
 * Output.   o_t is read from the state AFTER token t has been written (the
 *           article's code reads q S after S += ...), and the normaliser of
 *           linear attention includes token t as well.
 * dtype.    LA_DTYPE_F32 (0) or LA_DTYPE_BF16 (1); it applies to q, k, v,
 *           beta, g and o.  The state S and normaliser z are always float32.
 *           bf16 outputs are rounded to nearest even.
 * Pointers. Device pointers (hipMalloc'd or equivalent), owned by the caller.
 *           q, k, v and o of the prefill entry points (and dO, dq, dk, dv
 *           of the backward) and S of the decode entry points must be
 *           16-byte aligned (they are read or written in vectors of up to
 *           16 bytes); LA_ERR_ALIGN otherwise.  o must not alias any input.
 *           S (and z) are read and written.  The
 *           library keeps no state between calls; calls are re-entrant.  It
 *           never allocates device memory: the seven entry points that need
 *           scratch memory on some paths (la_prefill, gla_prefill,
 *           deltanet_prefill, deltanet_prefill_segmented and the three
 *           backward entry points) take a
 *           caller-owned workspace pointer and its size in bytes, and each
 *           has a *_workspace_bytes() query with the same sizes and dtype.
 *           The query returns 0 where no workspace is needed (the workspace
 *           may then be NULL), and 0 for arguments the call would reject.
 *           A workspace must be at least the queried size (LA_ERR_WORKSPACE
 *           otherwise) and 256-byte aligned (LA_ERR_ALIGN); its contents on
 *           entry do not matter, and it must not be used by other work
 *           until the call's kernels have finished on `stream`.  The sizes
 *           (C = ceil(T/64) chunks, bf16 inputs unless stated):
 *             - la_prefill, gla_prefill: 6 B*H*C*dk*dv + 4 B*H*C*dk (the
 *               per-chunk state increments in fp32, the state entering
 *               each chunk in bf16, the normaliser entering each chunk or
 *               the chunk's decay); 0 for float32;
 *             - deltanet_prefill with a per-channel gate, dk = 128 and
 *               dv % 32 == 0: 384 B*H*C*dk + 4 B*H*C*dk (decay-scaled
 *               copies of q and k); 0 otherwise;
 *             - deltanet_prefill_backward: 8 B*H*C*dk*dv (the state
 *               entering and the gradient leaving every chunk), plus
 *               2 B*H*C*dk*(dk+64) with bf16 inputs (every chunk's P and
 *               R^T); the gated backward adds 4 B*H*C; each region is
 *               rounded up to 256 bytes;
 *             - kda_prefill_backward: 388 B*H*C*dk (the gate pre-pass's
 *               copies and decays) + 4 B*H*C*dk*dv (the chunk states and
 *               their gradients, bf16) + 2 B*H*C*dk*(dk+64) (P and R^T),
 *               each region rounded up to 256 bytes;
 *             - deltanet_prefill_segmented: see its declaration.
 * Sizes.    B, H (or N, H) >= 1; T >= 0 for prefill, any length (the last
 *           64-token chunk may be partial).  T = 0 enqueues no work when
 *           use_initial_state is set and otherwise zero-fills S (and z);
 *           the token arrays may then be NULL.
 *           dk and dv each one of 16, 32, 64, 128.  deltanet_prefill with
 *           a per-channel gate and LA_DTYPE_F32 supports dk <= 64.
 * Stream.   stream is a hipStream_t passed as void*; NULL is the null stream.
 *           Work is enqueued asynchronously; nothing synchronises the host.
 * Errors.   0 (LA_OK) or a negative code.  Arguments are validated before
 *           any HIP call, so a bad call has no effect on the device; the
 *           order is pointers, dtype, shape, head dimensions, alignment,
 *           workspace.  A
 *           kernel-launch failure returns LA_ERR_LAUNCH.  Numerical problems
 *           (NaN/Inf inputs) are not errors: they propagate to the outputs.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_OK 0
#define LA_ERR_NULL (-1)            /* a required pointer is NULL            */
#define LA_ERR_SHAPE (-2)           /* B/H/N not positive, T < 0, too large  */
#define LA_ERR_DTYPE (-3)           /* dtype not LA_DTYPE_F32/LA_DTYPE_BF16  */
#define LA_ERR_UNSUPPORTED_DIM (-4) /* dk or dv not in {16, 32, 64, 128}     */
#define LA_ERR_LAUNCH (-5)          /* the HIP runtime rejected a launch     */
#define LA_ERR_ALIGN (-6)           /* a vector-accessed pointer is not      */
                                    /* 16-byte aligned, or a workspace not   */
                                    /* 256-byte aligned                      */
#define LA_ERR_WORKSPACE (-7)       /* the workspace is NULL or smaller than */
                                    /* its *_workspace_bytes() query         */
#define LA_ERR_SCRATCH_LIMIT (-8)   /* la_prefill_noalloc: the call needs    */
                                    /* more than its fixed scratch holds     */

#define LA_DTYPE_F32 0
#define LA_DTYPE_BF16 1

/*
 * la_prefill -- causal ELU+1 linear attention over T tokens, chunkwise.
 * Article section "Linear Attention" (cached forward, feature map
 * phi(x) = elu(x) + 1 with the default constant 1, i.e. x + 1 for x > 0 and
 * exp(x) otherwise) and the chunked form of section "DeltaNet (Parallelizing
 * Linear Transformers with Delta Rule)" (intra-chunk masked attention plus an
 * inter-chunk state read), extended with the normaliser:
 *   S_t = S_{t-1} + phi(k_t)^T v_t,  z_t = z_{t-1} + phi(k_t),
 *   o_t = phi(q_t) S_t / (phi(q_t) . z_t).
 * q, k [B,H,T,dk], v [B,H,T,dv] in:    dtype.
 * o [B,H,T,dv] out:                    dtype.
 * S [B,H,dk,dv], z [B,H,dk] in/out:   float32.  use_initial_state = 0: the
 *   incoming contents are ignored and the state starts at zero; otherwise
 *   they are the initial state.  On completion they hold the final state.
 * workspace: la_prefill_workspace_bytes(B, H, T, dk, dv, dtype) bytes (see
 *   "Pointers"); NULL when that is 0.
 */
size_t la_prefill_workspace_bytes(int B, int H, int T, int dk, int dv,
                                  int dtype);
int la_prefill(const void *q, const void *k, const void *v, void *o, float *S,
               float *z, int use_initial_state, int B, int H, int T, int dk,
               int dv, int dtype, void *workspace, size_t workspace_bytes,
               void *stream);

/*
 * la_decode_step -- one new token per sequence, state updated in place.
 * Article section "Linear Attention", the cached forward at t = 1:
 *   S <- S + phi(k)^T v,  z <- z + phi(k),  o = phi(q) S / (phi(q) . z).
 * q, k [N,H,dk], v [N,H,dv] in; o [N,H,dv] out (dtype).
 * S [N,H,dk,dv], z [N,H,dk] float32, read and written in place.
 */
int la_decode_step(const void *q, const void *k, const void *v, void *o,
                   float *S, float *z, int N, int H, int dk, int dv, int dtype,
                   void *stream);

/*
 * deltanet_prefill -- delta rule over T tokens in the chunkwise UT/WY form
 * (64-token chunks).  Article section "DeltaNet (Parallelizing Linear
 * Transformers with Delta Rule)": per token r = k_t S, u_t = beta_t (v_t - r),
 * S += k_t^T u_t, o_t = q_t S; computed per chunk as
 * T = (I + tril(diag(beta) K K^T, -1))^{-1}, u = T diag(beta) (V - K S),
 * O = Q S + tril(Q K^T) u, S += K^T u.
 * With g != NULL the per-key-channel gated rule of sections "Gated Delta Net"
 * and "KDA / Kimi Linear" is used instead:
 *   S_t = diag(a_t) S_{t-1} + beta_t k_t^T (v_t - k_t diag(a_t) S_{t-1}),
 * where g = log a (the log-decay, <= 0) is given per token and key channel.
 * The chunked gated form divides keys by the decay accumulated from the
 * start of their 64-token chunk.  A chunk in which some key channel's summed
 * log-decay leaves [-64, 64] (stronger decay, or growth where g > 0), where
 * that division would leave the float range, is computed token by token
 * with the recurrence itself instead: any finite g gives the recurrence's
 * result, such chunks only take longer.
 * q and k are used as given: no feature map, normalisation or scale.
 * q, k [B,H,T,dk], v [B,H,T,dv], beta [B,H,T], g [B,H,T,dk] or NULL (dtype).
 * o [B,H,T,dv] out (dtype).  S [B,H,dk,dv] float32 in/out as in la_prefill.
 * workspace: deltanet_prefill_workspace_bytes(g != NULL, B, H, T, dk, dv,
 *   dtype) bytes; NULL when that is 0 (always so without a gate).
 */
size_t deltanet_prefill_workspace_bytes(int gated, int B, int H, int T,
                                        int dk, int dv, int dtype);
int deltanet_prefill(const void *q, const void *k, const void *v,
                     const void *beta, const void *g, void *o, float *S,
                     int use_initial_state, int B, int H, int T, int dk,
                     int dv, int dtype, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * deltanet_decode_step -- one new token per sequence, state updated in
 * place.  Article section "DeltaNet (Fast Weight Programmers)" (the layer
 * forward at t = 1): optional decay S <- diag(exp(g)) S, then r = k S,
 * u = beta (v - r), S <- S + k^T u, o = q S.
 * q, k [N,H,dk], v [N,H,dv], beta [N,H], g [N,H,dk] or NULL in (dtype);
 * o [N,H,dv] out (dtype); S [N,H,dk,dv] float32 in place.
 */
int deltanet_decode_step(const void *q, const void *k, const void *v,
                         const void *beta, const void *g, void *o, float *S,
                         int N, int H, int dk, int dv, int dtype,
                         void *stream);

/*
 * gated_deltanet_prefill -- the delta rule with one decay per token and head
 * (Gated DeltaNet, section "Gated Delta Net": a data-dependent scalar in
 * (0, 1] decays the previous state):
 *   S_t = a_t S_{t-1} + beta_t k_t^T (v_t - k_t a_t S_{t-1}),  o_t = q_t S_t,
 * computed in the chunkwise form with per-token decay ratios exp(G_r - G_c)
 * (G the summed log-decay), which are never above 1, so any g <= 0 is
 * supported.  g [B,H,T] = log a (dtype, required).  Everything else as
 * deltanet_prefill.  The result equals deltanet_prefill with g broadcast
 * over the key channels.
 */
int gated_deltanet_prefill(const void *q, const void *k, const void *v,
                           const void *beta, const void *g, void *o, float *S,
                           int use_initial_state, int B, int H, int T, int dk,
                           int dv, int dtype, void *stream);

/*
 * gated_deltanet_decode_step -- one token of gated_deltanet_prefill, state
 * updated in place: S <- a S, r = k S, u = beta (v - r), S <- S + k^T u,
 * o = q S.  g [N,H] = log a (required); the rest as deltanet_decode_step.
 */
int gated_deltanet_decode_step(const void *q, const void *k, const void *v,
                               const void *beta, const void *g, void *o,
                               float *S, int N, int H, int dk, int dv,
                               int dtype, void *stream);

/*
 * gla_prefill -- gated linear attention: the additive cache of section
 * "Linear Attention" with the forgetting factor of section "Gated Delta Net"
 * (credited there to Mamba-2), with q and k used as given (no feature map,
 * no normaliser):
 *   S_t = a_t S_{t-1} + k_t^T v_t,  o_t = q_t S_t.
 * Chunkwise: O = diag(Gam) Q S + (tril(Q K^T) * exp(G_r - G_c)) V and
 * S <- Gam_C S + (K * Gam_C / Gam)^T V, with G the log-decay summed from the
 * chunk start and Gam = exp(G).
 * q, k [B,H,T,dk], v [B,H,T,dv], g [B,H,T] = log a or NULL (no decay), in
 * dtype; o [B,H,T,dv] out; S [B,H,dk,dv] float32 in/out as in la_prefill.
 * workspace: gla_prefill_workspace_bytes(B, H, T, dk, dv, dtype) bytes.
 */
size_t gla_prefill_workspace_bytes(int B, int H, int T, int dk, int dv,
                                   int dtype);
int gla_prefill(const void *q, const void *k, const void *v, const void *g,
                void *o, float *S, int use_initial_state, int B, int H, int T,
                int dk, int dv, int dtype, void *workspace,
                size_t workspace_bytes, void *stream);

/*
 * gla_decode_step -- one token of gla_prefill, state updated in place:
 * S <- a S + k^T v, o = q S.  q, k [N,H,dk], v [N,H,dv], g [N,H] or NULL
 * (dtype); o [N,H,dv] out; S [N,H,dk,dv] float32 in place.
 */
int gla_decode_step(const void *q, const void *k, const void *v, const void *g,
                    void *o, float *S, int N, int H, int dk, int dv, int dtype,
                    void *stream);

/*
 * deltanet_prefill_backward -- gradients of deltanet_prefill without a gate
 * (the delta rule), for training: the article gives the chunk form of
 * section "DeltaNet (Parallelizing Linear Transformers with Delta Rule)" as
 * the linear-time way to train it.  For the loss
 *   sum(dO * o) + sum(dST * S_T)
 * it writes dq, dk [B,H,T,dk], dv [B,H,T,dv], dbeta [B,H,T] (dtype) and,
 * if dS0 != NULL, the gradient of the initial state dS0 [B,H,dk,dv] (fp32).
 * Inputs: q, k, v, beta as for deltanet_prefill; S0 [B,H,dk,dv] fp32 or NULL
 * (zero initial state); dO [B,H,T,dv] (dtype); dST [B,H,dk,dv] fp32 or NULL
 * (no gradient on the final state).  Chunkwise, per 64-token chunk with
 * incoming state S and dSn the gradient of the state leaving it:
 *   du = A^T dO + K dSn, dX = T^T du, dV = diag(beta) dX,
 *   dQ = dO S^T + tril(dO u^T) K, dS = dSn + Q^T dO - K^T diag(beta) dX, ...
 * With W = T diag(beta) K the last one is dS = dSn - P dSn + R^T dO,
 * P = W^T K, R = Q - A W; for bf16 inputs P and R are formed for all chunks
 * at once and the walk over chunks is that one product per chunk.
 * It recomputes the forward chunk states into the workspace of
 * deltanet_prefill_backward_workspace_bytes(B, H, T, dk, dv, dtype) bytes
 * (sizes under "Pointers" above).  Sizes: dk, dv in {16, 32, 64, 128} for
 * bf16, up to 64 for float32.  T = 0 copies dST to dS0 (or zero-fills it).
 */
size_t deltanet_prefill_backward_workspace_bytes(int B, int H, int T, int dk,
                                                 int dv, int dtype);
int deltanet_prefill_backward(const void *q, const void *k, const void *v,
                              const void *beta, const float *S0,
                              const void *dO, const float *dST, void *dq,
                              void *dk_out, void *dv_out, void *dbeta,
                              float *dS0, int B, int H, int T, int dk, int dv,
                              int dtype, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * gated_deltanet_prefill_backward -- gradients of gated_deltanet_prefill (one
 * decay a_t = exp(g_t) per token, section "Gated Delta Net"), for the same
 * loss as deltanet_prefill_backward, with the gate's gradient dg [B,H,T]
 * (dtype) as well.  g [B,H,T] (dtype) is required; every other argument,
 * size limit and error is as for deltanet_prefill_backward.  Per chunk, with
 * G_r the log-decay summed from the chunk start and G_C its last value, the
 * ungated formulas take the decay ratios exp(G_r - G_c) in A = tril(Q K^T)
 * and L, exp(G_r) on the rows of K S, Q S and their gradients, and
 * exp(G_C - G_r) on the rows of K dSn and u dSn^T; the chain becomes
 * dS = exp(G_C) dSn - P dSn + R^T dO.  g_t enters only the log-decays G_r,
 * r >= t, of its own chunk, so dg_t is the sum over those rows of the
 * gradient of G_r, formed in the same chunk pass from the terms where G
 * appears (K S and Q S, the ratios in A and L, the state leaving the
 * chunk); each term carries its own decay, so dg keeps its relative
 * accuracy when the decays are strong.
 * The workspace, of gated_deltanet_prefill_backward_workspace_bytes(...)
 * bytes, is that of deltanet_prefill_backward plus one float per chunk.
 */
size_t gated_deltanet_prefill_backward_workspace_bytes(int B, int H, int T,
                                                       int dk, int dv,
                                                       int dtype);
int gated_deltanet_prefill_backward(const void *q, const void *k,
                                    const void *v, const void *beta,
                                    const void *g, const float *S0,
                                    const void *dO, const float *dST,
                                    void *dq, void *dk_out, void *dv_out,
                                    void *dbeta, void *dg, float *dS0, int B,
                                    int H, int T, int dk, int dv, int dtype,
                                    void *workspace, size_t workspace_bytes,
                                    void *stream);

/*
 * kda_prefill_backward -- gradients of deltanet_prefill with a per-key-channel
 * gate (sections "Gated Delta Net" and "KDA / Kimi Linear": a decay
 * a_t[i] = exp(g_t[i]) per key channel scales row i of the state before each
 * read), for the same loss as deltanet_prefill_backward, with the gate's
 * gradient dg [B,H,T,dk] (dtype) as well.  g [B,H,T,dk] (dtype) is required;
 * q, k, v, beta, S0, dO, dST, dq, dk_out, dv_out, dbeta and dS0 are as for
 * deltanet_prefill_backward.  bf16 only: LA_DTYPE_F32 returns
 * LA_ERR_UNSUPPORTED_DIM; dk and dv each one of 16, 32, 64, 128.
 * Per chunk, with G the log-decay summed from the chunk start per channel,
 * Q~ = e^G q, K~ = e^G k, K^ = e^-G k and Gam_C = e^(G_C), the chunk form is
 * the ungated one with K~ on the left of K S and of L, K^ on the right of A
 * and L and in the state update S' = diag(Gam_C)(S + K^^T u); its backward is
 * the ungated one in the same operands (the chain takes
 * dS = diag(Gam_C) dSn - P dSn + R^T dO, P = W^T K^ diag(Gam_C), R = Q~ - A W,
 * W = T diag(beta) K~), and the gradients of Q~, K~, K^ and Gam_C give dq,
 * dk and dg (g_t enters the G_r, r >= t, of its own chunk).  A chunk in
 * which some channel's summed log-decay leaves [-64, 64] (where K^ would
 * leave the float range) is computed from the recurrence itself, token by
 * token: its transition from the identity, its gradients backwards from its
 * entry state; any finite g gives the recurrence's gradients, more slowly
 * for such chunks.  The workspace, of
 * kda_prefill_backward_workspace_bytes(...) bytes, is described under
 * "Pointers".  T = 0 copies dST to dS0 (or zero-fills it).
 */
size_t kda_prefill_backward_workspace_bytes(int B, int H, int T, int dk, int dv,
                                            int dtype);
int kda_prefill_backward(const void *q, const void *k, const void *v,
                         const void *beta, const void *g, const float *S0,
                         const void *dO, const float *dST, void *dq,
                         void *dk_out, void *dv_out, void *dbeta, void *dg,
                         float *dS0, int B, int H, int T, int dk, int dv,
                         int dtype, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * deltanet_prologue -- the steps just before the delta rule in the layer of
 * section "DeltaNet (Fast Weight Programmers)":
 *   q_out = q_scale * normalize(silu(q_in)),  k_out = normalize(silu(k_in)),
 *   beta_out = sigmoid(beta_logits),
 * with normalize(x) = x / max(|x|_2, 1e-12) over the head dimension (torch's
 * F.normalize) and silu(x) = x sigmoid(x), skipped when apply_silu = 0.
 * q_in, k_in, q_out, k_out [B,H,T,dk] (dtype; 16-byte aligned; outputs may
 * alias their inputs).  beta_logits [B,beta_heads,T] with beta_heads = 1 (one
 * logit per token shared by every head, the article's [b,1,t,1] view) or H;
 * beta_out [B,H,T]; both NULL to skip beta.  q_scale = 1 for the article's
 * layer (a 1/sqrt(dk) attention-style scale is the caller's choice).  The
 * outputs feed deltanet_prefill / deltanet_decode_step directly.
 */
int deltanet_prologue(const void *q_in, const void *k_in,
                      const void *beta_logits, void *q_out, void *k_out,
                      void *beta_out, int B, int H, int T, int dk,
                      int beta_heads, int apply_silu, float q_scale, int dtype,
                      void *stream);

/*
 * deltanet_prefill_segmented -- the delta rule of deltanet_prefill (gate 0:
 * none; gate 1: a decay per key channel, g [B,H,T,dk]) or of
 * gated_deltanet_prefill (gate 2: one decay per token, g [B,H,T]), with each
 * head's sequence cut into P segments of T / P tokens that are processed side
 * by side: the sequence-parallel chunk-state scan, for calls with few heads
 * and long sequences, where one pass over the whole sequence leaves most of
 * the GPU idle.  Article "From GPT-2 to Kimi K3, explained", section "DeltaNet
 * (Parallelizing Linear Transformers with Delta Rule)": each chunk continues
 * from the state the previous one leaves; since a run of tokens maps its
 * incoming state affinely, S_out = M S_in + S_z, and each output likewise,
 * o_t = o_t(from zero) + (M_t^T q_t)^T S_in, the segments' passes need not
 * wait for each other:
 *   1. every segment from its start state (segment 0 from S when
 *      use_initial_state is set, the others from zero), outputs into o;
 *   2. every segment from the identity with v = 0: its transition M (and the
 *      rows M_t^T q_t);
 *   3. the segments' incoming states by a scan with float32 accumulation
 *      (the products take about 16 significant bits of each operand, as a
 *      bf16 high and low part): S_in[1] = S_z[0],
 *      S_in[p+1] = M[p] S_in[p] + S_z[p], and the final state
 *      M[P-1] S_in[P-1] + S_z[P-1] into S;
 *   4. o += (M_t^T q_t)^T S_in[p] for every token of segment p >= 1.
 * The result is the recurrence's up to rounding (S_in enters step 4 with
 * about 16 significant bits).  Arguments, layouts and errors as
 * deltanet_prefill (gate 1), gated_deltanet_prefill (gate 2), plus:
 *   gate      0, 1 or 2 as above; g must be NULL exactly when gate is 0
 *             (LA_ERR_NULL for a missing g, LA_ERR_SHAPE for a g with gate
 *             0 or a gate outside 0..2);
 *   segments  P; 0 lets the library choose (deltanet_prefill_segments), 1
 *             is one pass over the whole sequence (deltanet_prefill or
 *             gated_deltanet_prefill).  P >= 2 must divide T
 *             (LA_ERR_SHAPE otherwise);
 *   dtype     LA_DTYPE_BF16 only (LA_ERR_UNSUPPORTED_DIM for float32).
 * workspace: deltanet_prefill_segmented_workspace_bytes(gate, B, H, T, dk,
 *   dv, dtype, segments) bytes, for P >= 2 (n = B*H*P segment-heads, each
 *   region rounded up to 256 bytes): 4 n dk dv (every segment's state from
 *   its start) + 4 n dk dk (transitions) + 4 B*H*T*dk (the transition pass's
 *   outputs and its zero values, bf16) + 128 B*H*(P-1)*ceil(dk/32)*dv (the
 *   incoming states as bf16 high and low parts) + 128 n dk ceil(dk/32) (the
 *   transitions likewise) + what the two passes need
 *   over B x H*P heads of T/P tokens (deltanet_prefill's workspace for a
 *   per-channel gate); for P = 1 the one-pass entry point's.
 */
size_t deltanet_prefill_segmented_workspace_bytes(int gate, int B, int H,
                                                  int T, int dk, int dv,
                                                  int dtype, int segments);
int deltanet_prefill_segmented(const void *q, const void *k, const void *v,
                               const void *beta, const void *g, int gate,
                               void *o, float *S, int use_initial_state, int B,
                               int H, int T, int dk, int dv, int dtype,
                               int segments, void *workspace,
                               size_t workspace_bytes, void *stream);
/*
 * deltanet_prefill_segments -- the P that deltanet_prefill_segmented uses
 * for segments = 0: the largest power of two up to 64 for which one pass
 * over B*H*P heads (32 value columns per workgroup) still fits on the
 * MI355X's 256 compute units at once, with T % P == 0 and at least 512 tokens
 * per segment; 1 when that is below 4 (two passes over the sequence then cost
 * more than the idle units).  0 for arguments the call would reject.
 */
int deltanet_prefill_segments(int B, int H, int T, int dk, int dv);

/*
 * la_prefill_noalloc -- la_prefill for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation): the same computation, arguments (minus the workspace)
 * and errors, with the scratch memory that la_prefill takes as its
 * workspace held instead in a fixed array in the library's device memory.
 * Every GPU the library runs on holds its own array of
 * LA_NOALLOC_SCRATCH_BYTES (64 MiB) until the process ends; its address is
 * looked up on the first call on each device (the current device).  Nothing
 * is allocated, by the library or by this call.
 * Limit: la_prefill_workspace_bytes(B, H, T, dk, dv, dtype) must not exceed
 * LA_NOALLOC_SCRATCH_BYTES, else LA_ERR_SCRATCH_LIMIT (checked before any
 * HIP call).  With bf16 inputs that is 6 B*H*C*dk*dv + 4 B*H*C*dk bytes for
 * C = ceil(T/64) chunks (38 MB at B=8, H=12, T=1024, dk = dv = 64); float32
 * inputs need none.
 * Calls on one GPU share its array, so calls that can overlap on one GPU
 * (streams without ordering between them) race and must not be made; calls
 * ordered on one stream are safe.  No state is carried between calls.
 */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int la_prefill_noalloc(const void *q, const void *k, const void *v, void *o,
                       float *S, float *z, int use_initial_state, int B,
                       int H, int T, int dk, int dv, int dtype, void *stream);

/* la_strerror -- a static, NUL-terminated description of an error code. */
const char *la_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* LINATTN_H */
