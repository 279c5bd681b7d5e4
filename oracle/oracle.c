/*
 * oracle.c -- plain CPU float64 reference for causal linear attention with a
 * fixed d_k x d_v state: ELU+1 linear attention with a running normaliser,
 * the DeltaNet delta rule with its scalar and per-key-channel gated forms,
 * and decayed (gated) linear attention without a normaliser.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * Every function here is the per-token recurrence itself, written out one
 * token at a time with no chunking, blocking or reordering, so that it can be
 * checked against the article by eye.  Sources (all in the article "From GPT-2
 * to Kimi K3, explained", mirrored in Chinese on transcrab.onev.cat and in
 * German on youmind.com):
 *   - section "Linear Attention": the cached forward with the ELU+1 feature
 *     map, the running state S and normaliser z, and the division of q@S by
 *     q@z; plus the three-step description (non-negative scores, divide by
 *     their sum, weighted mean of v).
 *   - section "DeltaNet (Parallelizing Linear Transformers with Delta Rule)":
 *     the sequential prefill loop (read v_old = k S, u = beta (v - v_old),
 *     write S += k^T u, then read the output with q from the updated S).
 *   - section "Gated Delta Net" and "KDA / Kimi Linear": the state decays by a
 *     data-dependent factor before the delta step; for Gated DeltaNet the
 *     factor is one scalar per token, for KDA a separate value per key
 *     channel.  Reading used here: the decay a_t multiplies row i (key
 *     channel i) of S before the read at step t, i.e.
 *     S_t = diag(a_t) S_{t-1} + beta_t k_t (v_t - (diag(a_t) S_{t-1})^T k_t)^T.
 *   - section "Gated Delta Net", its first step (the additive cache with a
 *     forgetting factor, credited to Mamba-2): cache = alpha * S_old + k^T v,
 *     read with q, with q and k used as given (no feature map, no normaliser).
 *
 * Conventions: row-vector form of the article's code, S is d_k x d_v stored
 * row-major, a read is k S (= S^T k), a write adds k^T u.  Tensors are
 * row-major: q, k [B,H,T,d_k]; v [B,H,T,d_v]; beta [B,H,T]; g holds the
 * log-decay g = log a, [B,H,T,d_k] per key channel or [B,H,T] per token;
 * S [B,H,d_k,d_v]; z [B,H,d_k].
 *
 * Inputs are read in their stored precision (fp32, bf16 bit patterns, or
 * fp64) and widened to float64 element by element; all arithmetic is float64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };

/* Read element i of buffer p stored as dtype dt, widened to double. */
static double rd(const void *p, size_t i, int dt)
{
    if (dt == ORC_F32)
        return (double)((const float *)p)[i];
    if (dt == ORC_BF16) {
        /* bf16 is the top half of an IEEE binary32 */
        uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return ((const double *)p)[i];
}

/* phi(x) = elu(x) + 1 with the default elu constant 1:
 * x + 1 for x > 0, exp(x) otherwise.  Always positive. */
static double elu_plus_one(double x)
{
    return x > 0.0 ? x + 1.0 : exp(x);
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Causal ELU+1 linear attention with normaliser, one token at a time:
 *   S_t = S_{t-1} + phi(k_t)^T v_t        (d_k x d_v)
 *   z_t = z_{t-1} + phi(k_t)              (d_k)
 *   o_t = (phi(q_t) S_t) / (phi(q_t) . z_t)
 * Both the numerator and the denominator include token t itself.
 * S0/z0 may be NULL (zero initial state).  o [B,H,T,dv], S_out, z_out may be
 * NULL if not wanted.  S0 may alias S_out and z0 may alias z_out.
 * Returns 0, or -1 on allocation failure.
 */
int orc_la_recurrent(int B, int H, int T, int dk, int dv,
                     const void *q, const void *k, const void *v, int dt,
                     const double *S0, const double *z0,
                     double *o, double *S_out, double *z_out, int nthreads)
{
    int fail = 0;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; bh++) {
        double *S = malloc(sizeof(double) * (size_t)dk * dv);
        double *z = malloc(sizeof(double) * (size_t)dk);
        double *fq = malloc(sizeof(double) * (size_t)dk);
        double *fk = malloc(sizeof(double) * (size_t)dk);
        double *num = malloc(sizeof(double) * (size_t)dv);
        if (!S || !z || !fq || !fk || !num) {
#pragma omp atomic write
            fail = 1;
            free(S); free(z); free(fq); free(fk); free(num);
            continue;
        }
        const size_t sbase = (size_t)bh * dk * dv;
        for (size_t i = 0; i < (size_t)dk * dv; i++)
            S[i] = S0 ? S0[sbase + i] : 0.0;
        for (int i = 0; i < dk; i++)
            z[i] = z0 ? z0[(size_t)bh * dk + i] : 0.0;

        for (int t = 0; t < T; t++) {
            const size_t qk_row = ((size_t)bh * T + t) * dk;
            const size_t v_row = ((size_t)bh * T + t) * dv;
            for (int i = 0; i < dk; i++) {
                fq[i] = elu_plus_one(rd(q, qk_row + i, dt));
                fk[i] = elu_plus_one(rd(k, qk_row + i, dt));
            }
            /* write: S += phi(k)^T v, z += phi(k) */
            for (int i = 0; i < dk; i++) {
                for (int j = 0; j < dv; j++)
                    S[(size_t)i * dv + j] += fk[i] * rd(v, v_row + j, dt);
                z[i] += fk[i];
            }
            /* read with the updated state: o = phi(q) S / phi(q).z */
            if (o) {
                double den = 0.0;
                for (int i = 0; i < dk; i++)
                    den += fq[i] * z[i];
                for (int j = 0; j < dv; j++)
                    num[j] = 0.0;
                for (int i = 0; i < dk; i++)
                    for (int j = 0; j < dv; j++)
                        num[j] += fq[i] * S[(size_t)i * dv + j];
                for (int j = 0; j < dv; j++)
                    o[v_row + j] = num[j] / den;
            }
        }
        if (S_out)
            memcpy(S_out + sbase, S, sizeof(double) * (size_t)dk * dv);
        if (z_out)
            memcpy(z_out + (size_t)bh * dk, z, sizeof(double) * (size_t)dk);
        free(S); free(z); free(fq); free(fk); free(num);
    }
    return fail ? -1 : 0;
}

/*
 * Delta rule, optionally with a decay, one token at a time:
 *   (gated only)  S <- diag(exp(g_t)) S        row i scaled by exp(g_t[i]);
 *                                              g_per_channel = 0: every row
 *                                              by the one exp(g_t)
 *   r   = k_t S                                 (what the key reads now)
 *   u   = beta_t (v_t - r)                      (only what is new)
 *   S  <- S + k_t^T u                           (outer-product write)
 *   o_t = q_t S                                 (read after the write)
 * g may be NULL (ungated, decay 1).  S0 may be NULL (zero state) and may alias
 * S_out.  o and S_out may be NULL if not wanted.  A decode step is this loop
 * with T = 1 and S0 = the carried state.
 */
int orc_delta_recurrent(int B, int H, int T, int dk, int dv,
                        const void *q, const void *k, const void *v,
                        const void *beta, const void *g, int g_per_channel,
                        int dt, const double *S0, double *o, double *S_out,
                        int nthreads)
{
    int fail = 0;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; bh++) {
        double *S = malloc(sizeof(double) * (size_t)dk * dv);
        double *kt = malloc(sizeof(double) * (size_t)dk);
        double *qt = malloc(sizeof(double) * (size_t)dk);
        double *r = malloc(sizeof(double) * (size_t)dv);
        double *u = malloc(sizeof(double) * (size_t)dv);
        if (!S || !kt || !qt || !r || !u) {
#pragma omp atomic write
            fail = 1;
            free(S); free(kt); free(qt); free(r); free(u);
            continue;
        }
        const size_t sbase = (size_t)bh * dk * dv;
        for (size_t i = 0; i < (size_t)dk * dv; i++)
            S[i] = S0 ? S0[sbase + i] : 0.0;

        for (int t = 0; t < T; t++) {
            const size_t qk_row = ((size_t)bh * T + t) * dk;
            const size_t v_row = ((size_t)bh * T + t) * dv;
            const double b = rd(beta, (size_t)bh * T + t, dt);
            if (g) {
                for (int i = 0; i < dk; i++) {
                    const double a = g_per_channel ? exp(rd(g, qk_row + i, dt))
                                                   : exp(rd(g, (size_t)bh * T + t, dt));
                    for (int j = 0; j < dv; j++)
                        S[(size_t)i * dv + j] *= a;
                }
            }
            for (int i = 0; i < dk; i++) {
                kt[i] = rd(k, qk_row + i, dt);
                qt[i] = rd(q, qk_row + i, dt);
            }
            /* r = k S (sum over key rows i, in order) */
            for (int j = 0; j < dv; j++)
                r[j] = 0.0;
            for (int i = 0; i < dk; i++)
                for (int j = 0; j < dv; j++)
                    r[j] += kt[i] * S[(size_t)i * dv + j];
            for (int j = 0; j < dv; j++)
                u[j] = b * (rd(v, v_row + j, dt) - r[j]);
            for (int i = 0; i < dk; i++)
                for (int j = 0; j < dv; j++)
                    S[(size_t)i * dv + j] += kt[i] * u[j];
            /* o = q S with the updated state */
            if (o) {
                for (int j = 0; j < dv; j++)
                    o[v_row + j] = 0.0;
                for (int i = 0; i < dk; i++)
                    for (int j = 0; j < dv; j++)
                        o[v_row + j] += qt[i] * S[(size_t)i * dv + j];
            }
        }
        if (S_out)
            memcpy(S_out + sbase, S, sizeof(double) * (size_t)dk * dv);
        free(S); free(kt); free(qt); free(r); free(u);
    }
    return fail ? -1 : 0;
}

/*
 * Gated linear attention (the additive cache with a forgetting factor), one
 * token at a time:
 *   (gated only)  S <- exp(g_t) S              one scalar per token
 *   S   <- S + k_t^T v_t                        (outer-product write)
 *   o_t = q_t S                                 (read after the write)
 * q and k are used as given.  g [B,H,T] may be NULL (no decay).  S0 may be
 * NULL (zero state) and may alias S_out; o and S_out may be NULL.
 */
int orc_gla_recurrent(int B, int H, int T, int dk, int dv,
                      const void *q, const void *k, const void *v,
                      const void *g, int dt, const double *S0, double *o,
                      double *S_out, int nthreads)
{
    int fail = 0;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; bh++) {
        double *S = malloc(sizeof(double) * (size_t)dk * dv);
        double *kt = malloc(sizeof(double) * (size_t)dk);
        double *vt = malloc(sizeof(double) * (size_t)dv);
        if (!S || !kt || !vt) {
#pragma omp atomic write
            fail = 1;
            free(S); free(kt); free(vt);
            continue;
        }
        const size_t sbase = (size_t)bh * dk * dv;
        for (size_t i = 0; i < (size_t)dk * dv; i++)
            S[i] = S0 ? S0[sbase + i] : 0.0;

        for (int t = 0; t < T; t++) {
            const size_t qk_row = ((size_t)bh * T + t) * dk;
            const size_t v_row = ((size_t)bh * T + t) * dv;
            if (g) {
                const double a = exp(rd(g, (size_t)bh * T + t, dt));
                for (size_t i = 0; i < (size_t)dk * dv; i++)
                    S[i] *= a;
            }
            for (int i = 0; i < dk; i++)
                kt[i] = rd(k, qk_row + i, dt);
            for (int j = 0; j < dv; j++)
                vt[j] = rd(v, v_row + j, dt);
            for (int i = 0; i < dk; i++)
                for (int j = 0; j < dv; j++)
                    S[(size_t)i * dv + j] += kt[i] * vt[j];
            if (o) {
                for (int j = 0; j < dv; j++)
                    o[v_row + j] = 0.0;
                for (int i = 0; i < dk; i++) {
                    const double qi = rd(q, qk_row + i, dt);
                    for (int j = 0; j < dv; j++)
                        o[v_row + j] += qi * S[(size_t)i * dv + j];
                }
            }
        }
        if (S_out)
            memcpy(S_out + sbase, S, sizeof(double) * (size_t)dk * dv);
        free(S); free(kt); free(vt);
    }
    return fail ? -1 : 0;
}

/* ga[i] = exp(g) of token tok (tok = bh * T + t) for key row i: one gate per
 * token, or one per key channel; 1 without a gate */
static void decay_row(const void *g, int per_channel, int dt, size_t tok, int dk, double *ga)
{
    for (int i = 0; i < dk; i++)
        ga[i] = !g ? 1.0 : exp(rd(g, per_channel ? tok * (size_t)dk + i : tok, dt));
}

/*
 * Reverse-mode gradient of the ungated delta rule, one token at a time, for
 * the loss  sum_t do_t . o_t + sum dS_T * S_T  (do the output gradient, dS_T
 * the gradient of the final state).  Forward, per token: u = beta (v - S^T k),
 * S' = S + k u^T, o = S'^T q.  Backward, walking t from T-1 down to 0 with dS
 * the gradient of the state after token t:
 *   dS  += q do^T                       (o = S'^T q)
 *   dq   = S' do
 *   du   = dS^T k                       (S' = S + k u^T)
 *   dk   = dS u
 *   dv   = beta du                      (u = beta (v - S^T k))
 *   dbeta= du . (v - S^T k)
 *   dr   = -beta du                     (r = S^T k)
 *   dk  += S dr ;  dS += k dr^T         (the gradient of the state before t)
 * With a gate g (the decays of sections "Gated Delta Net" and "KDA / Kimi
 * Linear", as in orc_delta_recurrent: S_a = exp(g_t) S, one scalar per token,
 * or row i of S times exp(g_t,i), one per key channel), the steps above run
 * on the decayed state S_a in place of S, and then
 *   dg   = sum of dS_a * S_a            (over the whole state per token, over
 *                                        row i per key channel)
 *   dS   = exp(g_t) dS_a                (row-wise per key channel)
 * where dS_a is the gradient left after the last step above.
 * The states before every token are kept (recomputed forward), so memory is
 * T * dk * dv doubles per head: for small cases only.  S0 may be NULL (zero
 * start), dST may be NULL (no final-state gradient), g may be NULL (no gate;
 * dg is then not written).  dO has the inputs' dtype.  Outputs (float64): dq,
 * dk [B,H,T,dk], dv [B,H,T,dv], dbeta [B,H,T], dS0 [B,H,dk,dv], dg with g's
 * shape (any may be NULL).  Returns 0, or -1 on allocation failure.
 */
int orc_delta_backward(int B, int H, int T, int dk, int dv,
                       const void *q, const void *k, const void *v,
                       const void *beta, const void *g, int g_per_channel,
                       int dt, const double *S0,
                       const void *dO, const double *dST,
                       double *dq, double *dkk, double *dvv, double *dbeta,
                       double *dS0, double *dg, int nthreads)
{
    int fail = 0;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; bh++) {
        const size_t ss = (size_t)dk * dv;
        double *Sall = malloc(sizeof(double) * ss * ((size_t)T + 1));
        double *dS = malloc(sizeof(double) * ss);
        double *kt = malloc(sizeof(double) * (size_t)dk);
        double *r = malloc(sizeof(double) * (size_t)dv);
        double *u = malloc(sizeof(double) * (size_t)dv);
        double *du = malloc(sizeof(double) * (size_t)dv);
        double *dov = malloc(sizeof(double) * (size_t)dv);
        double *Sa = malloc(sizeof(double) * ss);
        double *ga = malloc(sizeof(double) * (size_t)dk);
        if (!Sall || !dS || !kt || !r || !u || !du || !dov || !Sa || !ga) {
#pragma omp atomic write
            fail = 1;
            free(Sall); free(dS); free(kt); free(r); free(u); free(du); free(dov);
            free(Sa); free(ga);
            continue;
        }
        const size_t sbase = (size_t)bh * ss;
        /* forward: Sall[t] is the state before token t, Sall[T] the final one */
        for (size_t i = 0; i < ss; i++)
            Sall[i] = S0 ? S0[sbase + i] : 0.0;
        for (int t = 0; t < T; t++) {
            double *Sn = Sall + (size_t)(t + 1) * ss;
            const size_t qk_row = ((size_t)bh * T + t) * dk;
            const size_t v_row = ((size_t)bh * T + t) * dv;
            const double b = rd(beta, (size_t)bh * T + t, dt);
            /* the decayed state S_a (S itself without a gate) */
            decay_row(g, g_per_channel, dt, (size_t)bh * T + t, dk, ga);
            for (int i = 0; i < dk; i++) {
                for (int j = 0; j < dv; j++)
                    Sa[(size_t)i * dv + j] = ga[i] * Sall[(size_t)t * ss + (size_t)i * dv + j];
            }
            for (int i = 0; i < dk; i++)
                kt[i] = rd(k, qk_row + i, dt);
            for (int j = 0; j < dv; j++) {
                r[j] = 0.0;
                for (int i = 0; i < dk; i++)
                    r[j] += Sa[(size_t)i * dv + j] * kt[i];
                u[j] = (rd(v, v_row + j, dt) - r[j]) * b;
            }
            for (int i = 0; i < dk; i++)
                for (int j = 0; j < dv; j++)
                    Sn[(size_t)i * dv + j] = Sa[(size_t)i * dv + j] + kt[i] * u[j];
        }
        /* backward */
        for (size_t i = 0; i < ss; i++)
            dS[i] = dST ? dST[sbase + i] : 0.0;
        for (int t = T - 1; t >= 0; t--) {
            const double *S = Sa;                           /* before token t, decayed */
            const double *Sn = Sall + (size_t)(t + 1) * ss; /* after token t */
            const size_t qk_row = ((size_t)bh * T + t) * dk;
            const size_t v_row = ((size_t)bh * T + t) * dv;
            const double b = rd(beta, (size_t)bh * T + t, dt);
            decay_row(g, g_per_channel, dt, (size_t)bh * T + t, dk, ga);
            for (int i = 0; i < dk; i++) {
                for (int j = 0; j < dv; j++)
                    Sa[(size_t)i * dv + j] = ga[i] * Sall[(size_t)t * ss + (size_t)i * dv + j];
            }
            for (int i = 0; i < dk; i++)
                kt[i] = rd(k, qk_row + i, dt);
            for (int j = 0; j < dv; j++)
                dov[j] = rd(dO, v_row + j, dt);
            /* o = S'^T q */
            for (int i = 0; i < dk; i++) {
                const double qa = rd(q, qk_row + i, dt);
                double acc = 0.0;
                for (int j = 0; j < dv; j++) {
                    dS[(size_t)i * dv + j] += qa * dov[j];
                    acc += Sn[(size_t)i * dv + j] * dov[j];
                }
                if (dq)
                    dq[qk_row + i] = acc;
            }
            /* recompute r and u of token t */
            for (int j = 0; j < dv; j++) {
                r[j] = 0.0;
                for (int i = 0; i < dk; i++)
                    r[j] += S[(size_t)i * dv + j] * kt[i];
                u[j] = (rd(v, v_row + j, dt) - r[j]) * b;
            }
            /* S' = S + k u^T */
            for (int j = 0; j < dv; j++) {
                du[j] = 0.0;
                for (int i = 0; i < dk; i++)
                    du[j] += dS[(size_t)i * dv + j] * kt[i];
            }
            double db = 0.0;
            for (int j = 0; j < dv; j++)
                db += du[j] * (rd(v, v_row + j, dt) - r[j]);
            if (dbeta)
                dbeta[(size_t)bh * T + t] = db;
            if (dvv)
                for (int j = 0; j < dv; j++)
                    dvv[v_row + j] = b * du[j];
            for (int i = 0; i < dk; i++) {
                double acc = 0.0;
                for (int j = 0; j < dv; j++)
                    acc += dS[(size_t)i * dv + j] * u[j] - b * S[(size_t)i * dv + j] * du[j];
                if (dkk)
                    dkk[qk_row + i] = acc;
            }
            /* the gradient of the decayed state: dS += k dr^T, dr = -b du */
            for (int i = 0; i < dk; i++)
                for (int j = 0; j < dv; j++)
                    dS[(size_t)i * dv + j] -= b * kt[i] * du[j];
            /* through the decay S_a = exp(g) S: dg, and the gradient of S */
            if (g) {
                double gsum = 0.0;
                for (int i = 0; i < dk; i++) {
                    double gi = 0.0;
                    for (int j = 0; j < dv; j++)
                        gi += dS[(size_t)i * dv + j] * Sa[(size_t)i * dv + j];
                    if (g_per_channel && dg)
                        dg[qk_row + i] = gi;
                    gsum += gi;
                    for (int j = 0; j < dv; j++)
                        dS[(size_t)i * dv + j] *= ga[i];
                }
                if (!g_per_channel && dg)
                    dg[(size_t)bh * T + t] = gsum;
            }
        }
        if (dS0)
            memcpy(dS0 + sbase, dS, sizeof(double) * ss);
        free(Sall); free(dS); free(kt); free(r); free(u); free(du); free(dov);
        free(Sa); free(ga);
    }
    return fail ? -1 : 0;
}

/*
 * The steps just before the delta rule in the layer of section "DeltaNet
 * (Fast Weight Programmers)": q and k are each passed through silu and then
 * L2-normalised over the head dimension (torch's F.normalize: x divided by
 * max(|x|_2, 1e-12)), and beta is the sigmoid of its logits, one per token,
 * shared by every head when the logits have a single head.
 *   orc_qk_prologue: x [rows, d] -> out = scale * n(s(x)), s = silu if
 *                    apply_silu else identity, n = the L2 normalisation.
 *   orc_beta_sigmoid: logits [B, Hb, T] (Hb = 1 or H) -> beta [B, H, T].
 */
int orc_qk_prologue(long rows, int d, const void *x, int dt, int apply_silu,
                    double scale, double *out)
{
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; r++) {
        double ss = 0.0;
        for (int i = 0; i < d; i++) {
            const double xi = rd(x, (size_t)r * d + i, dt);
            const double y = apply_silu ? xi / (1.0 + exp(-xi)) : xi;
            out[(size_t)r * d + i] = y;
            ss += y * y;
        }
        double nrm = sqrt(ss);
        if (nrm < 1e-12)
            nrm = 1e-12;
        for (int i = 0; i < d; i++)
            out[(size_t)r * d + i] = scale * out[(size_t)r * d + i] / nrm;
    }
    return 0;
}

int orc_beta_sigmoid(int B, int Hb, int H, int T, const void *logits, int dt,
                     double *beta)
{
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++)
            for (int t = 0; t < T; t++) {
                const int hs = Hb == 1 ? 0 : h;
                const double z = rd(logits, ((size_t)b * Hb + hs) * T + t, dt);
                beta[((size_t)b * H + h) * T + t] = 1.0 / (1.0 + exp(-z));
            }
    return 0;
}
