/* oracle_driver.c -- runs every oracle entry point under AddressSanitizer
 * and UndefinedBehaviorSanitizer on small seeded inputs (every stored
 * precision, ragged lengths, T = 0, with and without an initial state, both
 * gate layouts) and checks that the results are finite.  Test code: it
 * declares the oracle's functions itself. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_max_threads(void);
int orc_la_recurrent(int B, int H, int T, int dk, int dv, const void *q, const void *k, const void *v, int dt,
                     const double *S0, const double *z0, double *o, double *S_out, double *z_out, int nthreads);
int orc_delta_recurrent(int B, int H, int T, int dk, int dv, const void *q, const void *k, const void *v,
                        const void *beta, const void *g, int g_per_channel, int dt, const double *S0, double *o,
                        double *S_out, int nthreads);
int orc_gla_recurrent(int B, int H, int T, int dk, int dv, const void *q, const void *k, const void *v,
                      const void *g, int dt, const double *S0, double *o, double *S_out, int nthreads);
int orc_delta_backward(int B, int H, int T, int dk, int dv, const void *q, const void *k, const void *v,
                       const void *beta, const void *g, int g_per_channel, int dt, const double *S0,
                       const void *dO, const double *dST, double *dq, double *dkk, double *dvv, double *dbeta,
                       double *dS0, double *dg, int nthreads);
int orc_qk_prologue(long rows, int d, const void *x, int dt, int apply_silu, double scale, double *out);
int orc_beta_sigmoid(int B, int Hb, int H, int T, const void *logits, int dt, double *beta);

static uint64_t rng = 12345;
static double unif(void) { /* in (-1, 1) */
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (double)((rng * 2685821657736338717ull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

/* n values in stored precision dt (0 fp32, 1 bf16, 2 fp64), each lo + (hi - lo) * |u| */
static void *fill(size_t n, int dt, double lo, double hi) {
    size_t es = dt == 0 ? 4 : dt == 1 ? 2 : 8;
    unsigned char *p = malloc(n * es ? n * es : 1);
    for (size_t i = 0; i < n; i++) {
        double x = lo + (hi - lo) * fabs(unif());
        if (dt == 0) ((float *)p)[i] = (float)x;
        else if (dt == 2) ((double *)p)[i] = x;
        else { float f = (float)x; uint32_t b; memcpy(&b, &f, 4); ((uint16_t *)p)[i] = (uint16_t)(b >> 16); }
    }
    return p;
}
static double *dbl(size_t n) { return calloc(n ? n : 1, sizeof(double)); }
static int failures = 0;
static void finite(const double *x, size_t n, const char *what) {
    for (size_t i = 0; i < n; i++)
        if (!isfinite(x[i])) { fprintf(stderr, "%s: non-finite value at %zu\n", what, i); failures++; return; }
}

int main(void) {
    const int shapes[][5] = {{1, 1, 1, 4, 4}, {2, 3, 17, 8, 4}, {1, 2, 65, 16, 8}, {2, 1, 0, 4, 8}};
    for (int dt = 0; dt < 3; dt++)
        for (size_t si = 0; si < sizeof shapes / sizeof shapes[0]; si++) {
            const int B = shapes[si][0], H = shapes[si][1], T = shapes[si][2], dk = shapes[si][3], dv = shapes[si][4];
            const size_t nq = (size_t)B * H * T * dk, nv = (size_t)B * H * T * dv, nt = (size_t)B * H * T;
            const size_t ns = (size_t)B * H * dk * dv, nz = (size_t)B * H * dk;
            void *q = fill(nq, dt, -1, 1), *k = fill(nq, dt, -1, 1), *v = fill(nv, dt, -1, 1);
            void *beta = fill(nt, dt, 0, 1), *gt = fill(nt, dt, -0.5, 0), *gc = fill(nq, dt, -0.5, 0);
            void *dO = fill(nv, dt, -1, 1);
            double *S0 = dbl(ns), *z0 = dbl(nz), *dST = dbl(ns);
            for (size_t i = 0; i < ns; i++) { S0[i] = 0.1 * unif(); dST[i] = unif(); }
            for (size_t i = 0; i < nz; i++) z0[i] = 1.0 + fabs(unif());
            double *o = dbl(nv), *S = dbl(ns), *z = dbl(nz);
            for (int init = 0; init < 2; init++) {
                if (orc_la_recurrent(B, H, T, dk, dv, q, k, v, dt, init ? S0 : NULL, init ? z0 : NULL, o, S, z, 2))
                    failures++;
                finite(o, nv, "la o"); finite(S, ns, "la S"); finite(z, nz, "la z");
                for (int gm = 0; gm < 3; gm++) {
                    const void *g = gm == 0 ? NULL : gm == 1 ? gt : gc;
                    if (orc_delta_recurrent(B, H, T, dk, dv, q, k, v, beta, g, gm == 2, dt, init ? S0 : NULL, o, S, 2))
                        failures++;
                    finite(o, nv, "delta o"); finite(S, ns, "delta S");
                    double *dq = dbl(nq), *dk_ = dbl(nq), *dv_ = dbl(nv), *db = dbl(nt), *dS0 = dbl(ns);
                    double *dg = dbl(gm == 2 ? nq : nt);
                    if (orc_delta_backward(B, H, T, dk, dv, q, k, v, beta, g, gm == 2, dt, init ? S0 : NULL, dO,
                                           init ? dST : NULL, dq, dk_, dv_, db, dS0, g ? dg : NULL, 2))
                        failures++;
                    finite(dq, nq, "dq"); finite(dk_, nq, "dk"); finite(dv_, nv, "dv"); finite(db, nt, "dbeta");
                    finite(dS0, ns, "dS0");
                    if (g) finite(dg, gm == 2 ? nq : nt, "dg");
                    free(dq); free(dk_); free(dv_); free(db); free(dS0); free(dg);
                }
                if (orc_gla_recurrent(B, H, T, dk, dv, q, k, v, init ? gt : NULL, dt, init ? S0 : NULL, o, S, 2))
                    failures++;
                finite(o, nv, "gla o"); finite(S, ns, "gla S");
            }
            double *pq = dbl(nq);
            if (orc_qk_prologue((long)B * H * T, dk, q, dt, 1, 0.5, pq)) failures++;
            finite(pq, nq, "prologue");
            double *pb = dbl(nt);
            if (orc_beta_sigmoid(B, 1, H, T, beta, dt, pb)) failures++;
            finite(pb, nt, "beta");
            free(pq); free(pb);
            free(q); free(k); free(v); free(beta); free(gt); free(gc); free(dO);
            free(S0); free(z0); free(dST); free(o); free(S); free(z);
        }
    if (orc_max_threads() < 1) failures++;
    if (failures) { fprintf(stderr, "%d failure(s)\n", failures); return 1; }
    printf("oracle driver: every entry point ran, no sanitizer report\n");
    return 0;
}
