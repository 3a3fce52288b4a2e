/* oracle_driver.c -- runs every function of the fp64 oracle (oracle/la_oracle.c) on
 * small seeded inputs in exactly-sized heap buffers, so that an AddressSanitizer /
 * UndefinedBehaviorSanitizer build catches any out-of-bounds access or undefined
 * behaviour in its indexing, and checks a few of the oracle's pins on the way
 * (recurrent form = quadratic form, backward sweeps = quadratic backward, elu+1
 * given as features = the built-in map, a decode step = one more causal row).
 * Exit status 0: all checks passed and the sanitizers reported nothing. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "la_oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double rnd(void) { /* uniform in [-1, 1): a 64-bit LCG, inputs only */
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(g_state >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}
static double* arr(size_t n, int fill) {
    double* p = (double*)malloc((n ? n : 1) * sizeof(double));
    if (!p) exit(3);
    for (size_t i = 0; i < n; ++i) p[i] = fill ? 0.5 * rnd() : 0.0;
    return p;
}
static int g_fail = 0;
/* max |a - b| <= tol * max(max |b|, 1): inputs are of order 1, so an exactly-zero
 * reference (dq, dk at N = 1) is held to the same absolute scale. */
static void close_to(const char* what, const double* a, const double* b, size_t n, double tol) {
    double worst = 0.0, scale = 1.0;
    for (size_t i = 0; i < n; ++i) {
        const double e = fabs(a[i] - b[i]);
        if (!(e <= worst)) worst = e;
        if (fabs(b[i]) > scale) scale = fabs(b[i]);
    }
    if (!(worst <= tol * scale)) {
        fprintf(stderr, "FAIL %s: max abs diff %.3e (scale %.3e)\n", what, worst, scale);
        g_fail = 1;
    }
}

static void run(int64_t BH, int64_t N, int64_t d, int64_t m) {
    const size_t t = (size_t)(BH * N * d), h = (size_t)(BH * N), st = (size_t)(BH * d * d), zv = (size_t)(BH * d);
    double *q = arr(t, 1), *k = arr(t, 1), *v = arr(t, 1), *dout = arr(t, 1);
    double *o = arr(t, 0), *o2 = arr(t, 0), *den = arr(h, 0), *den2 = arr(h, 0), *S = arr(st, 0), *z = arr(zv, 0);
    double *dq = arr(t, 0), *dk = arr(t, 0), *dv = arr(t, 0), *dq2 = arr(t, 0), *dk2 = arr(t, 0), *dv2 = arr(t, 0);
    for (int causal = 0; causal < 2; ++causal) {
        if (causal) la_oracle_forward_causal(BH, N, d, q, k, v, o, den, S, z);
        else la_oracle_forward_noncausal(BH, N, d, q, k, v, o, den, S, z);
        la_oracle_quadratic_forward(BH, N, d, causal, q, k, v, o2, den2);
        close_to("forward: recurrent = quadratic", o, o2, t, 1e-12);
        close_to("den: recurrent = quadratic", den, den2, h, 1e-12);
        if (causal) la_oracle_backward_causal(BH, N, d, q, k, v, dout, dq, dk, dv);
        else la_oracle_backward_noncausal(BH, N, d, q, k, v, dout, dq, dk, dv);
        la_oracle_quadratic_backward(BH, N, d, causal, q, k, v, dout, dq2, dk2, dv2);
        close_to("dq: sweeps = quadratic", dq, dq2, t, 1e-10);
        close_to("dk: sweeps = quadratic", dk, dk2, t, 1e-10);
        close_to("dv: sweeps = quadratic", dv, dv2, t, 1e-10);
        /* elu + 1 given as features reproduces the built-in map */
        double *fq = arr(t, 0), *fk = arr(t, 0), *fo = arr(t, 0), *fden = arr(h, 0);
        double *fS = arr(st, 0), *fz = arr(zv, 0), *dfq = arr(t, 0), *dfk = arr(t, 0), *fdv = arr(t, 0);
        for (size_t i = 0; i < t; ++i) { fq[i] = la_oracle_phi(q[i]); fk[i] = la_oracle_phi(k[i]); }
        la_oracle_forward_features(BH, N, d, d, causal, fq, fk, v, fo, fden, fS, fz);
        close_to("features = built-in map", fo, o, t, 1e-12);
        la_oracle_backward_features(BH, N, d, d, causal, fq, fk, v, dout, dfq, dfk, fdv);
        for (size_t i = 0; i < t; ++i) { dfq[i] *= la_oracle_dphi(q[i]); dfk[i] *= la_oracle_dphi(k[i]); }
        close_to("feature dq = dq", dfq, dq, t, 1e-10);
        close_to("feature dk = dk", dfk, dk, t, 1e-10);
        free(fq); free(fk); free(fo); free(fden); free(fS); free(fz); free(dfq); free(dfk); free(fdv);
    }
    /* start states, upstream state gradients, and one decode step continuing the sequence */
    double *S0 = arr(st, 1), *z0 = arr(zv, 0), *dSN = arr(st, 1), *dzN = arr(zv, 1), *dS0 = arr(st, 0), *dz0 = arr(zv, 0);
    for (size_t i = 0; i < zv; ++i) z0[i] = 1.0 + fabs(rnd());
    la_oracle_forward_causal_from(BH, N, d, S0, z0, q, k, v, o, den, S, z);
    la_oracle_backward_causal_state(BH, N, d, q, k, v, dout, S0, z0, dSN, dzN, dq, dk, dv, dS0, dz0);
    la_oracle_backward_causal_state(BH, N, d, q, k, v, dout, NULL, NULL, NULL, NULL, dq2, dk2, dv2, NULL, NULL);
    la_oracle_backward_causal(BH, N, d, q, k, v, dout, dq, dk, dv);
    close_to("state backward from zero = backward", dq2, dq, t, 1e-12);
    {
        double *dq_ = arr((size_t)(BH * d), 1), *dk_ = arr((size_t)(BH * d), 1), *dv_ = arr((size_t)(BH * d), 1);
        double* dov = arr((size_t)(BH * d), 0);
        double *S1 = arr(st, 0), *z1 = arr(zv, 0);
        la_oracle_forward_causal(BH, N, d, q, k, v, o, den, S1, z1);
        la_oracle_decode_step(BH, d, S1, z1, dq_, dk_, dv_, dov);
        free(dq_); free(dk_); free(dv_); free(dov); free(S1); free(z1);
    }
    /* FAVOR+ features (m random directions) and their gradient */
    {
        const size_t fx = (size_t)(BH * N * m);
        double *om = arr((size_t)(m * d), 1), *F = arr(fx, 0), *dF = arr(fx, 1), *dx = arr(t, 0);
        la_oracle_favor_features(BH * N, d, m, q, om, F);
        la_oracle_favor_features_backward(BH * N, d, m, q, om, dF, dx);
        double *Fk = arr(fx, 0), *fo = arr(t, 0), *fden = arr(h, 0), *fS = arr((size_t)(BH * m * d), 0);
        double *fz = arr((size_t)(BH * m), 0), *dfq = arr(fx, 0), *dfk = arr(fx, 0), *fdv = arr(t, 0);
        la_oracle_favor_features(BH * N, d, m, k, om, Fk);
        for (int causal = 0; causal < 2; ++causal) {
            la_oracle_forward_features(BH, N, m, d, causal, F, Fk, v, fo, fden, fS, fz);
            la_oracle_backward_features(BH, N, m, d, causal, F, Fk, v, dout, dfq, dfk, fdv);
        }
        free(om); free(F); free(dF); free(dx); free(Fk); free(fo); free(fden); free(fS); free(fz); free(dfq);
        free(dfk); free(fdv);
    }
    free(S0); free(z0); free(dSN); free(dzN); free(dS0); free(dz0);
    free(q); free(k); free(v); free(dout); free(o); free(o2); free(den); free(den2); free(S); free(z);
    free(dq); free(dk); free(dv); free(dq2); free(dk2); free(dv2);
}

int main(void) {
    la_oracle_set_threads(2);
    const int64_t shapes[][4] = {{1, 1, 1, 3}, {3, 2, 1, 2}, {2, 37, 5, 10}, {1, 64, 8, 8}, {3, 65, 4, 12}};
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
        run(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3]);
    if (g_fail) return 1;
    printf("oracle driver: all checks passed\n");
    return 0;
}
