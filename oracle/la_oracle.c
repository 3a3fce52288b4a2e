/*
 * la_oracle.c -- fp64 CPU oracle for kernelized linear attention.
 *
 * TEST INFRASTRUCTURE ONLY (see la_oracle.h): used by the tests, the smoke
 * check and the CPU-baseline leg of the benchmark, never by the product path.
 *
 * Each function follows one passage of the page "Efficient Transformers Survey"
 * (economicspath.com), section "Linear Attention", Proposition "Linear
 * Attention via Kernel Decomposition", or the chain rule applied to it.  Loops
 * are written out plainly, per head, in fp64, with no blocking or reordering
 * beyond what the cited formula states.  Heads are independent and run in
 * parallel (OpenMP); nothing inside a head is parallel.
 */
#include "la_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 0;

void la_oracle_set_threads(int n) { g_threads = n; }

int la_oracle_get_threads(void) {
#ifdef _OPENMP
    return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
    return 1;
#endif
}

/* phi(x) = elu(x) + 1 (ELU with alpha = 1): x + 1 for x > 0, exp(x) otherwise.
 * Positive everywhere, so every denominator below is positive. */
double la_oracle_phi(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

/* d phi / dx: 1 for x > 0, exp(x) otherwise (both branches agree at 0). */
double la_oracle_dphi(double x) { return x > 0.0 ? 1.0 : exp(x); }

static double* zalloc(int64_t n) { return (double*)calloc((size_t)(n > 0 ? n : 1), sizeof(double)); }

/* ---- forward, non-causal --------------------------------------------------
 * Statement of the proposition: S = sum_j phi(K_j) V_j^T, z = sum_j phi(K_j),
 * Attn_i = phi(Q_i)^T S / phi(Q_i)^T z. */
static void fwd_noncausal_head(int64_t N, int64_t d, const double* q, const double* k,
                               const double* v, double* o, double* den_out, double* S_out,
                               double* z_out) {
    double* S = zalloc(d * d);
    double* z = zalloc(d);
    double* f = zalloc(d);
    for (int64_t j = 0; j < N; ++j) {
        for (int64_t a = 0; a < d; ++a) f[a] = la_oracle_phi(k[j * d + a]);
        for (int64_t a = 0; a < d; ++a) {
            z[a] += f[a];
            for (int64_t b = 0; b < d; ++b) S[a * d + b] += f[a] * v[j * d + b];
        }
    }
    for (int64_t i = 0; i < N; ++i) {
        for (int64_t a = 0; a < d; ++a) f[a] = la_oracle_phi(q[i * d + a]);
        double den = 0.0;
        for (int64_t a = 0; a < d; ++a) den += f[a] * z[a];
        for (int64_t b = 0; b < d; ++b) {
            double num = 0.0;
            for (int64_t a = 0; a < d; ++a) num += f[a] * S[a * d + b];
            o[i * d + b] = num / den;
        }
        if (den_out) den_out[i] = den;
    }
    if (S_out) memcpy(S_out, S, (size_t)(d * d) * sizeof(double));
    if (z_out) memcpy(z_out, z, (size_t)d * sizeof(double));
    free(S);
    free(z);
    free(f);
}

void la_oracle_forward_noncausal(int64_t BH, int64_t N, int64_t d, const double* q,
                                 const double* k, const double* v, double* o, double* den_out,
                                 double* S_out, double* z_out) {
    int nt = la_oracle_get_threads();
    (void)nt;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        const int64_t off = h * N * d;
        fwd_noncausal_head(N, d, q + off, k + off, v + off, o + off,
                           den_out ? den_out + h * N : NULL, S_out ? S_out + h * d * d : NULL,
                           z_out ? z_out + h * d : NULL);
    }
}

/* ---- forward, causal (recurrent) ------------------------------------------
 * "Why it matters": tokens are processed one by one, S and z are updated
 * incrementally.  Row i reads the state after token i has been added.  The
 * recurrence starts from (S0, z0) when given (the state a previous call left,
 * as when a long sequence is processed piece by piece), else from zero. */
static void fwd_causal_head(int64_t N, int64_t d, const double* S0, const double* z0,
                            const double* q, const double* k, const double* v, double* o,
                            double* den_out, double* S_out, double* z_out) {
    double* S = zalloc(d * d);
    double* z = zalloc(d);
    double* f = zalloc(d);
    if (S0) memcpy(S, S0, (size_t)(d * d) * sizeof(double));
    if (z0) memcpy(z, z0, (size_t)d * sizeof(double));
    for (int64_t i = 0; i < N; ++i) {
        for (int64_t a = 0; a < d; ++a) f[a] = la_oracle_phi(k[i * d + a]);
        for (int64_t a = 0; a < d; ++a) {
            z[a] += f[a];
            for (int64_t b = 0; b < d; ++b) S[a * d + b] += f[a] * v[i * d + b];
        }
        for (int64_t a = 0; a < d; ++a) f[a] = la_oracle_phi(q[i * d + a]);
        double den = 0.0;
        for (int64_t a = 0; a < d; ++a) den += f[a] * z[a];
        for (int64_t b = 0; b < d; ++b) {
            double num = 0.0;
            for (int64_t a = 0; a < d; ++a) num += f[a] * S[a * d + b];
            o[i * d + b] = num / den;
        }
        if (den_out) den_out[i] = den;
    }
    if (S_out) memcpy(S_out, S, (size_t)(d * d) * sizeof(double));
    if (z_out) memcpy(z_out, z, (size_t)d * sizeof(double));
    free(S);
    free(z);
    free(f);
}

void la_oracle_forward_causal_from(int64_t BH, int64_t N, int64_t d, const double* S0,
                                   const double* z0, const double* q, const double* k,
                                   const double* v, double* o, double* den_out, double* S_out,
                                   double* z_out) {
    int nt = la_oracle_get_threads();
    (void)nt;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        const int64_t off = h * N * d;
        fwd_causal_head(N, d, S0 ? S0 + h * d * d : NULL, z0 ? z0 + h * d : NULL, q + off, k + off,
                        v + off, o + off, den_out ? den_out + h * N : NULL,
                        S_out ? S_out + h * d * d : NULL, z_out ? z_out + h * d : NULL);
    }
}

void la_oracle_forward_causal(int64_t BH, int64_t N, int64_t d, const double* q,
                              const double* k, const double* v, double* o, double* den_out,
                              double* S_out, double* z_out) {
    la_oracle_forward_causal_from(BH, N, d, NULL, NULL, q, k, v, o, den_out, S_out, z_out);
}

/* ---- backward --------------------------------------------------------------
 * Chain rule through Attn_i = num_i / den_i with num_i = sum_j A_ij V_j,
 * den_i = sum_j A_ij, A_ij = phi(Q_i) . phi(K_j) (j <= i when causal):
 *   G_i  = dL/dnum_i = dO_i / den_i
 *   g_i  = dL/dden_i = -(dO_i . O_i) / den_i = -G_i . O_i
 *   dA_ij = G_i . V_j + g_i
 *   dphi(Q_i) = sum_j dA_ij phi(K_j)  = S_i G_i + g_i z_i       (prefix state)
 *   dphi(K_j) = sum_i dA_ij phi(Q_i)  = R_j V_j + r_j           (suffix state)
 *   dV_j      = sum_i A_ij G_i        = R_j^T phi(K_j)
 * with R_j = sum_{i >= j} phi(Q_i) G_i^T and r_j = sum_{i >= j} g_i phi(Q_i)
 * (all i for the non-causal form), then dQ = dphi(Q) * phi'(Q) and
 * dK = dphi(K) * phi'(K) elementwise. */
/* With a start state (causal only): the forward's recurrence starts from
 * (S0, z0), and the loss may also depend on the final state (S_N, z_N) with
 * upstream gradients (dSN, dzN).  S_N = S0 + sum_j phi(K_j) V_j^T, so dSN adds
 * to every suffix sum R_j and dzN to every r_j, i.e. the suffix sums start from
 * (dSN, dzN); and S_i = S0 + ..., so the gradient reaching S0 (and z0) is the
 * suffix sum at the first token, R_0 (r_0).  Any of these may be NULL (zero; no
 * output). */
static void bwd_head_state(int64_t N, int64_t d, int causal, const double* q, const double* k,
                           const double* v, const double* dout, const double* S0, const double* z0,
                           const double* dSN, const double* dzN, double* dq, double* dk, double* dv,
                           double* dS0, double* dz0) {
    double* S = zalloc(d * d);
    double* z = zalloc(d);
    double* R = zalloc(d * d);
    double* r = zalloc(d);
    if (S0) memcpy(S, S0, (size_t)(d * d) * sizeof(double));
    if (z0) memcpy(z, z0, (size_t)d * sizeof(double));
    if (dSN) memcpy(R, dSN, (size_t)(d * d) * sizeof(double));
    if (dzN) memcpy(r, dzN, (size_t)d * sizeof(double));
    double* f = zalloc(d);
    double* kf = zalloc(d);
    double* O = zalloc(d);
    double* G = zalloc(N * d);
    double* g = zalloc(N);

    if (!causal) { /* global state first */
        for (int64_t j = 0; j < N; ++j) {
            for (int64_t a = 0; a < d; ++a) kf[a] = la_oracle_phi(k[j * d + a]);
            for (int64_t a = 0; a < d; ++a) {
                z[a] += kf[a];
                for (int64_t b = 0; b < d; ++b) S[a * d + b] += kf[a] * v[j * d + b];
            }
        }
    }
    /* prefix sweep: recompute O_i, den_i from the state, then G_i, g_i, dQ_i */
    for (int64_t i = 0; i < N; ++i) {
        if (causal) {
            for (int64_t a = 0; a < d; ++a) kf[a] = la_oracle_phi(k[i * d + a]);
            for (int64_t a = 0; a < d; ++a) {
                z[a] += kf[a];
                for (int64_t b = 0; b < d; ++b) S[a * d + b] += kf[a] * v[i * d + b];
            }
        }
        for (int64_t a = 0; a < d; ++a) f[a] = la_oracle_phi(q[i * d + a]);
        double den = 0.0;
        for (int64_t a = 0; a < d; ++a) den += f[a] * z[a];
        double dot = 0.0;
        for (int64_t b = 0; b < d; ++b) {
            double num = 0.0;
            for (int64_t a = 0; a < d; ++a) num += f[a] * S[a * d + b];
            O[b] = num / den;
            G[i * d + b] = dout[i * d + b] / den;
            dot += G[i * d + b] * O[b];
        }
        g[i] = -dot;
        for (int64_t a = 0; a < d; ++a) {
            double s = g[i] * z[a];
            for (int64_t b = 0; b < d; ++b) s += S[a * d + b] * G[i * d + b];
            dq[i * d + a] = s * la_oracle_dphi(q[i * d + a]);
        }
    }
    if (!causal) { /* global suffix sums */
        for (int64_t i = 0; i < N; ++i) {
            for (int64_t a = 0; a < d; ++a) f[a] = la_oracle_phi(q[i * d + a]);
            for (int64_t a = 0; a < d; ++a) {
                r[a] += g[i] * f[a];
                for (int64_t b = 0; b < d; ++b) R[a * d + b] += f[a] * G[i * d + b];
            }
        }
    }
    /* suffix sweep: R, r accumulate rows i >= j (causal), then dK_j, dV_j */
    for (int64_t j = N - 1; j >= 0; --j) {
        if (causal) {
            for (int64_t a = 0; a < d; ++a) f[a] = la_oracle_phi(q[j * d + a]);
            for (int64_t a = 0; a < d; ++a) {
                r[a] += g[j] * f[a];
                for (int64_t b = 0; b < d; ++b) R[a * d + b] += f[a] * G[j * d + b];
            }
        }
        for (int64_t a = 0; a < d; ++a) kf[a] = la_oracle_phi(k[j * d + a]);
        for (int64_t a = 0; a < d; ++a) {
            double s = r[a];
            for (int64_t b = 0; b < d; ++b) s += R[a * d + b] * v[j * d + b];
            dk[j * d + a] = s * la_oracle_dphi(k[j * d + a]);
        }
        for (int64_t b = 0; b < d; ++b) {
            double s = 0.0;
            for (int64_t a = 0; a < d; ++a) s += R[a * d + b] * kf[a];
            dv[j * d + b] = s;
        }
    }
    if (dS0) memcpy(dS0, R, (size_t)(d * d) * sizeof(double));
    if (dz0) memcpy(dz0, r, (size_t)d * sizeof(double));
    free(S);
    free(z);
    free(R);
    free(r);
    free(f);
    free(kf);
    free(O);
    free(G);
    free(g);
}

static void bwd_head(int64_t N, int64_t d, int causal, const double* q, const double* k,
                     const double* v, const double* dout, double* dq, double* dk, double* dv) {
    bwd_head_state(N, d, causal, q, k, v, dout, NULL, NULL, NULL, NULL, dq, dk, dv, NULL, NULL);
}

void la_oracle_backward_causal_state(int64_t BH, int64_t N, int64_t d, const double* q,
                                     const double* k, const double* v, const double* dout,
                                     const double* S0, const double* z0, const double* dSN,
                                     const double* dzN, double* dq, double* dk, double* dv,
                                     double* dS0, double* dz0) {
    int nt = la_oracle_get_threads();
    (void)nt;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        const int64_t off = h * N * d, so = h * d * d, zo = h * d;
        bwd_head_state(N, d, 1, q + off, k + off, v + off, dout + off, S0 ? S0 + so : NULL,
                       z0 ? z0 + zo : NULL, dSN ? dSN + so : NULL, dzN ? dzN + zo : NULL, dq + off,
                       dk + off, dv + off, dS0 ? dS0 + so : NULL, dz0 ? dz0 + zo : NULL);
    }
}

void la_oracle_backward_causal(int64_t BH, int64_t N, int64_t d, const double* q,
                               const double* k, const double* v, const double* dout, double* dq,
                               double* dk, double* dv) {
    int nt = la_oracle_get_threads();
    (void)nt;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        const int64_t off = h * N * d;
        bwd_head(N, d, 1, q + off, k + off, v + off, dout + off, dq + off, dk + off, dv + off);
    }
}

void la_oracle_backward_noncausal(int64_t BH, int64_t N, int64_t d, const double* q,
                                  const double* k, const double* v, const double* dout, double* dq,
                                  double* dk, double* dv) {
    int nt = la_oracle_get_threads();
    (void)nt;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        const int64_t off = h * N * d;
        bwd_head(N, d, 0, q + off, k + off, v + off, dout + off, dq + off, dk + off, dv + off);
    }
}

/* ---- decode ----------------------------------------------------------------
 * One step of the recurrence: add the new token to (S, z), then read. */
void la_oracle_decode_step(int64_t BH, int64_t d, double* S, double* z, const double* q,
                           const double* k, const double* v, double* o) {
    int nt = la_oracle_get_threads();
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        double* Sh = S + h * d * d;
        double* zh = z + h * d;
        const double* qh = q + h * d;
        const double* kh = k + h * d;
        const double* vh = v + h * d;
        double* oh = o + h * d;
        for (int64_t a = 0; a < d; ++a) {
            double kf = la_oracle_phi(kh[a]);
            zh[a] += kf;
            for (int64_t b = 0; b < d; ++b) Sh[a * d + b] += kf * vh[b];
        }
        double den = 0.0;
        for (int64_t a = 0; a < d; ++a) den += la_oracle_phi(qh[a]) * zh[a];
        for (int64_t b = 0; b < d; ++b) {
            double num = 0.0;
            for (int64_t a = 0; a < d; ++a) num += la_oracle_phi(qh[a]) * Sh[a * d + b];
            oh[b] = num / den;
        }
    }
}

/* ---- quadratic forms ---------------------------------------------------------
 * Proof sketch: Attn_i = sum_j k(Q_i,K_j) V_j / sum_j k(Q_i,K_j) with
 * k(q,k) = phi(q) . phi(k); the n x n weights are formed explicitly. */
static double kern(int64_t d, const double* qi, const double* kj) {
    double s = 0.0;
    for (int64_t a = 0; a < d; ++a) s += la_oracle_phi(qi[a]) * la_oracle_phi(kj[a]);
    return s;
}

void la_oracle_quadratic_forward(int64_t BH, int64_t N, int64_t d, int causal, const double* q,
                                 const double* k, const double* v, double* o, double* den_out) {
    for (int64_t h = 0; h < BH; ++h) {
        const double* qh = q + h * N * d;
        const double* kh = k + h * N * d;
        const double* vh = v + h * N * d;
        double* oh = o + h * N * d;
        for (int64_t i = 0; i < N; ++i) {
            const int64_t jend = causal ? i + 1 : N;
            double den = 0.0;
            for (int64_t b = 0; b < d; ++b) oh[i * d + b] = 0.0;
            for (int64_t j = 0; j < jend; ++j) {
                double w = kern(d, qh + i * d, kh + j * d);
                den += w;
                for (int64_t b = 0; b < d; ++b) oh[i * d + b] += w * vh[j * d + b];
            }
            for (int64_t b = 0; b < d; ++b) oh[i * d + b] /= den;
            if (den_out) den_out[h * N + i] = den;
        }
    }
}

/* Quadratic backward: the n x n weights A_ij and their gradient
 * dA_ij = G_i . (V_j - O_i) are formed explicitly, then
 * dphi(Q_i) = sum_j dA_ij phi(K_j), dphi(K_j) = sum_i dA_ij phi(Q_i),
 * dV_j = sum_i A_ij G_i. */
void la_oracle_quadratic_backward(int64_t BH, int64_t N, int64_t d, int causal, const double* q,
                                  const double* k, const double* v, const double* dout, double* dq,
                                  double* dk, double* dv) {
    double* O = zalloc(N * d);
    double* den = zalloc(N);
    double* A = zalloc(N * N);
    double* dA = zalloc(N * N);
    for (int64_t h = 0; h < BH; ++h) {
        const double* qh = q + h * N * d;
        const double* kh = k + h * N * d;
        const double* vh = v + h * N * d;
        const double* doh = dout + h * N * d;
        double* dqh = dq + h * N * d;
        double* dkh = dk + h * N * d;
        double* dvh = dv + h * N * d;
        la_oracle_quadratic_forward(1, N, d, causal, qh, kh, vh, O, den);
        for (int64_t i = 0; i < N; ++i)
            for (int64_t j = 0; j < N; ++j) {
                const int live = !causal || j <= i;
                A[i * N + j] = live ? kern(d, qh + i * d, kh + j * d) : 0.0;
                double s = 0.0;
                if (live)
                    for (int64_t b = 0; b < d; ++b)
                        s += doh[i * d + b] / den[i] * (vh[j * d + b] - O[i * d + b]);
                dA[i * N + j] = s;
            }
        for (int64_t i = 0; i < N; ++i)
            for (int64_t a = 0; a < d; ++a) {
                double s = 0.0;
                for (int64_t j = 0; j < N; ++j) s += dA[i * N + j] * la_oracle_phi(kh[j * d + a]);
                dqh[i * d + a] = s * la_oracle_dphi(qh[i * d + a]);
            }
        for (int64_t j = 0; j < N; ++j) {
            for (int64_t a = 0; a < d; ++a) {
                double s = 0.0;
                for (int64_t i = 0; i < N; ++i) s += dA[i * N + j] * la_oracle_phi(qh[i * d + a]);
                dkh[j * d + a] = s * la_oracle_dphi(kh[j * d + a]);
            }
            for (int64_t b = 0; b < d; ++b) {
                double s = 0.0;
                for (int64_t i = 0; i < N; ++i) s += A[i * N + j] * doh[i * d + b] / den[i];
                dvh[j * d + b] = s;
            }
        }
    }
    free(O);
    free(den);
    free(A);
    free(dA);
}

/* ---- FAVOR+ positive random features ------------------------------------------
 * Page "Efficient Transformers Survey", section on Performer (FAVOR+):
 *   phi(x) = m^{-1/2} exp(-|x|^2 / 2) [exp(w_1 . x), ..., exp(w_m . x)],
 * w_i ~ N(0, I_d) given as the rows of omega [m][d]; x is taken as given (any
 * 1/sqrt(d) scaling is the caller's pre-normalization). */
void la_oracle_favor_features(int64_t rows, int64_t d, int64_t m, const double* x, const double* omega,
                              double* out) {
    const double c = 1.0 / sqrt((double)m);
    for (int64_t r = 0; r < rows; ++r) {
        const double* xr = x + r * d;
        double nrm = 0.0;
        for (int64_t a = 0; a < d; ++a) nrm += xr[a] * xr[a];
        for (int64_t i = 0; i < m; ++i) {
            double u = 0.0;
            for (int64_t a = 0; a < d; ++a) u += omega[i * d + a] * xr[a];
            out[r * m + i] = c * exp(u - 0.5 * nrm);
        }
    }
}

/* ---- linear attention on given features ----------------------------------------
 * The Statement of the linear-attention proposition with the feature map
 * applied beforehand: fq = phi(Q) [N][m], fk = phi(K) [N][m], V [N][dv],
 *   S = sum_j fk_j V_j^T (m x dv), z = sum_j fk_j, O_i = fq_i^T S / fq_i^T z,
 * the sums over all j (causal == 0) or j <= i with the state updated before the
 * read (causal != 0, the recurrent form of "Why It Matters"). */
void la_oracle_forward_features(int64_t BH, int64_t N, int64_t m, int64_t dv, int causal,
                                const double* fq, const double* fk, const double* v, double* o,
                                double* den_out, double* S_out, double* z_out) {
    int nt = la_oracle_get_threads();
    (void)nt;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        const double* qh = fq + h * N * m;
        const double* kh = fk + h * N * m;
        const double* vh = v + h * N * dv;
        double* oh = o + h * N * dv;
        double* S = zalloc(m * dv);
        double* z = zalloc(m);
        int64_t added = 0; /* keys folded into (S, z) so far */
        for (int64_t i = 0; i < N; ++i) {
            const int64_t upto = causal ? i + 1 : N;
            for (; added < upto; ++added) {
                for (int64_t a = 0; a < m; ++a) {
                    z[a] += kh[added * m + a];
                    for (int64_t b = 0; b < dv; ++b) S[a * dv + b] += kh[added * m + a] * vh[added * dv + b];
                }
            }
            double den = 0.0;
            for (int64_t a = 0; a < m; ++a) den += qh[i * m + a] * z[a];
            for (int64_t b = 0; b < dv; ++b) {
                double num = 0.0;
                for (int64_t a = 0; a < m; ++a) num += qh[i * m + a] * S[a * dv + b];
                oh[i * dv + b] = num / den;
            }
            if (den_out) den_out[h * N + i] = den;
        }
        if (S_out) memcpy(S_out + h * m * dv, S, (size_t)(m * dv) * sizeof(double));
        if (z_out) memcpy(z_out + h * m, z, (size_t)m * sizeof(double));
        free(S);
        free(z);
    }
}

/* ---- backward on given features ------------------------------------------------
 * Gradients of L = sum(dout * O) for la_oracle_forward_features, by the chain rule
 * (the pages print no backward).  With den_i, O_i of the forward, G_i = dout_i / den_i
 * and g_i = -G_i . O_i (the derivative of O_i = num_i / den_i):
 *   dfq_i = S_i G_i + g_i z_i           (S_i, z_i: the state row i reads),
 *   dfk_j = R_j V_j + r_j,  dV_j = R_j^T fk_j,
 * where R_j = sum fq_i G_i^T and r_j = sum g_i fq_i run over the rows i that read key j
 * (i >= j in the recurrent form, every row otherwise). */
void la_oracle_backward_features(int64_t BH, int64_t N, int64_t m, int64_t dv, int causal,
                                 const double* fq, const double* fk, const double* v,
                                 const double* dout, double* dfq, double* dfk, double* dvo) {
    int nt = la_oracle_get_threads();
    (void)nt;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        const double* qh = fq + h * N * m;
        const double* kh = fk + h * N * m;
        const double* vh = v + h * N * dv;
        const double* doh = dout + h * N * dv;
        double* S = zalloc(m * dv);
        double* z = zalloc(m);
        double* G = zalloc(N * dv);
        double* g = zalloc(N);
        /* forward sweep: the state each row reads, den, O, G, g and dfq */
        int64_t added = 0;
        for (int64_t i = 0; i < N; ++i) {
            const int64_t upto = causal ? i + 1 : N;
            for (; added < upto; ++added)
                for (int64_t a = 0; a < m; ++a) {
                    z[a] += kh[added * m + a];
                    for (int64_t b = 0; b < dv; ++b) S[a * dv + b] += kh[added * m + a] * vh[added * dv + b];
                }
            double den = 0.0;
            for (int64_t a = 0; a < m; ++a) den += qh[i * m + a] * z[a];
            double go = 0.0;
            for (int64_t b = 0; b < dv; ++b) {
                double num = 0.0;
                for (int64_t a = 0; a < m; ++a) num += qh[i * m + a] * S[a * dv + b];
                G[i * dv + b] = doh[i * dv + b] / den;
                go += G[i * dv + b] * (num / den);
            }
            g[i] = -go;
            for (int64_t a = 0; a < m; ++a) {
                double x = g[i] * z[a];
                for (int64_t b = 0; b < dv; ++b) x += S[a * dv + b] * G[i * dv + b];
                dfq[(h * N + i) * m + a] = x;
            }
        }
        /* backward sweep over the keys: R, r over the rows that read key j */
        double* R = zalloc(m * dv);
        double* r = zalloc(m);
        int64_t taken = N; /* rows folded into (R, r): i >= taken */
        for (int64_t j = N - 1; j >= 0; --j) {
            const int64_t from = causal ? j : 0;
            for (; taken > from; ) {
                --taken;
                for (int64_t a = 0; a < m; ++a) {
                    r[a] += g[taken] * qh[taken * m + a];
                    for (int64_t b = 0; b < dv; ++b) R[a * dv + b] += qh[taken * m + a] * G[taken * dv + b];
                }
            }
            for (int64_t a = 0; a < m; ++a) {
                double x = r[a];
                for (int64_t b = 0; b < dv; ++b) x += R[a * dv + b] * vh[j * dv + b];
                dfk[(h * N + j) * m + a] = x;
            }
            for (int64_t b = 0; b < dv; ++b) {
                double x = 0.0;
                for (int64_t a = 0; a < m; ++a) x += R[a * dv + b] * kh[j * m + a];
                dvo[(h * N + j) * dv + b] = x;
            }
        }
        free(S); free(z); free(G); free(g); free(R); free(r);
    }
}

/* Gradient through the FAVOR+ features: out_ri = m^{-1/2} exp(omega_i . x_r - |x_r|^2 / 2)
 * has d out_ri / d x_r = out_ri (omega_i - x_r), so for an upstream gradient dout [rows][m]
 * dx_r = sum_i dout_ri out_ri (omega_i - x_r). */
void la_oracle_favor_features_backward(int64_t rows, int64_t d, int64_t m, const double* x,
                                       const double* omega, const double* dout, double* dx) {
    const double c = 1.0 / sqrt((double)m);
    for (int64_t r = 0; r < rows; ++r) {
        const double* xr = x + r * d;
        double nrm = 0.0;
        for (int64_t a = 0; a < d; ++a) nrm += xr[a] * xr[a];
        for (int64_t a = 0; a < d; ++a) dx[r * d + a] = 0.0;
        for (int64_t i = 0; i < m; ++i) {
            double u = 0.0;
            for (int64_t a = 0; a < d; ++a) u += omega[i * d + a] * xr[a];
            const double w = dout[r * m + i] * c * exp(u - 0.5 * nrm);
            for (int64_t a = 0; a < d; ++a) dx[r * d + a] += w * (omega[i * d + a] - xr[a]);
        }
    }
}
