/*
 * la_oracle.h -- plain, slow, fp64 CPU oracle for kernelized linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this library; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes comes from the page "Efficient Transformers Survey"
 * (economicspath.com), section "Linear Attention", Proposition "Linear
 * Attention via Kernel Decomposition":
 *   - Statement:      Attn_i = phi(Q_i)^T S / phi(Q_i)^T z,
 *                     S = sum_j phi(K_j) V_j^T (m x d), z = sum_j phi(K_j) (m).
 *   - Proof sketch:   Attn_i = sum_j k(Q_i,K_j) V_j / sum_j k(Q_i,K_j) with
 *                     k(q,k) = phi(q)^T phi(k)   (the quadratic form).
 *   - Why it matters: the causal / recurrent form processes tokens one at a
 *                     time, updating S and z incrementally.
 * The feature map is phi(x) = elu(x) + 1 applied elementwise (so m = d); the
 * pages leave phi abstract and this is the reading taken.  The backward pass is
 * not written out on the pages (the arXiv 2510.21956 abstract only says one
 * exists); it is derived from the forward by the chain rule, see
 * la_oracle_backward_causal below.
 *
 * Layout: every tensor is row-major [B][H][N][d] (tokens x features per head),
 * den is [B][H][N], a state S is [B][H][d][d] with S[a][b] (a = feature of
 * phi(K), b = value column) and z is [B][H][d].  All arrays are double; the
 * caller widens bf16 / fp32 inputs exactly.  Heads run in parallel under
 * OpenMP; each head is a plain sequential loop.
 */
#ifndef LA_ORACLE_H
#define LA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* phi(x) = elu(x) + 1 and its derivative. */
double la_oracle_phi(double x);
double la_oracle_dphi(double x);

/* Non-causal forward: global S, z over all N keys, then every row reads them.
 * o: [BH][N][d]; S_out [BH][d][d], z_out [BH][d], den_out [BH][N] may be NULL. */
void la_oracle_forward_noncausal(int64_t BH, int64_t N, int64_t d,
                                 const double* q, const double* k, const double* v,
                                 double* o, double* den_out, double* S_out, double* z_out);

/* Causal forward, recurrent form: for i = 0..N-1, first S += phi(k_i) v_i^T and
 * z += phi(k_i), then o_i = phi(q_i)^T S / phi(q_i)^T z (inclusive: row i sees
 * keys 0..i).  S_out / z_out receive the final state; any output may be NULL
 * except o. */
void la_oracle_forward_causal(int64_t BH, int64_t N, int64_t d,
                              const double* q, const double* k, const double* v,
                              double* o, double* den_out, double* S_out, double* z_out);

/* The same recurrence started from the state (S0 [BH][d][d], z0 [BH][d]) instead
 * of zero (either may be NULL for zero): the continuation of a sequence whose
 * earlier tokens left that state.  S_out / z_out then hold S0 + the new tokens. */
void la_oracle_forward_causal_from(int64_t BH, int64_t N, int64_t d,
                                   const double* S0, const double* z0,
                                   const double* q, const double* k, const double* v,
                                   double* o, double* den_out, double* S_out, double* z_out);

/* Causal backward: gradients of L = sum(dout * o) w.r.t. q, k, v for the causal
 * forward above.  Prefix sweep gives dq, suffix sweep gives dk, dv. */
void la_oracle_backward_causal(int64_t BH, int64_t N, int64_t d,
                               const double* q, const double* k, const double* v,
                               const double* dout, double* dq, double* dk, double* dv);

/* Causal backward of the recurrence started from (S0, z0) (la_oracle_forward_causal_from),
 * for L = sum(dout * o) + sum(dSN * S_N) + sum(dzN * z_N), i.e. with upstream gradients
 * dSN [BH][d][d], dzN [BH][d] of the final state: the suffix sums start from them, and
 * dS0, dz0 receive the gradient of L with respect to the start state (the suffix sums
 * at the first token).  S0, z0, dSN, dzN, dS0, dz0 may be NULL (zero / not wanted). */
void la_oracle_backward_causal_state(int64_t BH, int64_t N, int64_t d, const double* q,
                                     const double* k, const double* v, const double* dout,
                                     const double* S0, const double* z0, const double* dSN,
                                     const double* dzN, double* dq, double* dk, double* dv,
                                     double* dS0, double* dz0);

/* Non-causal backward (same algebra with global S, z and global suffix sums). */
void la_oracle_backward_noncausal(int64_t BH, int64_t N, int64_t d,
                                  const double* q, const double* k, const double* v,
                                  const double* dout, double* dq, double* dk, double* dv);

/* One decode step per head, in place: S += phi(k) v^T, z += phi(k), then
 * o = phi(q)^T S / phi(q)^T z.  S: [BH][d][d], z: [BH][d], q/k/v/o: [BH][d]. */
void la_oracle_decode_step(int64_t BH, int64_t d, double* S, double* z,
                           const double* q, const double* k, const double* v, double* o);

/* Quadratic (brute-force) forms, O(N^2 d): the proof-sketch definition.
 * causal != 0 restricts row i to keys j <= i.  For small inputs only. */
void la_oracle_quadratic_forward(int64_t BH, int64_t N, int64_t d, int causal,
                                 const double* q, const double* k, const double* v,
                                 double* o, double* den_out);
void la_oracle_quadratic_backward(int64_t BH, int64_t N, int64_t d, int causal,
                                  const double* q, const double* k, const double* v,
                                  const double* dout, double* dq, double* dk, double* dv);

/* FAVOR+ positive random features (Performer section of the same page):
 * out[r][i] = m^{-1/2} exp(omega_i . x_r - |x_r|^2 / 2) for rows x [rows][d] and
 * omega [m][d] (one random direction per row). */
void la_oracle_favor_features(int64_t rows, int64_t d, int64_t m, const double* x,
                              const double* omega, double* out);

/* Linear attention on given features fq, fk [BH][N][m] with values v [BH][N][dv]:
 * global (causal == 0) or recurrent inclusive (causal != 0) sums; den_out
 * [BH][N], S_out [BH][m][dv], z_out [BH][m] may be NULL. */
void la_oracle_forward_features(int64_t BH, int64_t N, int64_t m, int64_t dv, int causal,
                                const double* fq, const double* fk, const double* v, double* o,
                                double* den_out, double* S_out, double* z_out);

/* Gradients of L = sum(dout * o) for la_oracle_forward_features: dfq, dfk [BH][N][m],
 * dv [BH][N][dv] (chain rule: G = dout / den, g = -G . o, dfq_i = S_i G_i + g_i z_i,
 * dfk_j = R_j v_j + r_j, dv_j = R_j^T fk_j with R, r summed over the rows reading key j). */
void la_oracle_backward_features(int64_t BH, int64_t N, int64_t m, int64_t dv, int causal,
                                 const double* fq, const double* fk, const double* v,
                                 const double* dout, double* dfq, double* dfk, double* dvo);

/* Gradient through la_oracle_favor_features: dx_r = sum_i dout_ri out_ri (omega_i - x_r). */
void la_oracle_favor_features_backward(int64_t rows, int64_t d, int64_t m, const double* x,
                                       const double* omega, const double* dout, double* dx);

/* Number of OpenMP threads the oracle's parallel loops use (0 = runtime default). */
void la_oracle_set_threads(int n);
int la_oracle_get_threads(void);

#ifdef __cplusplus
}
#endif
#endif
