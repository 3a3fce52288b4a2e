/*
 * linattn.h -- C ABI of the MI355X (gfx950) kernelized linear-attention library.
 *
 * The operation is the one stated on the page "Efficient Transformers Survey"
 * (economicspath.com), section "Linear Attention", Proposition "Linear
 * Attention via Kernel Decomposition":
 *
 *     Attn_i = phi(Q_i)^T S / phi(Q_i)^T z,
 *     S = sum_j phi(K_j) V_j^T  (m x d),   z = sum_j phi(K_j)  (m),
 *
 * evaluated in O(N m d) by reassociating (phi(Q) phi(K)^T) V as
 * phi(Q) (phi(K)^T V) ("Intuition" of the same proposition; also the page on
 * memory-efficient Transformers at blopig.com, "Softmax approximators").  The
 * causal form updates S and z token by token ("Why It Matters"), so row i reads
 * keys 0..i inclusive.  The feature map is phi(x) = elu(x) + 1 elementwise, so
 * m = d; the *_features calls take features the caller applied instead (FAVOR+,
 * below, with m = d or, in blocks of d, m > d).  No 1/sqrt(d) scale is applied
 * inside: the formula has none, callers
 * scale Q or K themselves.  No epsilon is added to the denominator: phi > 0.
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers to contiguous row-major arrays,
 *     aligned to 16 bytes.  Q, K, V, O, dO, dQ, dK, dV are [B][H][N][d];
 *     den is [B][H][N] fp32; a state S is [B][H][d][d] fp32 with S[a][b]
 *     (a = feature of phi(K), b = value column); z is [B][H][d] fp32.
 *   - dtype is LA_BF16 (bf16 inputs/outputs, fp32 accumulation and state) or
 *     LA_F32 (fp32 everywhere).  Outputs take the input dtype, rounded to
 *     nearest-even from fp32.
 *   - d must be 32, 64 or 128; B, H, N >= 1 (N = 0 is accepted and does
 *     nothing).
 *   - chunk is 0 (default) or 64, the one chunk length built; 16, 32, 128 and
 *     every other value return LA_ERR_UNSUPPORTED.  The chunk length changes no
 *     result beyond rounding (the reassociation of "Intuition"): it is a tiling
 *     choice, and the kernels map a 64-token chunk onto four 16-row MFMA tiles,
 *     one per wavefront of a role.
 *   - LA_F32 at d = 128: the non-causal forward and decode run native kernels;
 *     the causal forward and both backwards run on two blocks of 64 features of
 *     phi(Q), phi(K) (formed in the workspace), one half of the value columns at a
 *     time (the one-kernel fp32 tiles and states at d = 128 need more LDS and
 *     registers than a CU has): phi = elu + 1 from a zero state in the backward
 *     (no S0 / z0, no state gradients), no grouped heads, and a saved state is
 *     taken but left unused by the causal forward and both backwards (they
 *     recompute on the blocks).  The *_features calls on given features keep
 *     fp32 at d = 32 and 64 for their backward and causal forward.  bf16 covers
 *     d = 128 on every call.
 *   - The caller owns every buffer, including the workspace, whose size comes
 *     from la_workspace_size().  The library never allocates or frees device
 *     memory and keeps no device state between calls.
 *   - Outputs may not overlap inputs (decode's S and z are in/out by design).
 *   - stream is a hipStream_t (NULL = the default stream).  Every call is
 *     stream-ordered and returns without synchronising the host.
 *   - Every call validates its arguments before launching anything and never
 *     throws.  A non-OK status leaves outputs untouched;
 *     la_last_error_message() gives a thread-local description.  Device-side
 *     faults surface at the caller's next synchronisation.
 *   - Results are deterministic: the same inputs give bitwise-identical
 *     outputs (fixed-order reductions, no floating-point atomics).
 *   - Non-finite inputs: causality is strict.  An inf or NaN in q, k, v (or dout)
 *     of token t never reaches an output row that does not read token t: causal
 *     rows before t are bitwise as without it, and in the backward the key-side
 *     gradients of later keys likewise.  Inside a chunk the masked products take
 *     such operands replaced by 0 and the rows that do read token t get their
 *     non-finite result back explicitly.  phi(NaN) = NaN (the feature map
 *     propagates NaN); a result the exact form gives as +-inf may come out NaN.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LA_OK = 0,
    LA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misalignment, overlap */
    LA_ERR_UNSUPPORTED = 2,      /* d, chunk or dtype outside what is built */
    LA_ERR_WORKSPACE = 3,        /* workspace missing or smaller than la_workspace_size() */
    LA_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} la_status;

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

typedef enum {
    LA_OP_FWD_NONCAUSAL = 0,
    LA_OP_FWD_CAUSAL = 1,
    LA_OP_BWD_CAUSAL = 2,
    LA_OP_BWD_NONCAUSAL = 3
} la_op;

/* Bytes of device workspace that `op` needs for this shape (0 is possible).
 * Pure host computation; no device is touched. */
la_status la_workspace_size(la_op op, int64_t B, int64_t H, int64_t N, int64_t d, int chunk,
                            la_dtype dt, size_t* bytes_out);

/* Bytes of the opaque forward state that la_forward_causal (la_forward_noncausal)
 * can save for la_backward_causal (la_backward_noncausal) on the same inputs:
 * the keys' contribution to (S, z) of every sequence segment.  The size is the
 * same for both forms but the contents are not (for long heads the causal form
 * keeps running sums): a state feeds only the backward of the form that saved
 * it.  Pure host computation. */
la_status la_saved_state_size(int64_t B, int64_t H, int64_t N, int64_t d, int chunk, la_dtype dt,
                              size_t* bytes_out);

/* Non-causal forward (Statement of the proposition): one reduction of
 * S = sum_j phi(K_j) V_j^T and z = sum_j phi(K_j) over all N keys per head,
 * then O_i = phi(Q_i)^T S / phi(Q_i)^T z for every row.
 * In: q, k, v [B][H][N][d].  Out: o [B][H][N][d]; saved_state (nullable,
 * saved_state_bytes >= la_saved_state_size()) receives the per-segment key
 * aggregates so that la_backward_noncausal on the same k, v need not rebuild them. */
la_status la_forward_noncausal(const void* q, const void* k, const void* v, void* o, void* saved_state,
                               size_t saved_state_bytes, int64_t B, int64_t H, int64_t N, int64_t d,
                               la_dtype dt, void* workspace, size_t workspace_bytes, void* stream);

/* Causal forward (the recurrent form of "Why It Matters", evaluated chunk by
 * chunk): O_i = phi(Q_i)^T S_i / phi(Q_i)^T z_i with S_i, z_i summed over keys
 * j <= i.  Optional inputs (NULL for a zero state): S0 [B][H][d][d] and z0
 * [B][H][d] fp32, a state the recurrence starts from (the state earlier tokens
 * of the same sequences left, e.g. from a previous call's S_out, z_out: a long
 * prefill in pieces); S0 may be the same buffer as S_out and z0 as z_out
 * (continuing in place), and may overlap no other output.  Optional outputs
 * (NULL to skip): den_out [B][H][N] fp32 holds phi(Q_i)^T z_i; S_out
 * [B][H][d][d] and z_out [B][H][d] receive the state after the last token,
 * ready for la_decode_step / la_decode_steps (with N = 0 they receive the start
 * state); saved_state (device, saved_state_bytes >= la_saved_state_size())
 * receives the per-segment carried state so that la_backward_causal on the same
 * q, k, v need not rebuild it.  The backward starts from a zero state, so a
 * saved_state together with S0 / z0 is LA_ERR_INVALID_ARGUMENT; fp32 at d = 128
 * leaves saved_state unwritten (its backward recomputes) and needs a larger
 * workspace (the feature blocks: la_workspace_size gives it). */
la_status la_forward_causal(const void* q, const void* k, const void* v, void* o, const float* S0,
                            const float* z0, float* den_out, float* S_out, float* z_out,
                            void* saved_state, size_t saved_state_bytes, int64_t B, int64_t H,
                            int64_t N, int64_t d, int chunk, la_dtype dt, void* workspace,
                            size_t workspace_bytes, void* stream);

/* The causal forward with H query heads sharing Hkv key/value heads (grouped or
 * multi-query heads; H a multiple of Hkv): query head h reads the keys and values
 * of key/value head h / (H / Hkv), whose state (S, z) is formed once for the group.
 * q, o [B][H][N][d] and den_out [B][H][N]; k, v [B][Hkv][N][d]; S0, z0, S_out,
 * z_out [B][Hkv][d][d], [B][Hkv][d] (the states la_decode_steps takes with the same
 * H, Hkv).  Workspace: la_workspace_size(LA_OP_FWD_CAUSAL, B, H, N, d, ...).  No
 * saved state (the backward has no grouped heads).  Otherwise as la_forward_causal;
 * Hkv = H is la_forward_causal. */
la_status la_forward_causal_grouped(const void* q, const void* k, const void* v, void* o,
                                    const float* S0, const float* z0, float* den_out, float* S_out,
                                    float* z_out, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                                    int chunk, la_dtype dt, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* Causal backward: dQ, dK, dV of L = sum(dO * O) for the causal forward, by
 * the chain rule (the arXiv 2510.21956 abstract on vix.ing states that a
 * forward and backward pass exist; the formulas are derived, not printed):
 *   G_i = dO_i / den_i, g_i = -G_i . O_i,
 *   dphi(Q_i) = S_i G_i + g_i z_i,
 *   dphi(K_j) = R_j V_j + r_j, dV_j = R_j^T phi(K_j),
 *   R_j = sum_{i>=j} phi(Q_i) G_i^T, r_j = sum_{i>=j} g_i phi(Q_i),
 * then dQ = dphi(Q) * phi'(Q), dK = dphi(K) * phi'(K).  O and den are
 * recomputed in fp32 from q, k, v; the forward's outputs are not inputs here.
 * saved_state (nullable) is the buffer a la_forward_causal call on the same
 * q, k, v and shape filled; when NULL the carried state is rebuilt from k, v.
 * Either way the results are bitwise the same.  fp32 at d = 128 runs per half of
 * the value columns on two 64-feature blocks: the forward on the blocks gives that
 * half's O and den, the blocks' backward takes g_i from that half alone (the
 * halves' g_i add up to the row's, and dphi(Q), dphi(K) are linear in G and g,
 * so the halves' feature gradients add up), and dQ, dK = their sum * phi'; the
 * saved state is not read there.  la_backward_causal_state at fp32 d = 128 with
 * any state pointer set returns LA_ERR_UNSUPPORTED.
 * In: q, k, v, dout [B][H][N][d].  Out: dq, dk, dv [B][H][N][d]. */
la_status la_backward_causal(const void* q, const void* k, const void* v, const void* dout,
                             void* dq, void* dk, void* dv, const void* saved_state,
                             size_t saved_state_bytes, int64_t B, int64_t H, int64_t N, int64_t d,
                             int chunk, la_dtype dt, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Non-causal backward: dQ, dK, dV of L = sum(dO * O) for the non-causal forward,
 * by the chain rule on the Statement's formula (the pages print no backward):
 *   G_i = dO_i / den_i, g_i = -G_i . O_i, den_i = phi(Q_i)^T z,
 *   dphi(Q_i) = S G_i + g_i z,
 *   dphi(K_j) = R V_j + r, dV_j = R^T phi(K_j),
 *   R = sum_i phi(Q_i) G_i^T, r = sum_i g_i phi(Q_i)   (over every query row),
 * then dQ = dphi(Q) * phi'(Q), dK = dphi(K) * phi'(K).  den and O are
 * recomputed in fp32 from q, k, v.  saved_state (nullable) is the buffer a
 * la_forward_noncausal call on the same k, v and shape filled; when NULL the
 * key aggregates are rebuilt from k, v, with bitwise the same results.  fp32 at
 * d = 128 runs per value half on two 64-feature blocks as la_backward_causal does
 * there (the saved state is not read).
 * In: q, k, v, dout [B][H][N][d].  Out: dq, dk, dv [B][H][N][d]. */
la_status la_backward_noncausal(const void* q, const void* k, const void* v, const void* dout,
                                void* dq, void* dk, void* dv, const void* saved_state,
                                size_t saved_state_bytes, int64_t B, int64_t H, int64_t N, int64_t d,
                                la_dtype dt, void* workspace, size_t workspace_bytes, void* stream);

/* Causal backward of la_forward_causal started from (S0, z0), for a sequence fed in
 * pieces (truncated back-propagation): the loss may also depend on the final state
 * (S_N, z_N), whose gradients dS_out [B][H][d][d], dz_out [B][H][d] fp32 (the start
 * state's gradients the next piece's backward returned) join every suffix sum
 * R_j, r_j; dS0, dz0 [B][H][d][d], [B][H][d] fp32 receive the gradients of the
 * start state, R_0 and r_0, to pass to the previous piece as its dS_out, dz_out.
 * Every state pointer is nullable (NULL input: zero; NULL output: not written);
 * with all NULL this is la_backward_causal.  q, k, v, dout, dq, dk, dv, chunk,
 * dtype, workspace (la_workspace_size(LA_OP_BWD_CAUSAL, ...)) and errors as there;
 * the carried state is always rebuilt from k, v (no saved state). */
la_status la_backward_causal_state(const void* q, const void* k, const void* v, const void* dout,
                                   const float* S0, const float* z0, const float* dS_out,
                                   const float* dz_out, void* dq, void* dk, void* dv, float* dS0,
                                   float* dz0, int64_t B, int64_t H, int64_t N, int64_t d, int chunk,
                                   la_dtype dt, void* workspace, size_t workspace_bytes, void* stream);

/* One recurrent decode step per (b, h), in place ("Why It Matters": constant
 * memory per step): S += phi(k) v^T, z += phi(k), then
 * o = phi(q)^T S / phi(q)^T z.  S [B][H][d][d] and z [B][H][d] are fp32 and
 * updated in place; q, k, v, o are [B][H][d] in dtype dt.  Needs no workspace. */
la_status la_decode_step(float* S, float* z, const void* q, const void* k, const void* v, void* o,
                         int64_t B, int64_t H, int64_t d, la_dtype dt, void* stream);

/* T recurrent decode steps in one call, in place ("Why It Matters": tokens one
 * by one), with H query heads sharing Hkv key/value heads (H a multiple of Hkv;
 * Hkv = H: one state per head; Hkv = 1: one state for all query heads).  Query
 * head h reads the state of key/value head h / (H / Hkv).  Per key/value head
 * (b, j) and token t = 0 .. T-1: S += phi(k_t) v_t^T, z += phi(k_t), then for
 * each query head h of the group o_{h,t} = phi(q_{h,t})^T S / phi(q_{h,t})^T z.
 * With Hkv = H this is T calls of la_decode_step up to fp32 rounding.  The state
 * is read and written once per call (not once per token) and once per group
 * (not once per query head).  S [B][Hkv][d][d] and z [B][Hkv][d] are fp32 and
 * updated in place; q, o are [B][H][T][d] and k, v [B][Hkv][T][d] in dtype dt
 * (token t at row t).  T = 0 does nothing.  Needs no workspace.  With several
 * query heads per state (H > Hkv) at d = 64 or 128 the rows (t, h) are formed in
 * blocks of tokens by the chunked form of the same recurrence (MFMA products,
 * the state updated in fp32 after each block's whole tokens; for bf16 inputs the
 * products with phi(q) take hi + lo bf16 splits of both operands, about 2^-16
 * relative per product): the same values up to that rounding, and an inf or NaN
 * of token t reaches no row of an earlier token. */
la_status la_decode_steps(float* S, float* z, const void* q, const void* k, const void* v, void* o,
                          int64_t B, int64_t H, int64_t Hkv, int64_t T, int64_t d, la_dtype dt,
                          void* stream);

/* ---- Given feature maps: FAVOR+ (Performer section of the same page) ------------------
 * FAVOR+ positive random features: out[r][i] = exp(omega_i . x_r - |x_r|^2 / 2) for
 * every row x_r of x [rows][d] and every row omega_i of omega [d][d] fp32 (m = d
 * random directions, e.g. drawn from N(0, I_d)).  The page's constant 1/sqrt(m)
 * is left out: it scales all weights of a row alike and cancels in every output
 * O (states and denominators computed from these features carry the factor m).
 * Any 1/sqrt(d) scaling of queries and keys is the caller's pre-normalization
 * (x = q d^(-1/4) puts it into q.k); features are computed in fp32, so rows with
 * |x|^2 far beyond 100 underflow (every feature of such a row may round to 0).
 * x and out in dtype dt (out rounded from fp32); omega is not overwritten. */
la_status la_favor_features(const void* x, const float* omega, void* out, int64_t rows, int64_t d,
                            la_dtype dt, void* stream);

/* The forward calls and multi-token decode on features the caller has already
 * applied (phi(Q), phi(K): FAVOR+ features from la_favor_features, or any other
 * positive map with m = d features): O_i = fq_i^T S / fq_i^T z with S and z summed
 * from fk and v exactly as in la_forward_causal / la_forward_noncausal /
 * la_decode_steps, which apply phi = elu + 1 themselves.  Features must be
 * positive (denominators must not vanish; an exact 0 is read as the padding
 * past a sequence's end and adds nothing to the state).  Same layouts, workspaces
 * (la_workspace_size of the matching op), start states and errors as those
 * calls; no saved state (la_backward_causal_features / la_backward_noncausal_features
 * rebuild the key aggregates themselves). */
la_status la_forward_causal_features(const void* fq, const void* fk, const void* v, void* o,
                                     const float* S0, const float* z0, float* den_out, float* S_out,
                                     float* z_out, int64_t B, int64_t H, int64_t N, int64_t d,
                                     la_dtype dt, void* workspace, size_t workspace_bytes, void* stream);
la_status la_forward_noncausal_features(const void* fq, const void* fk, const void* v, void* o,
                                        int64_t B, int64_t H, int64_t N, int64_t d, la_dtype dt,
                                        void* workspace, size_t workspace_bytes, void* stream);
la_status la_decode_steps_features(float* S, float* z, const void* fq, const void* fk, const void* v,
                                   void* o, int64_t B, int64_t H, int64_t Hkv, int64_t T, int64_t d,
                                   la_dtype dt, void* stream);

/* Backward on given features (m = d): the gradients dfq, dfk, dv of L = sum(dO * O) for
 * la_forward_causal_features / la_forward_noncausal_features (the same chain rule as
 * la_backward_causal with phi the identity: G = dO / den, g = -G . O, dfq_i = S_i G_i +
 * g_i z_i, dfk_j = R_j v_j + r_j, dv_j = R_j^T fk_j).  Layouts, workspaces
 * (la_workspace_size of LA_OP_BWD_CAUSAL / LA_OP_BWD_NONCAUSAL) and errors as those
 * calls; no saved state or start state.  Features must be positive (as in the forward). */
la_status la_backward_causal_features(const void* fq, const void* fk, const void* v, const void* dout,
                                      void* dfq, void* dfk, void* dv, int64_t B, int64_t H, int64_t N,
                                      int64_t d, la_dtype dt, void* workspace, size_t workspace_bytes,
                                      void* stream);
la_status la_backward_noncausal_features(const void* fq, const void* fk, const void* v, const void* dout,
                                         void* dfq, void* dfk, void* dv, int64_t B, int64_t H, int64_t N,
                                         int64_t d, la_dtype dt, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* The gradient through la_favor_features (m = d): F_i = exp(omega_i . x - |x|^2 / 2) has
 * dF_i / dx = F_i (omega_i - x), so for features F [rows][d] of x [rows][d] (the forward's
 * output, passed back in) and their upstream gradient dF [rows][d]:
 *   dx = omega^T (dF * F) - x sum_i (dF * F)_i   per row.
 * x, F, dF, dx in dtype dt; omega [d][d] fp32 as in the forward. */
la_status la_favor_features_backward(const void* x, const float* omega, const void* F, const void* dF,
                                     void* dx, int64_t rows, int64_t d, la_dtype dt, void* stream);

/* ---- More random features than d: m = KF d, KF = m / d feature blocks --------------------
 * The Performer section of the same page draws m random directions, and m may exceed d
 * (the estimate's variance falls as 1/m).  Features come in blocks of d: block j holds
 * features j d .. j d + d - 1, and each head's features are stored block by block,
 * [B][H][KF][N][d] (the "block layout"; KF = 1 is the plain [B][H][N][d]).  States keep
 * the natural layout S [B][H][m][d] (row a = feature a) and z [B][H][m], which read block
 * by block is one [d][d] state per block.  m must be a positive multiple of d with
 * m / d <= 64 (LA_ERR_INVALID_ARGUMENT / LA_ERR_UNSUPPORTED otherwise); m = d is the
 * plain call.
 *
 * la_favor_features_blocks: the features of x [heads][N][d] (heads = B H) for omega
 * [m][d] fp32 into out [heads][KF][N][d]; otherwise as la_favor_features.
 *
 * la_forward_causal_features_blocks / la_forward_noncausal_features_blocks: attention on
 * such features: fq, fk in block layout; v, o [B][H][N][d]; den_out [B][H][N] fp32
 * (nullable) receives phi(Q_i)^T z over all m features.  Each block runs as a head of its
 * own over its head's values (num_j, den_j), and O = sum_j num_j / sum_j den_j is formed
 * as sum_j den_j O_j / sum_j den_j (O_j kept in dt in the workspace).  Start and final
 * states (causal only, nullable, natural layout above) as la_forward_causal_features.
 * Workspace: la_features_workspace_size(causal != 0, B, H, N, d, m, dt, &bytes), which
 * for KF > 1 holds the blocks' outputs besides the plain call's workspace (causal = 2:
 * the workspace of la_decode_steps_features_blocks with N = T; causal = 3: that of
 * la_backward_causal_features_blocks; causal = 4: that of la_backward_noncausal_features_blocks). */
la_status la_features_workspace_size(int causal, int64_t B, int64_t H, int64_t N, int64_t d, int64_t m,
                                     la_dtype dt, size_t* bytes_out);
la_status la_favor_features_blocks(const void* x, const float* omega, void* out, int64_t heads, int64_t N,
                                   int64_t d, int64_t m, la_dtype dt, void* stream);
/* The gradient through la_favor_features_blocks: x [heads][N][d], omega [m][d] fp32, F and dF
 * [heads][KF][N][d] in block layout; dx [heads][N][d] = sum_j (omega_j^T (dF_j * F_j) - x sum(dF_j * F_j))
 * over the blocks j (the formula of la_favor_features_backward, which is linear in dF_j * F_j). */
la_status la_favor_features_blocks_backward(const void* x, const float* omega, const void* F, const void* dF,
                                            void* dx, int64_t heads, int64_t N, int64_t d, int64_t m, la_dtype dt,
                                            void* stream);
la_status la_forward_causal_features_blocks(const void* fq, const void* fk, const void* v, void* o,
                                            const float* S0, const float* z0, float* den_out, float* S_out,
                                            float* z_out, int64_t B, int64_t H, int64_t N, int64_t d, int64_t m,
                                            la_dtype dt, void* workspace, size_t workspace_bytes, void* stream);
la_status la_forward_noncausal_features_blocks(const void* fq, const void* fk, const void* v, void* o,
                                               float* den_out, int64_t B, int64_t H, int64_t N, int64_t d,
                                               int64_t m, la_dtype dt, void* workspace, size_t workspace_bytes,
                                               void* stream);
/* Causal backward on m = KF d features (block layout, as la_forward_causal_features_blocks
 * from a zero state): dfq, dfk [B][H][KF][N][d] and dv [B][H][N][d] of L = sum(dO * O).  The
 * blocks share one normalization, so every block uses the head's G = dO / den and
 * g = -G . O: den [B][H][N] fp32 is the forward's den_out (the head's, over all m
 * features).  A statistics sweep per block gives each row's G . num_j, their sum gives g,
 * then the block's sweeps give dfq_j, dfk_j and its share of dv (summed over the blocks).
 * o (nullable) [B][H][N][d]: the forward's output; when given, g = -G . O of every row comes
 * from it in one elementwise pass and the statistics sweep is skipped (the same gradients
 * to the rounding of O).
 * Workspace: la_features_workspace_size(3, B, H, N, d, m, dt, &bytes); m = d is
 * la_backward_causal_features (den and o unused). */
la_status la_backward_causal_features_blocks(const void* fq, const void* fk, const void* v, const void* dout,
                                             const float* den, const void* o, void* dfq, void* dfk, void* dv, int64_t B,
                                             int64_t H, int64_t N, int64_t d, int64_t m, la_dtype dt,
                                             void* workspace, size_t workspace_bytes, void* stream);
/* Non-causal backward on m = KF d features (block layout, as la_forward_noncausal_features_blocks):
 * dfq, dfk [B][H][KF][N][d] and dv [B][H][N][d] of L = sum(dO * O), with den [B][H][N] fp32 the
 * forward's den_out.  The same derivative of the non-causal form as la_backward_noncausal_features,
 * with the head's G = dO / den and g = -G . O in every block: a statistics pass gives each row's
 * G . num_j per block, their sum gives g, then each block's passes give dfq_j, dfk_j and its share
 * of dv (summed over the blocks); o (nullable) as in la_backward_causal_features_blocks.
 * Workspace: la_features_workspace_size(4, B, H, N, d, m, dt,
 * &bytes); m = d is la_backward_noncausal_features (den and o unused). */
la_status la_backward_noncausal_features_blocks(const void* fq, const void* fk, const void* v, const void* dout,
                                                const float* den, const void* o, void* dfq, void* dfk, void* dv, int64_t B,
                                                int64_t H, int64_t N, int64_t d, int64_t m, la_dtype dt,
                                                void* workspace, size_t workspace_bytes, void* stream);
/* Multi-token decode (la_decode_steps_features) on m = KF d features: fq [B][H][KF][T][d]
 * and fk [B][Hkv][KF][T][d] in block layout, v, o as la_decode_steps; the state of key/value
 * head j is S [B][Hkv][m][d], z [B][Hkv][m] (what la_forward_causal_features_blocks leaves
 * with H = Hkv).  Workspace (KF > 1): la_features_workspace_size(2, B, H, T, d, m, dt, &bytes);
 * m = d needs none and is la_decode_steps_features. */
la_status la_decode_steps_features_blocks(float* S, float* z, const void* fq, const void* fk, const void* v,
                                          void* o, int64_t B, int64_t H, int64_t Hkv, int64_t T, int64_t d,
                                          int64_t m, la_dtype dt, void* workspace, size_t workspace_bytes,
                                          void* stream);

/* For callers that cannot allocate device memory (code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid hipMalloc): la_forward_causal
 * without the workspace argument.  Its workspace is a 64 MiB array that the library
 * holds as a static device object, one per GPU it runs on, for the life of the
 * process; the call allocates nothing (with per-kernel timing off, the default) and
 * takes the array's device address, looked up once per device on its first call
 * there.  Shapes whose workspace (la_workspace_size(LA_OP_FWD_CAUSAL, ...)) exceeds
 * 64 MiB are rejected with LA_ERR_WORKSPACE before anything is launched (B H = 64
 * heads of N = 4096 at d = 64 take 9.7 MiB).  The array is shared by every call on
 * that GPU and keeps the last call's contents, all of which a call writes before it
 * reads: calls that overlap on one GPU (other streams, other host threads) race and
 * must be serialised by the caller.  No saved state.  Everything else (operation,
 * layouts, start and final states, den_out, chunk, errors) as la_forward_causal. */
la_status la_forward_causal_noalloc(const void* q, const void* k, const void* v, void* o, const float* S0,
                                    const float* z0, float* den_out, float* S_out, float* z_out, int64_t B, int64_t H,
                                    int64_t N, int64_t d, int chunk, la_dtype dt, void* stream);

/* Static description of a status code. */
const char* la_status_string(la_status s);

/* Thread-local description of the last non-OK status returned on this thread. */
const char* la_last_error_message(void);

/* Library version string. */
const char* la_version(void);

/* Test hook for the launches that wait for other workgroups: the fused causal
 * backward (where a head has at most 12 segments and d <= 64) and the fused causal
 * forward (where a head has at most 12 segments and every query head has its own
 * key/value head).  There each workgroup publishes its segment's aggregates and
 * waits for those of the other segments of its head that it needs (the later ones
 * in the backward, the earlier ones in the forward); a wait that sees no data after
 * `polls` polls (default 65536, tens of milliseconds) gives up, and that segment's
 * rows (dk and dv in the backward, o in the forward) become NaN instead of using
 * data that never arrived.  polls = 0 makes every such wait give up at once (the
 * segments that wait for nothing, the last of each head in the backward and the
 * first in the forward, are unaffected).  Process-wide; LA_ERR_INVALID_ARGUMENT for
 * polls < 0.  la_debug_wait_limit() returns the bound. */
la_status la_debug_set_wait_limit(int polls);
int la_debug_wait_limit(void);

/* For callers that must tell a poisoned result from real NaN data: the number of
 * workgroups whose wait gave up (see above) in the last launch of `op` that ran on
 * `workspace` for this shape.  op = LA_OP_BWD_CAUSAL: the fused causal backward
 * (la_backward_causal, la_backward_causal_state, la_backward_causal_features), each
 * give-up leaving NaN in its segment's dk and dv rows; op = LA_OP_FWD_CAUSAL: the
 * fused causal forward (la_forward_causal, la_forward_causal_features,
 * la_forward_causal_noalloc), each give-up leaving NaN in its segment's o rows (a
 * causal forward whose key/value heads are shared, la_forward_causal_grouped with
 * fewer key/value heads or la_forward_causal_features_blocks, runs as two launches,
 * waits for nothing and sets the counts to zero).  Every workgroup of such
 * a launch writes its own count into the workspace, so no clearing is needed between
 * calls.  Synchronises `stream` (a hipStream_t, NULL = the default stream) and copies
 * the counts to the host.  *failures_out = 0 for shapes whose launches never wait
 * (more than 12 segments per head; for the backward also d = 128).  Errors:
 * LA_ERR_INVALID_ARGUMENT (failures_out NULL, or another op), shape errors as
 * la_workspace_size, LA_ERR_WORKSPACE (workspace NULL or smaller than
 * la_workspace_size(op, ...)), LA_ERR_HIP (the synchronisation or the copy failed). */
la_status la_wait_failures(la_op op, const void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t N,
                           int64_t d, la_dtype dt, void* stream, int64_t* failures_out);

/* Per-kernel timing for benchmarks and profiling.  While enabled (on != 0) on
 * the calling thread, every kernel that a call on this thread launches is
 * bracketed by two HIP events recorded on the call's stream; enabling or
 * disabling clears the list.  Events come from a per-thread pool that the
 * library creates once with hipEventCreate and reuses (no device memory).
 * la_profile_count() is the number of launches recorded since; entry i
 * synchronises on its stop event and returns the kernel's name ("seg_state",
 * "total", "scan", "causal_fwd", "causal_fwd_fused", "noncausal_fwd", "bwd_prefix",
 * "rseg", "rscan", "bwd_suffix", "bwd_fused", "ncbwd_q", "ncbwd_kv", "decode",
 * "decode_steps", "state_split", "favor_features", "favor_features_bwd",
 * "combine_blocks", "combine_stats", "stats_from_output", "fill_zero") and its
 * duration in milliseconds. */
la_status la_profile_enable(int on);
int la_profile_count(void);
la_status la_profile_entry(int i, const char** name, float* ms);

#ifdef __cplusplus
}
#endif
#endif /* LINATTN_H */
