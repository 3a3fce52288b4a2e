// bwd.hip -- causal backward of kernelized linear attention for gfx950.
//
// The pages state that linear attention has a forward and a backward pass (the
// arXiv 2510.21956 abstract on vix.ing) but print no formulas; the ones used
// here follow from the chain rule on the causal form of the proposition
// "Linear Attention via Kernel Decomposition" (page "Efficient Transformers
// Survey").  With A_ij = phi(Q_i).phi(K_j) (j <= i), num_i = sum_j A_ij V_j,
// den_i = sum_j A_ij, O_i = num_i / den_i:
//   G_i = dO_i / den_i,  g_i = -G_i . O_i,  dA_ij = G_i . V_j + g_i,
//   dphi(Q_i) = sum_{j<=i} dA_ij phi(K_j),  dphi(K_j) = sum_{i>=j} dA_ij phi(Q_i),
//   dV_j = sum_{i>=j} A_ij G_i,  dQ = dphi(Q) phi'(Q),  dK = dphi(K) phi'(K).
//
// Numerics.  phi(K) = 1 + E(K) is close to 1 at the usual input scales, and
// dphi(Q_i) is orthogonal to phi(Q_i) (O_i is homogeneous of degree 0 in
// phi(Q_i)), so dQ is a small residual of large terms.  Rounding phi(K) to
// bf16 would cost about 2^-9 absolute per element and wreck that residual, so
// K enters every MFMA as E(K) and the constant part is carried exactly in fp32
// rank-1 terms (state S = 1 P^T + S_E, z = n 1 + z_E as in the forward):
//   dphi(Q_t) = [rowsum(dA)_t + G_t.P + g_t n] 1 + dA E(K) + S_E G_t + g_t z_E.
// O_t and den_t are recomputed in fp32 from the same split (never read back
// from a bf16 output), and G is rounded to bf16 once and that rounded value is
// used everywhere, so the identity sum_s A_ts dA_ts = 0 holds for the values
// actually used.
//
// Work decomposition (one workgroup of 4 wavefronts per (head, segment)):
//   seg_state + scan (forward kernels) : prefix states (S_E, z_E, P) per segment
//   bwd_prefix : chunks in order; recompute den, O; G, g; dA; dQ.  Saves den, g
//                per row and the segment aggregates R = sum phi(Q) G^T,
//                r = sum g phi(Q), w = sum q_sum G.
//   rscan      : exclusive suffix of (R, r, w) over segments (fixed order).
//   bwd_suffix : chunks in reverse; dK, dV from the in-chunk terms plus the
//                suffix state.
// Chunks are 64 tokens, or 32 where the LDS tiles would not fit (d = 128 in
// bf16, d = 64 in fp32); segments are whole multiples of 64 tokens.
#include "chunk.h"

namespace la {

template <int D, int C>
struct BwdShape {
    static constexpr int TT = C / 16;     // token tiles per chunk
    static constexpr int WPT = 4 / TT;    // wavefronts per token tile
    static constexpr int DT = D / 16;     // feature tiles
    static constexpr int DPW = DT / WPT;  // feature tiles per wavefront in token-row products
    static_assert(TT * WPT == 4 && DPW * WPT == DT, "wavefront layout");
};

// Chunk length used by the backward for (dtype, d); 0 = unsupported.
__host__ __device__ constexpr int bwd_chunk(bool bf, int d) {
    return bf ? (d == 128 ? 32 : 64) : (d == 32 ? 64 : (d == 64 ? 32 : 0));
}

// ---------------------------------------------------------------------------------------
template <typename T, int D, int C>
__global__ __launch_bounds__(kBlock) void bwd_prefix_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    T* __restrict__ dq, float2* __restrict__ rowstat, float* __restrict__ rrec, const float* __restrict__ rec,
    int N, int cps, int nseg) {
    using M = Mma<T>;
    using SH = BwdShape<D, C>;
    using CR = ChunkRegs<T, D, C>;
    constexpr int KS = M::KSTEP;
    __shared__ __attribute__((aligned(16))) T sm_qf[C * D];
    __shared__ __attribute__((aligned(16))) T sm_qft[D * C];
    __shared__ __attribute__((aligned(16))) T sm_ek[C * D];
    __shared__ __attribute__((aligned(16))) T sm_ekt[D * C];
    __shared__ __attribute__((aligned(16))) T sm_v[C * D];
    __shared__ __attribute__((aligned(16))) T sm_vt[D * C];
    __shared__ __attribute__((aligned(16))) T sm_g[C * D];
    __shared__ __attribute__((aligned(16))) T sm_gt[D * C];
    __shared__ __attribute__((aligned(16))) T sm_b[C * C];
    __shared__ __attribute__((aligned(16))) T sm_da[C * C];
    __shared__ __attribute__((aligned(16))) T sm_st[D * D];
    __shared__ __attribute__((aligned(16))) T sm_s[D * D];
    __shared__ float s_qsum[C], s_den[C], s_g[C], s_z[D], s_p[D];
    __shared__ float s_part[2][SH::WPT][C];
    const Tile<T, C, D> tQf{sm_qf}, tEk{sm_ek}, tV{sm_v}, tG{sm_g};
    const Tile<T, D, C> tQft{sm_qft}, tEkt{sm_ekt}, tVt{sm_vt}, tGt{sm_gt};
    const Tile<T, C, C> tB{sm_b}, tdA{sm_da};
    const Tile<T, D, D> tSt{sm_st}, tS{sm_s};

    const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4;
    const int tt = w % SH::TT, dp = w / SH::TT;
    const int t0 = 16 * tt, tl = t0 + (lane & 15);
    const int kend = ((16 * (tt + 1) + KS - 1) / KS) * KS;
    const int64_t hoff = (int64_t)bh * N * D;
    const int tok_begin = seg * cps * kChunk;
    const int tok_end = min(N, tok_begin + cps * kChunk);

    // Prefix state (S_E, z_E, P) at the start of the segment.
    const float* r0 = rec + ((int64_t)bh * nseg + seg) * Rec<D>::kSize;
    StateAcc<D> stS, stR;
    load_state_acc<D>(r0, stS, lane, w);
    publish_state<T, D, true, true>(stS, tSt, tS, lane, w);
    zero_state<D>(stR);
    float zp = 0.f, rp = 0.f;  // tid < D: z_E[a], r[a];  D <= tid < 2D: P[b], w[b]
    if (tid < D) {
        zp = r0[Rec<D>::kZ + tid];
        s_z[tid] = zp;
    } else if (tid < 2 * D) {
        zp = r0[Rec<D>::kP + tid - D];
        s_p[tid - D] = zp;
    }
    float n = (float)tok_begin;

    CR cq, ck, cv, cdo, cdo_cur;
    cq.load(q + hoff, tok_begin, N, tid);
    ck.load(k + hoff, tok_begin, N, tid);
    cv.load(v + hoff, tok_begin, N, tid);
    cdo.load(dout + hoff, tok_begin, N, tid);

    for (int c0 = tok_begin; c0 < tok_end; c0 += C) {
        stage_q<T, D, C, true>(cq, tQf, tQft, s_qsum, tid);
        stage_e<T, D, C, true, true>(ck, tEk, tEkt, tid);
        stage_raw<T, D, C, true, true>(cv, tV, tVt, tid);
        cdo_cur = cdo;
        if (c0 + C < tok_end) {
            cq.load(q + hoff, c0 + C, N, tid);
            ck.load(k + hoff, c0 + C, N, tid);
            cv.load(v + hoff, c0 + C, N, tid);
            cdo.load(dout + hoff, c0 + C, N, tid);
        }
        __syncthreads();

        // (1) B_ts = phi(Q_t).E(K_s), s <= t; den_t.
        const float qs_t = s_qsum[tl];
        float rowB = 0.f;
        {
            f32x4 acc_b[SH::TT];
#pragma unroll
            for (int j = 0; j < SH::TT; ++j) acc_b[j] = zero4();
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += KS) {
                const typename M::frag yf = M::load(tQf, t0, k0, lane);
#pragma unroll
                for (int j = 0; j < SH::TT; ++j)
                    if (j <= tt) acc_b[j] = M::mma(M::load(tEk, 16 * j, k0, lane), yf, acc_b[j]);
            }
#pragma unroll
            for (int j = 0; j < SH::TT; ++j) {
                if (j <= tt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float b = (16 * j + 4 * g + e) <= tl ? acc_b[j][e] : 0.f;
                        acc_b[j][e] = b;
                        rowB += b;
                    }
                    if (dp == 0) store_T(tB, 16 * j, t0, acc_b[j], lane);
                } else if (dp == 0 && 16 * j < kend) {
                    store_T(tB, 16 * j, t0, zero4(), lane);
                }
            }
        }
        const float den = qs_t * (n + (float)(tl + 1)) + sum_over_groups(rowB) +
                          row_dot_quarters<T, D, C>(tQf, s_z, tl, lane);
        if (dp == 0 && g == 0) s_den[tl] = den;
        __syncthreads();

        // (2) G = round(dO / den), staged row-major and transposed.
#pragma unroll
        for (int i = 0; i < CR::NV; ++i) {
            const int t = CR::row(i, tid), gi = CR::gran(i, tid);
            const float dn = s_den[t];
            const bool valid = c0 + t < N;
            uint4 packed;
            T* pk = reinterpret_cast<T*>(&packed);
#pragma unroll
            for (int e = 0; e < CR::EV; ++e) {
                const T gv = from_f32<T>(valid ? cdo_cur.get(i, e) / dn : 0.f);
                pk[e] = gv;
                tGt.at(gi * CR::EV + e, t) = gv;
            }
            *reinterpret_cast<uint4*>(tG.granule(t, gi)) = packed;
        }
        __syncthreads();

        // (3) Recompute O_t for this wave's value tiles; g_t = -G_t.O_t and G_t.P.
        float gpart = 0.f, gppart = 0.f;
        {
            f32x4 accL[SH::DPW], accN[SH::DPW];
#pragma unroll
            for (int m = 0; m < SH::DPW; ++m) {
                accL[m] = zero4();
                accN[m] = zero4();
            }
            for (int k0 = 0; k0 < kend; k0 += KS) {
                const typename M::frag yb = M::load(tB, t0, k0, lane);
                const typename M::frag yl = OnesFrag<T>::lower(tl, k0, lane);
#pragma unroll
                for (int m = 0; m < SH::DPW; ++m) {
                    const typename M::frag xv = M::load(tVt, 16 * (dp * SH::DPW + m), k0, lane);
                    accL[m] = M::mma(xv, yl, accL[m]);
                    accN[m] = M::mma(xv, yb, accN[m]);
                }
            }
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += KS) {
                const typename M::frag yq = M::load(tQf, t0, k0, lane);
#pragma unroll
                for (int m = 0; m < SH::DPW; ++m)
                    accN[m] = M::mma(M::load(tSt, 16 * (dp * SH::DPW + m), k0, lane), yq, accN[m]);
            }
#pragma unroll
            for (int m = 0; m < SH::DPW; ++m) {
                const int b0 = 16 * (dp * SH::DPW + m) + 4 * g;
                const f32x4 gv = lds_load4(tG, tl, b0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float pb = s_p[b0 + e];
                    const float o = (qs_t * (pb + accL[m][e]) + accN[m][e]) / den;
                    gpart -= gv[e] * o;
                    gppart += gv[e] * pb;
                }
            }
        }
        gpart = sum_over_groups(gpart);
        gppart = sum_over_groups(gppart);
        if (SH::WPT > 1) {
            if (g == 0) {
                s_part[0][dp][tl] = gpart;
                s_part[1][dp][tl] = gppart;
            }
            __syncthreads();
            gpart = 0.f;
            gppart = 0.f;
#pragma unroll
            for (int x = 0; x < SH::WPT; ++x) {
                gpart += s_part[0][x][tl];
                gppart += s_part[1][x][tl];
            }
        }
        const float gt = gpart;  // g_t
        const int tok = c0 + tl;
        if (dp == 0 && g == 0) {
            s_g[tl] = gt;
            if (tok < N) rowstat[(int64_t)bh * N + tok] = make_float2(den, gt);
        }

        // (4) dA_ts = G_t.V_s + g_t for s <= t; its row sums.
        float rowdA = 0.f;
        {
            f32x4 acc_d[SH::TT];
#pragma unroll
            for (int j = 0; j < SH::TT; ++j) acc_d[j] = zero4();
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += KS) {
                const typename M::frag yg = M::load(tG, t0, k0, lane);
#pragma unroll
                for (int j = 0; j < SH::TT; ++j)
                    if (j <= tt) acc_d[j] = M::mma(M::load(tV, 16 * j, k0, lane), yg, acc_d[j]);
            }
#pragma unroll
            for (int j = 0; j < SH::TT; ++j) {
                if (j <= tt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float a = (16 * j + 4 * g + e) <= tl ? acc_d[j][e] + gt : 0.f;
                        acc_d[j][e] = a;
                        rowdA += a;
                    }
                    if (dp == 0) store_T(tdA, 16 * j, t0, acc_d[j], lane);
                } else if (dp == 0 && 16 * j < kend) {
                    store_T(tdA, 16 * j, t0, zero4(), lane);
                }
            }
        }
        rowdA = sum_over_groups(rowdA);
        __syncthreads();

        // (5) dphi(Q)^T[a][t] = sum_s E^T[a][s] dA[t][s] + sum_b S_E[a][b] G[t][b] + ..., then dQ.
        {
            f32x4 acc[SH::DPW];
#pragma unroll
            for (int m = 0; m < SH::DPW; ++m) acc[m] = zero4();
            for (int k0 = 0; k0 < kend; k0 += KS) {
                const typename M::frag yd = M::load(tdA, t0, k0, lane);
#pragma unroll
                for (int m = 0; m < SH::DPW; ++m)
                    acc[m] = M::mma(M::load(tEkt, 16 * (dp * SH::DPW + m), k0, lane), yd, acc[m]);
            }
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += KS) {
                const typename M::frag yg = M::load(tG, t0, k0, lane);
#pragma unroll
                for (int m = 0; m < SH::DPW; ++m)
                    acc[m] = M::mma(M::load(tS, 16 * (dp * SH::DPW + m), k0, lane), yg, acc[m]);
            }
            if (tok < N) {
                const float bracket = rowdA + gppart + gt * n;
                const int64_t roff = hoff + (int64_t)tok * D;
#pragma unroll
                for (int m = 0; m < SH::DPW; ++m) {
                    const int a0 = 16 * (dp * SH::DPW + m) + 4 * g;
                    const f32x4 qraw = gload4(q + roff + a0);
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (acc[m][e] + s_z[a0 + e] * gt + bracket) * dphi_f(qraw[e]);
                    gstore4(dq + roff + a0, x);
                }
            }
        }

        // (6) State updates: S_E += E^T V, z_E, P; segment aggregates R += phi(Q)^T G, r, w.
        state_mma<T, D, D, C>(stS, tEkt, tVt, lane, w);
        state_mma<T, D, D, C>(stR, tQft, tGt, lane, w);
        if (tid < D) {
            zp += row_sum(tEkt, tid);
            rp += row_dot(tQft, tid, s_g);
        } else if (tid < 2 * D) {
            zp += row_sum(tVt, tid - D);
            rp += row_dot(tGt, tid - D, s_qsum);
        }
        n += (float)min(C, N - c0);
        __syncthreads();
        publish_state<T, D, true, true>(stS, tSt, tS, lane, w);
        if (tid < D) s_z[tid] = zp;
        else if (tid < 2 * D) s_p[tid - D] = zp;
    }
    float* rr = rrec + ((int64_t)bh * nseg + seg) * Rec<D>::kSize;
    store_state_acc<D>(rr, stR, lane, w);
    if (tid < D) rr[Rec<D>::kZ + tid] = rp;
    else if (tid < 2 * D) rr[Rec<D>::kP + tid - D] = rp;
}

// ---------------------------------------------------------------------------------------
template <typename T, int D, int C>
__global__ __launch_bounds__(kBlock) void bwd_suffix_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    T* __restrict__ dk, T* __restrict__ dv, const float2* __restrict__ rowstat, const float* __restrict__ rrec,
    int N, int cps, int nseg) {
    using M = Mma<T>;
    using SH = BwdShape<D, C>;
    using CR = ChunkRegs<T, D, C>;
    constexpr int KS = M::KSTEP;
    __shared__ __attribute__((aligned(16))) T sm_qf[C * D];
    __shared__ __attribute__((aligned(16))) T sm_qft[D * C];
    __shared__ __attribute__((aligned(16))) T sm_ek[C * D];
    __shared__ __attribute__((aligned(16))) T sm_v[C * D];
    __shared__ __attribute__((aligned(16))) T sm_g[C * D];
    __shared__ __attribute__((aligned(16))) T sm_gt[D * C];
    __shared__ __attribute__((aligned(16))) T sm_dat[C * C];
    __shared__ __attribute__((aligned(16))) T sm_at[C * C];
    __shared__ __attribute__((aligned(16))) T sm_r[D * D];
    __shared__ __attribute__((aligned(16))) T sm_rt[D * D];
    __shared__ float s_qsum[C], s_g[C], s_r[D], s_w[D];
    const Tile<T, C, D> tQf{sm_qf}, tEk{sm_ek}, tV{sm_v}, tG{sm_g};
    const Tile<T, D, C> tQft{sm_qft}, tGt{sm_gt}, tNoneT{nullptr};
    const Tile<T, C, C> tdAt{sm_dat}, tAt{sm_at};
    const Tile<T, D, D> tR{sm_r}, tRt{sm_rt};

    const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4;
    const int tt = w % SH::TT, dp = w / SH::TT;  // tt: this wave's key tile s
    const int s0 = 16 * tt, sl = s0 + (lane & 15);
    const int kstart = (s0 / KS) * KS;
    const int64_t hoff = (int64_t)bh * N * D;
    const int tok_begin = seg * cps * kChunk;
    const int tok_end = min(N, tok_begin + cps * kChunk);
    const int nch = (tok_end - tok_begin + C - 1) / C;

    // Suffix state (R, r, w) of the segments after this one.
    const float* r0 = rrec + ((int64_t)bh * nseg + seg) * Rec<D>::kSize;
    StateAcc<D> stR;
    load_state_acc<D>(r0, stR, lane, w);
    publish_state<T, D, true, true>(stR, tRt, tR, lane, w);
    float rp = 0.f;
    if (tid < D) {
        rp = r0[Rec<D>::kZ + tid];
        s_r[tid] = rp;
    } else if (tid < 2 * D) {
        rp = r0[Rec<D>::kP + tid - D];
        s_w[tid - D] = rp;
    }

    CR cq, ck, cv, cdo;
    const int clast = tok_begin + (nch - 1) * C;
    cq.load(q + hoff, clast, N, tid);
    ck.load(k + hoff, clast, N, tid);
    cv.load(v + hoff, clast, N, tid);
    cdo.load(dout + hoff, clast, N, tid);

    for (int ci = nch - 1; ci >= 0; --ci) {
        const int c0 = tok_begin + ci * C;
        stage_q<T, D, C, true>(cq, tQf, tQft, s_qsum, tid);
        stage_e<T, D, C, true, false>(ck, tEk, tNoneT, tid);
        stage_raw<T, D, C, true, false>(cv, tV, tNoneT, tid);
        // G = round(dO / den) with the den saved by the prefix sweep (bitwise the same G).
#pragma unroll
        for (int i = 0; i < CR::NV; ++i) {
            const int t = CR::row(i, tid), gi = CR::gran(i, tid);
            const int tok = c0 + t;
            const float dn = tok < N ? rowstat[(int64_t)bh * N + tok].x : 1.f;
            uint4 packed;
            T* pk = reinterpret_cast<T*>(&packed);
#pragma unroll
            for (int e = 0; e < CR::EV; ++e) {
                const T gv = from_f32<T>(tok < N ? cdo.get(i, e) / dn : 0.f);
                pk[e] = gv;
                tGt.at(gi * CR::EV + e, t) = gv;
            }
            *reinterpret_cast<uint4*>(tG.granule(t, gi)) = packed;
        }
        if (tid < C) s_g[tid] = c0 + tid < N ? rowstat[(int64_t)bh * N + c0 + tid].y : 0.f;
        if (ci > 0) {
            cq.load(q + hoff, c0 - C, N, tid);
            ck.load(k + hoff, c0 - C, N, tid);
            cv.load(v + hoff, c0 - C, N, tid);
            cdo.load(dout + hoff, c0 - C, N, tid);
        }
        __syncthreads();

        // (1) dA_ts = G_t.V_s + g_t and A_ts = q_sum_t + phi(Q_t).E(K_s) for s <= t,
        //     as dA^T, A^T rows of this wave's key tile.
        {
#pragma unroll
            for (int i = 0; i < SH::TT; ++i) {
                if (i >= tt) {
                    f32x4 acc_d = zero4(), acc_b = zero4();
#pragma unroll
                    for (int k0 = 0; k0 < D; k0 += KS) {
                        const typename M::frag ys = M::load(tV, s0, k0, lane);
                        const typename M::frag ye = M::load(tEk, s0, k0, lane);
                        acc_d = M::mma(M::load(tG, 16 * i, k0, lane), ys, acc_d);
                        acc_b = M::mma(M::load(tQf, 16 * i, k0, lane), ye, acc_b);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = 16 * i + 4 * g + e;
                        const bool live = sl <= t;
                        acc_d[e] = live ? acc_d[e] + s_g[t] : 0.f;
                        acc_b[e] = live ? acc_b[e] + s_qsum[t] : 0.f;
                    }
                    if (dp == 0) {
                        store_T(tdAt, 16 * i, s0, acc_d, lane);
                        store_T(tAt, 16 * i, s0, acc_b, lane);
                    }
                } else if (dp == 0 && 16 * i >= kstart) {
                    store_T(tdAt, 16 * i, s0, zero4(), lane);
                    store_T(tAt, 16 * i, s0, zero4(), lane);
                }
            }
        }
        __syncthreads();

        // (2) dphi(K)^T[a][s] = sum_t phi(Q)^T[a][t] dA^T[s][t] + sum_b R[a][b] V[s][b] + r[a]
        //     dV^T[b][s]      = sum_t G^T[b][t] A^T[s][t] + sum_a R^T[b][a] E[s][a] + w[b]
        {
            f32x4 acck[SH::DPW], accv[SH::DPW];
#pragma unroll
            for (int m = 0; m < SH::DPW; ++m) {
                acck[m] = zero4();
                accv[m] = zero4();
            }
            for (int k0 = kstart; k0 < C; k0 += KS) {
                const typename M::frag yd = M::load(tdAt, s0, k0, lane);
                const typename M::frag ya = M::load(tAt, s0, k0, lane);
#pragma unroll
                for (int m = 0; m < SH::DPW; ++m) {
                    const int f0 = 16 * (dp * SH::DPW + m);
                    acck[m] = M::mma(M::load(tQft, f0, k0, lane), yd, acck[m]);
                    accv[m] = M::mma(M::load(tGt, f0, k0, lane), ya, accv[m]);
                }
            }
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += KS) {
                const typename M::frag yv = M::load(tV, s0, k0, lane);
                const typename M::frag ye = M::load(tEk, s0, k0, lane);
#pragma unroll
                for (int m = 0; m < SH::DPW; ++m) {
                    const int f0 = 16 * (dp * SH::DPW + m);
                    acck[m] = M::mma(M::load(tR, f0, k0, lane), yv, acck[m]);
                    accv[m] = M::mma(M::load(tRt, f0, k0, lane), ye, accv[m]);
                }
            }
            const int tok = c0 + sl;
            if (tok < N) {
                const int64_t roff = hoff + (int64_t)tok * D;
#pragma unroll
                for (int m = 0; m < SH::DPW; ++m) {
                    const int f0 = 16 * (dp * SH::DPW + m) + 4 * g;
                    const f32x4 kraw = gload4(k + roff + f0);
                    f32x4 xk, xv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        xk[e] = (acck[m][e] + s_r[f0 + e]) * dphi_f(kraw[e]);
                        xv[e] = accv[m][e] + s_w[f0 + e];
                    }
                    gstore4(dk + roff + f0, xk);
                    gstore4(dv + roff + f0, xv);
                }
            }
        }

        // (3) Suffix state update: R += phi(Q)^T G, r += phi(Q)^T g, w += G^T q_sum.
        state_mma<T, D, D, C>(stR, tQft, tGt, lane, w);
        if (tid < D) rp += row_dot(tQft, tid, s_g);
        else if (tid < 2 * D) rp += row_dot(tGt, tid - D, s_qsum);
        __syncthreads();
        publish_state<T, D, true, true>(stR, tRt, tR, lane, w);
        if (tid < D) s_r[tid] = rp;
        else if (tid < 2 * D) s_w[tid - D] = rp;
    }
}

// ---------------------------------------------------------------------------------------
hipError_t launch_bwd_prefix(int dt, int d, const void* q, const void* k, const void* v,
                             const void* dout, void* dq, float* rowstat, float* rrec,
                             const float* rec, int64_t BH, int64_t N, SegPlan p, hipStream_t s) {
    const dim3 grid((unsigned)(p.nseg * BH));
#define LA_BWDP(TT, DD)                                                                                \
    hipLaunchKernelGGL((bwd_prefix_kernel<TT, DD, bwd_chunk(sizeof(TT) == 2, DD)>), grid, dim3(kBlock), 0, s, \
                       (const TT*)q, (const TT*)k, (const TT*)v, (const TT*)dout, (TT*)dq, (float2*)rowstat,  \
                       rrec, rec, (int)N, p.cps, p.nseg)
    if (dt == kBF16) {
        switch (d) {
            case 32: LA_BWDP(bf16, 32); break;
            case 64: LA_BWDP(bf16, 64); break;
            case 128: LA_BWDP(bf16, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (d) {
            case 32: LA_BWDP(float, 32); break;
            case 64: LA_BWDP(float, 64); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef LA_BWDP
    return hipGetLastError();
}

hipError_t launch_bwd_suffix(int dt, int d, const void* q, const void* k, const void* v,
                             const void* dout, void* dk, void* dv, const float* rowstat,
                             const float* rrec, int64_t BH, int64_t N, SegPlan p, hipStream_t s) {
    const dim3 grid((unsigned)(p.nseg * BH));
#define LA_BWDS(TT, DD)                                                                                \
    hipLaunchKernelGGL((bwd_suffix_kernel<TT, DD, bwd_chunk(sizeof(TT) == 2, DD)>), grid, dim3(kBlock), 0, s, \
                       (const TT*)q, (const TT*)k, (const TT*)v, (const TT*)dout, (TT*)dk, (TT*)dv,          \
                       (const float2*)rowstat, rrec, (int)N, p.cps, p.nseg)
    if (dt == kBF16) {
        switch (d) {
            case 32: LA_BWDS(bf16, 32); break;
            case 64: LA_BWDS(bf16, 64); break;
            case 128: LA_BWDS(bf16, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (d) {
            case 32: LA_BWDS(float, 32); break;
            case 64: LA_BWDS(float, 64); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef LA_BWDS
    return hipGetLastError();
}

}  // namespace la
