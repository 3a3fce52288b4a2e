// bwd.hip -- causal backward of kernelized linear attention for gfx950.
//
// The pages state that linear attention has a forward and a backward pass (the
// arXiv 2510.21956 abstract on vix.ing) but print no formulas; the ones used
// here follow from the chain rule on the causal form of the proposition
// "Linear Attention via Kernel Decomposition" (page "Efficient Transformers
// Survey").  With A_ij = phi(Q_i).phi(K_j) (j <= i), num_i = sum_j A_ij V_j,
// den_i = sum_j A_ij, O_i = num_i / den_i:
//   G_i = dO_i / den_i,  g_i = -G_i . O_i = -(G_i . num_i) / den_i,
//   dA_ij = G_i . V_j + g_i,
//   dphi(Q_i) = sum_{j<=i} dA_ij phi(K_j),  dphi(K_j) = sum_{i>=j} dA_ij phi(Q_i),
//   dV_j = sum_{i>=j} A_ij G_i,  dQ = dphi(Q) phi'(Q),  dK = dphi(K) phi'(K).
//
// Numerics.  phi(K) = 1 + E(K) is close to 1 at the usual input scales and
// dphi(Q_i) is orthogonal to phi(Q_i) (O_i is homogeneous of degree 0 in
// phi(Q_i)), so dQ is a small residual of large terms.  K therefore enters
// every MFMA as E(K) and the constant part is carried exactly in fp32 rank-1
// terms, with the prefix state S = 1 P^T + S_E, z = n 1 + z_E of the forward:
//   dphi(Q_t) = [rowsum(dA)_t + G_t.P + g_t n] 1 + dA E(K) + S_E G_t + g_t z_E.
// G is rounded to bf16 once, and g is formed from the very products that build
// dA (no separate output O):
//   G_t . num_t = sum_{s<=t} A_ts (G_t.V_s) + q_sum_t (G_t.P) + phi(Q_t).(S_E G_t),
// so that sum_j A_tj dA_tj = 0 holds for the values actually used.
//
// Work decomposition (one workgroup of 4 wavefronts per (head, segment)):
//   seg_state + scan (forward kernels): prefix states (S_E, z_E, P) per segment;
//   bwd_prefix: chunks in order: den, G, g, dA, dQ; saves den and g per row and
//               the segment's R = sum phi(Q) G^T, r = sum g phi(Q), w = sum q_sum G;
//   rscan     : exclusive suffix of (R, r, w) over segments (fixed order);
//   bwd_suffix: chunks in reverse: dK, dV from the in-chunk terms plus the suffix state.
#include "chunk.h"

namespace la {

// ---------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kBlock, LA_HEAVY_WAVES_PER_SIMD) void bwd_prefix_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    T* __restrict__ dq, float2* __restrict__ rowstat, float* __restrict__ rrec, const float* __restrict__ rec, int N,
    int cps, int nseg) {
    using M = Mma<T>;
    constexpr int KS = M::KSTEP;
    constexpr int DT = D / 16;
    __shared__ __attribute__((aligned(16))) T sm_q[kC * D];
    __shared__ __attribute__((aligned(16))) T sm_e[kC * D];
    __shared__ __attribute__((aligned(16))) T sm_v[kC * D];
    __shared__ __attribute__((aligned(16))) T sm_g[kC * D];
    __shared__ __attribute__((aligned(16))) T sm_da[kC * kC];
    __shared__ __attribute__((aligned(16))) T sm_st[D * D];
    __shared__ __attribute__((aligned(16))) float sm_b[kC * kC];
    __shared__ __attribute__((aligned(16))) float s_den[kC], s_g[kC], s_z[D], s_p[D];
    const Tile<T, kC, D> tQ{sm_q}, tE{sm_e}, tV{sm_v}, tG{sm_g};
    const Tile<T, kC, kC> tdA{sm_da};
    const Tile<float, kC, kC> tB{sm_b};
    const Tile<T, D, D> tSt{sm_st};

    const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 4;
    const int t0 = 16 * w, tl = t0 + (lane & 15);
    const int64_t hoff = (int64_t)bh * N * D;
    const int tok_begin = seg * cps * kC;
    const int tok_end = min(N, tok_begin + cps * kC);

    // Prefix state (S_E, z_E, P) at the start of the segment; segment aggregates from zero.
    const float* r0 = rec + ((int64_t)bh * nseg + seg) * Rec<D>::kSize;
    StateAcc<D> stS, stR;
    VecAcc<D> vz, vp, vr;
    load_state<D>(r0, stS, lane, w);
    load_vec<D>(r0 + Rec<D>::kZ, vz, lane, w);
    load_vec<D>(r0 + Rec<D>::kP, vp, lane, w);
    zero_state<D>(stR);
    zero_vec<D>(vr);
    float n = (float)tok_begin;

    ChunkRegs<T, D> cq, ck, cv;
    ChunkRegs<T, D, true> cdo;
    cq.load(q + hoff, tok_begin, N, tid);
    ck.load(k + hoff, tok_begin, N, tid);
    cv.load(v + hoff, tok_begin, N, tid);

    for (int c0 = tok_begin; c0 < tok_end; c0 += kC) {
        publish_state<T, D>(stS, tSt, lane, w);
        store_vec<D>(s_z, vz, lane, w);
        store_vec<D>(s_p, vp, lane, w);
        stage_phi<T, D>(cq, tQ, tid);
        stage_elu<T, D>(ck, tE, tid);
        stage_raw<T, D>(cv, tV, tid);
        cdo.load(dout + hoff, c0, N, tid);
        if (c0 + kC < tok_end) {
            cq.load(q + hoff, c0 + kC, N, tid);
            ck.load(k + hoff, c0 + kC, N, tid);
            cv.load(v + hoff, c0 + kC, N, tid);
        }
        const int tok = c0 + tl;
        const bool valid = tok < N;
        __syncthreads();

        // (1) B_ts = phi(Q_t).E(K_s) (accumulator [s][t], all key tiles) and q_sum_t; den_t.
        float qs_t, rowB = 0.f;
        {
            const typename M::frag one = M::ones();
            f32x4 accB[4], accq = zero4();
#pragma unroll
            for (int j = 0; j < 4; ++j) accB[j] = zero4();
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += KS) {
                const typename M::frag yq = M::ld(tQ, t0, k0, lane);
                accq = M::mma(one, yq, accq);
#pragma unroll
                for (int j = 0; j < 4; ++j) accB[j] = M::mma(M::ld(tE, 16 * j, k0, lane), yq, accB[j]);
            }
            qs_t = accq[0];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float b = (16 * j + 4 * g + e) <= tl ? accB[j][e] : 0.f;
                    accB[j][e] = b;
                    rowB += b;
                }
                store_T(tB, 16 * j, t0, accB[j], lane);  // fp32 B[t][s], this wave's rows
            }
        }
        const float den = qs_t * (n + (float)(tl + 1)) + sum_over_groups(rowB) +
                          row_dot_quarters<T, D>(tQ, s_z, tl, lane);
        const float inv_den = rcp_f(den);
        if (g == 0) s_den[tl] = den;
        wave_lds_sync();

        // (2) G = round(dO / den) for this wave's rows.
        stage_grad<T, D, true>(cdo, tG, s_den, c0, N, tid);
        wave_lds_sync();

        // (3) G_t.V_s (accumulator [s][t]) and (S_E G_t)_a (accumulator [a][t]).
        f32x4 accGV[4], accQ[DT];
#pragma unroll
        for (int j = 0; j < 4; ++j) accGV[j] = zero4();
#pragma unroll
        for (int m = 0; m < DT; ++m) accQ[m] = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += KS) {
            const typename M::frag yg = M::ld(tG, t0, k0, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) accGV[j] = M::mma(M::ld(tV, 16 * j, k0, lane), yg, accGV[j]);
#pragma unroll
            for (int m = 0; m < DT; ++m) accQ[m] = M::mma(M::ld_tr(tSt, k0, 16 * m, lane), yg, accQ[m]);
        }

        // (4) g_t = -(G_t . num_t) / den_t.
        float s1 = 0.f, gp = 0.f, s3 = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 b4 = lds4(&tB.at(tl, 16 * j + 4 * g));
#pragma unroll
            for (int e = 0; e < 4; ++e) s1 += (16 * j + 4 * g + e) <= tl ? (qs_t + b4[e]) * accGV[j][e] : 0.f;
        }
#pragma unroll
        for (int m = 0; m < DT; ++m) {
            const int f0 = 16 * m + 4 * g;
            const f32x4 gv = lds4(&tG.at(tl, f0));
            const f32x4 qv = lds4(&tQ.at(tl, f0));
            const f32x4 pv = lds4(&s_p[f0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gp += gv[e] * pv[e];
                s3 += qv[e] * accQ[m][e];
            }
        }
        gp = sum_over_groups(gp);
        const float gt = -(sum_over_groups(s1) + qs_t * gp + sum_over_groups(s3)) * inv_den;
        if (g == 0) {
            s_g[tl] = gt;
            if (valid) rowstat[(int64_t)bh * N + tok] = make_float2(den, gt);
        }

        // (5) dA_ts = G_t.V_s + g_t for s <= t, stored [t][s]; its row sums.
        float rowdA = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = (16 * j + 4 * g + e) <= tl ? accGV[j][e] + gt : 0.f;
                accGV[j][e] = a;
                rowdA += a;
            }
            store_T(tdA, 16 * j, t0, accGV[j], lane);
        }
        rowdA = sum_over_groups(rowdA);
        // phi'(Q) needs the raw inputs of the lane's output elements (cache-resident).
        Raw4<T> qraw[DT];
#pragma unroll
        for (int m = 0; m < DT; ++m) {
            if (valid) qraw[m].load(q + hoff + (int64_t)tok * D + 16 * m + 4 * g);
            else qraw[m].clear();
        }
        __syncthreads();  // dA rows, s_g and all rows of G are visible

        // (6) dphi(Q)^T[a][t] = (S_E G_t)_a + sum_s E[s][a] dA[t][s] + z_E[a] g_t + bracket_t.
#pragma unroll
        for (int k0 = 0; k0 < kC; k0 += KS) {
            const typename M::frag yd = M::ld(tdA, t0, k0, lane);
#pragma unroll
            for (int m = 0; m < DT; ++m) accQ[m] = M::mma(M::ld_tr(tE, k0, 16 * m, lane), yd, accQ[m]);
        }
        if (valid) {
            const float bracket = rowdA + gp + gt * n;
            T* drow = dq + hoff + (int64_t)tok * D;
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                const int f0 = 16 * m + 4 * g;
                const f32x4 zv = lds4(&s_z[f0]);
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = (accQ[m][e] + zv[e] * gt + bracket) * dphi_f(qraw[m].get(e));
                gstore4(drow + f0, x);
            }
        }

        // (7) State S_E += E^T V, z_E, P; segment aggregates R += phi(Q)^T G, r += phi(Q)^T g.
        state_update<T, D, true, true>(stS, vz, vp, tE, tV, nullptr, nullptr, lane, w);
        state_update<T, D, true, false>(stR, vr, vr, tQ, tG, s_g, nullptr, lane, w);
        n += (float)min(kC, N - c0);
        __syncthreads();
    }
    float* rr = rrec + ((int64_t)bh * nseg + seg) * Rec<D>::kSize;
    store_state<D>(rr, stR, lane, w);
    store_vec<D>(rr + Rec<D>::kZ, vr, lane, w);
    // The record's last vector (w = sum over a of R) is formed from R where it is used.
    if (tid < D) rr[Rec<D>::kP + tid] = 0.f;
}

// ---------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kBlock, LA_HEAVY_WAVES_PER_SIMD) void bwd_suffix_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    T* __restrict__ dk, T* __restrict__ dv, const float2* __restrict__ rowstat, const float* __restrict__ rrec, int N,
    int cps, int nseg) {
    using M = Mma<T>;
    using CR = ChunkRegs<T, D>;
    using ST = StateTiles<D>;
    constexpr int KS = M::KSTEP;
    constexpr int DT = D / 16;
    __shared__ __attribute__((aligned(16))) T sm_q[kC * D];
    __shared__ __attribute__((aligned(16))) T sm_e[kC * D];
    __shared__ __attribute__((aligned(16))) T sm_v[kC * D];
    __shared__ __attribute__((aligned(16))) T sm_g[kC * D];
    __shared__ __attribute__((aligned(16))) T sm_dat[kC * kC];
    __shared__ __attribute__((aligned(16))) T sm_at[kC * kC];
    __shared__ __attribute__((aligned(16))) T sm_rt[D * D];
    __shared__ __attribute__((aligned(16))) float s_g[kC], s_r[D], s_w[D], s_wpart[DT][D];
    const Tile<T, kC, D> tQ{sm_q}, tE{sm_e}, tV{sm_v}, tG{sm_g};
    const Tile<T, kC, kC> tdAt{sm_dat}, tAt{sm_at};
    const Tile<T, D, D> tRt{sm_rt};

    const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 4;
    const int s0 = 16 * w, sl = s0 + (lane & 15);  // this wave's key tile, this lane's key
    const int64_t hoff = (int64_t)bh * N * D;
    const float2* rs = rowstat + (int64_t)bh * N;
    const int tok_begin = seg * cps * kC;
    const int tok_end = min(N, tok_begin + cps * kC);
    const int nch = (tok_end - tok_begin + kC - 1) / kC;

    // Suffix state (R, r) of the segments after this one; w = sum_a R[a][b] is formed from R.
    const float* r0 = rrec + ((int64_t)bh * nseg + seg) * Rec<D>::kSize;
    StateAcc<D> stR;
    VecAcc<D> vr;
    load_state<D>(r0, stR, lane, w);
    load_vec<D>(r0 + Rec<D>::kZ, vr, lane, w);

    CR cq, ck, cv, cdo;
    float dn[CR::NV];
    float gv = 0.f;
    auto load_chunk = [&](int c) {
        cq.load(q + hoff, c, N, tid);
        ck.load(k + hoff, c, N, tid);
        cv.load(v + hoff, c, N, tid);
        cdo.load(dout + hoff, c, N, tid);
#pragma unroll
        for (int i = 0; i < CR::NV; ++i) {
            const int tok = c + CR::row(i, tid);
            dn[i] = tok < N ? rs[tok].x : 1.f;
        }
        if (tid < kC) gv = c + tid < N ? rs[c + tid].y : 0.f;
    };
    load_chunk(tok_begin + (nch - 1) * kC);

    for (int ci = nch - 1; ci >= 0; --ci) {
        const int c0 = tok_begin + ci * kC;
        publish_state<T, D>(stR, tRt, lane, w);
        store_vec<D>(s_r, vr, lane, w);
        // partial column sums of R over each state tile's 16 features
#pragma unroll
        for (int ia = 0; ia < ST::NAT; ++ia)
#pragma unroll
            for (int ib = 0; ib < ST::NBT; ++ib) {
                const f32x4 x = stR[ia][ib];
                const float cs = sum_over_groups(x[0] + x[1] + x[2] + x[3]);
                if (g == 0) s_wpart[ST::at0(w) + ia][(ST::bt0(w) + ib) * 16 + (lane & 15)] = cs;
            }
        stage_phi<T, D>(cq, tQ, tid);
        stage_elu<T, D>(ck, tE, tid);
        stage_raw<T, D>(cv, tV, tid);
        // G = round(dO / den) with the den saved by the prefix sweep (bitwise the same G).
#pragma unroll
        for (int i = 0; i < CR::NV; ++i) {
            const int t = CR::row(i, tid);
            const float inv = c0 + t < N ? rcp_f(dn[i]) : 0.f;
            uint4 packed;
            T* pk = reinterpret_cast<T*>(&packed);
#pragma unroll
            for (int e = 0; e < CR::EV; ++e) pk[e] = from_f32<T>(cdo.get(i, e) * inv);
            *reinterpret_cast<uint4*>(tG.granule(t, CR::gran(i, tid))) = packed;
        }
        if (tid < kC) s_g[tid] = gv;
        if (ci > 0) load_chunk(c0 - kC);
        const int tok = c0 + sl;
        const bool valid = tok < N;
        __syncthreads();
        if (tid < D) {
            float ws = 0.f;
#pragma unroll
            for (int at = 0; at < DT; ++at) ws += s_wpart[at][tid];
            s_w[tid] = ws;
        }

        // (1) dA_ts = G_t.V_s + g_t and A_ts = q_sum_t + phi(Q_t).E(K_s) for s <= t,
        //     stored [s][t] for this wave's key tile (all four token tiles, branch free).
        {
            const typename M::frag one = M::ones();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 acc_d = zero4(), acc_b = zero4(), acc_q = zero4();
#pragma unroll
                for (int k0 = 0; k0 < D; k0 += KS) {
                    const typename M::frag xq = M::ld(tQ, 16 * i, k0, lane);
                    acc_d = M::mma(M::ld(tG, 16 * i, k0, lane), M::ld(tV, s0, k0, lane), acc_d);
                    acc_b = M::mma(xq, M::ld(tE, s0, k0, lane), acc_b);
                    acc_q = M::mma(xq, one, acc_q);
                }
                const f32x4 gt4 = lds4(&s_g[16 * i + 4 * g]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool live = sl <= 16 * i + 4 * g + e;
                    acc_d[e] = live ? acc_d[e] + gt4[e] : 0.f;
                    acc_b[e] = live ? acc_b[e] + acc_q[e] : 0.f;
                }
                store_T(tdAt, 16 * i, s0, acc_d, lane);
                store_T(tAt, 16 * i, s0, acc_b, lane);
            }
        }
        // phi'(K) needs the raw inputs of the lane's output elements (cache-resident).
        Raw4<T> kraw[DT];
#pragma unroll
        for (int m = 0; m < DT; ++m) {
            if (valid) kraw[m].load(k + hoff + (int64_t)tok * D + 16 * m + 4 * g);
            else kraw[m].clear();
        }
        __syncthreads();  // s_w complete; this wave's dA^T, A^T rows written

        // (2) dphi(K)^T[a][s] = sum_t phi(Q)[t][a] dA[t][s] + sum_b R[a][b] V[s][b] + r[a]
        //     dV^T[b][s]      = sum_t G[t][b] A[t][s] + sum_a R[a][b] E[s][a] + w[b]
        f32x4 acck[DT], accv[DT];
#pragma unroll
        for (int m = 0; m < DT; ++m) {
            acck[m] = zero4();
            accv[m] = zero4();
        }
#pragma unroll
        for (int k0 = 0; k0 < kC; k0 += KS) {
            const typename M::frag yd = M::ld(tdAt, s0, k0, lane);
            const typename M::frag ya = M::ld(tAt, s0, k0, lane);
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                acck[m] = M::mma(M::ld_tr(tQ, k0, 16 * m, lane), yd, acck[m]);
                accv[m] = M::mma(M::ld_tr(tG, k0, 16 * m, lane), ya, accv[m]);
            }
        }
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += KS) {
            const typename M::frag yv = M::ld(tV, s0, k0, lane);
            const typename M::frag ye = M::ld(tE, s0, k0, lane);
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                acck[m] = M::mma(M::ld_tr(tRt, k0, 16 * m, lane), yv, acck[m]);
                accv[m] = M::mma(M::ld(tRt, 16 * m, k0, lane), ye, accv[m]);
            }
        }
        if (valid) {
            const int64_t roff = hoff + (int64_t)tok * D;
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                const int f0 = 16 * m + 4 * g;
                const f32x4 rv = lds4(&s_r[f0]);
                const f32x4 wv = lds4(&s_w[f0]);
                f32x4 xk, xv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xk[e] = (acck[m][e] + rv[e]) * dphi_f(kraw[m].get(e));
                    xv[e] = accv[m][e] + wv[e];
                }
                gstore4(dk + roff + f0, xk);
                gstore4(dv + roff + f0, xv);
            }
        }

        // (3) Suffix state: R += phi(Q)^T G, r += phi(Q)^T g.
        state_update<T, D, true, false>(stR, vr, vr, tQ, tG, s_g, nullptr, lane, w);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------
hipError_t launch_bwd_prefix(int dt, int d, const void* q, const void* k, const void* v, const void* dout, void* dq,
                             float* rowstat, float* rrec, const float* rec, int64_t BH, int64_t N, SegPlan p,
                             hipStream_t s) {
    const dim3 grid((unsigned)(p.nseg * BH));
#define LA_BWDP(TT, DD)                                                                                           \
    hipLaunchKernelGGL((bwd_prefix_kernel<TT, DD>), grid, dim3(kBlock), 0, s, (const TT*)q, (const TT*)k,        \
                       (const TT*)v, (const TT*)dout, (TT*)dq, (float2*)rowstat, rrec, rec, (int)N, p.cps, p.nseg)
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

hipError_t launch_bwd_suffix(int dt, int d, const void* q, const void* k, const void* v, const void* dout, void* dk,
                             void* dv, const float* rowstat, const float* rrec, int64_t BH, int64_t N, SegPlan p,
                             hipStream_t s) {
    const dim3 grid((unsigned)(p.nseg * BH));
#define LA_BWDS(TT, DD)                                                                                           \
    hipLaunchKernelGGL((bwd_suffix_kernel<TT, DD>), grid, dim3(kBlock), 0, s, (const TT*)q, (const TT*)k,        \
                       (const TT*)v, (const TT*)dout, (TT*)dk, (TT*)dv, (const float2*)rowstat, rrec, (int)N, p.cps, \
                       p.nseg)
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
