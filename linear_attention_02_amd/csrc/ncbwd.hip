// ncbwd.hip -- non-causal backward of kernelized linear attention for gfx950.
//
// The non-causal form of the proposition "Linear Attention via Kernel
// Decomposition" (page "Efficient Transformers Survey", section "Linear
// Attention") reads one global state per head:
//   O_i = phi(Q_i)^T S / phi(Q_i)^T z,  S = sum_j phi(K_j) V_j^T,  z = sum_j phi(K_j).
// The pages print no backward; the chain rule on that form gives, with
// den_i = phi(Q_i).z, G_i = dO_i / den_i and g_i = -G_i . O_i:
//   dphi(Q_i) = S G_i + g_i z,
//   dphi(K_j) = R V_j + r,  dV_j = R^T phi(K_j),
//   R = sum_i phi(Q_i) G_i^T,  r = sum_i g_i phi(Q_i)   (both over every query),
// then dQ = dphi(Q) phi'(Q) and dK = dphi(K) phi'(K).
//
// Numerics follow the causal backward: the key state is split around the
// constant 1 in phi(K) = 1 + E(K) (S = 1 P^T + S_E, z = N 1 + z_E) so that only
// S_E enters an MFMA, and
//   dphi(Q_i) = [G_i.P + g_i N] 1 + S_E G_i + g_i z_E,
//   G_i . num_i = q_sum_i (G_i.P) + phi(Q_i).(S_E G_i)   (num_i = S^T phi(Q_i)),
// with G rounded to the operand type once and g formed from the very S_E G
// that dQ uses, so sum_a dphi(Q_i)_a phi(Q_ia) = 0 holds for the values used.
// On the key side dV_j = w + R^T E(K_j) with w = sum_a R[a][.].
//
// Work decomposition (one workgroup of 4 wavefronts per (segment, head), numbered
// segment-major like the forward's):
//   seg_state (or the forward's saved records) [+ total]: the key aggregates;
//   ncbwd_q : every row of the segment: den, G, g, dQ; the segment's (R, r) record;
//   [total]  : per head, the sum of the (R, r) records;
//   ncbwd_kv: every key row of the segment: dK, dV from (R, r).
#include "chunk.h"

namespace la {

// ---------------------------------------------------------------------------------------
// ncbwd_q.  Wavefront w owns token tile 16 w .. 16 w + 15 of every chunk and holds
// phi(Q) and dO of its rows in accumulator order (lane l: row l & 15, features
// 16 m + 4 (l >> 4) + e), so S_E G comes out of the MFMAs in the layout of the
// row reductions and the dQ epilogue.  phi(Q), G and g of the chunk are staged
// in LDS (double-buffered, one barrier per chunk) for the update of (R, r),
// which contracts over all 64 tokens.
// FM: the feature map (FeatGiven: phi is the identity and the rank-1 parts vanish).
// kMode (given features, for heads whose features come in several blocks): 0 the pass
// above; 1 statistics only: den of every row from den_in (one per value head), and
// (den, G . num of this block) to rowstat, no dQ and no record; 2 the pass with (den, g)
// of every row read from rowstat.  dout is read at head bh / Gv.
template <typename T, int D, class FM = FeatElu, int kMode = 0>
__global__ __launch_bounds__(kBlock, 2) void ncbwd_q_kernel(const T* __restrict__ q, const T* __restrict__ dout,
                                                         T* __restrict__ dq, const float* __restrict__ total,
                                                         int ntotal, float* __restrict__ rrec, int N, int cps,
                                                         int nseg, int BH, int Gv, const float* __restrict__ den_in,
                                                         float2* __restrict__ rowstat) {
    static_assert(kMode == 0 || !FM::kSplit, "the statistics modes are built for given features");
    using M = Mma<T>;
    constexpr int KS = M::KSTEP;
    constexpr int DT = D / 16;
    constexpr int NY = D / 4;
    __shared__ __attribute__((aligned(16))) T sm_st[D * D];
    __shared__ __attribute__((aligned(16))) T sm_q[2][kC * D];
    __shared__ __attribute__((aligned(16))) T sm_g[2][kC * D];
    __shared__ __attribute__((aligned(16))) float s_z[D], s_p[D], s_g[2][kC];
    const Tile<T, D, D> tSt{sm_st};

    const int seg = blockIdx.x / BH, bh = blockIdx.x % BH;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 4;
    const int64_t hoff = (int64_t)bh * N * D;
    const uint32_t hbytes = (uint32_t)N * D * sizeof(T);
    const int64_t voff = (int64_t)(bh / Gv) * N * D;
    const GBuf bq(q + hoff, hbytes), bdo(dout + voff, hbytes), bdq(dq + hoff, hbytes);
    const int tok_begin = seg * cps * kC;
    const int tok_end = min(N, tok_begin + cps * kC);

    // The head's key state: the in-order sum of its ntotal records (the segment
    // records themselves, or one precomputed total).
    {
        StateAcc<D> st;
        VecAcc<D> vz, vp;
        zero_state<D>(st);
        zero_vec<D>(vz);
        zero_vec<D>(vp);
        add_records<D, 64>(total + (int64_t)bh * ntotal * Rec<D>::kSize, Rec<D>::kSize, ntotal, st, vz, vp, lane, w);
        publish_state<T, D>(st, tSt, lane, w);
        store_vec<D>(s_z, vz, lane, w);
        store_vec<D>(s_p, vp, lane, w);
    }
    StateAcc<D> stR;
    VecAcc<D> vr;
    zero_state<D>(stR);
    zero_vec<D>(vr);
    const float n = (float)N;
    const int tl = 16 * w + (lane & 15);

    // Rows of kAhead chunks are in flight per wave (one: a second measured no faster here).
    constexpr int kAhead = 1;
    RowAcc<T, D> qb[kAhead], db[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
        const int c = tok_begin + u * kC;
        qb[u].load(bq, c < tok_end ? c + 16 * w : N, lane);  // past the segment: row N, zeros, no traffic
        db[u].load(bdo, c < tok_end ? c + 16 * w : N, lane);
    }
    __syncthreads();

    auto chunk = [&](RowAcc<T, D>& qrow, RowAcc<T, D>& cdo, int c0, int buf) {
        const Tile<T, kC, D> tQ{sm_q[buf]}, tG{sm_g[buf]};
        const int tok = c0 + tl;
        const bool valid = tok < N;
        // phi(Q) of this lane's row as the operand type rounds it (rows past
        // the head read as 0 and give phi = 1; their G and g are 0), q_sum, phi(Q).z_E.
        float y[NY];
        float qs = 0.f, zd = 0.f;
#pragma unroll
        for (int m = 0; m < DT; ++m) {
            const f32x4 zv = lds4(&s_z[16 * m + 4 * g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = to_f32(from_f32<T>(FM::phi(qrow.get(4 * m + e))));
                y[4 * m + e] = x;
                qs += x;
                zd += x * zv[e];
            }
            store4(&tQ.at(tl, 16 * m + 4 * g), f32x4{y[4 * m], y[4 * m + 1], y[4 * m + 2], y[4 * m + 3]});
        }
        qs = FM::kSplit ? sum_over_groups(qs) : 0.f;  // no rank-1 parts when unsplit
        float den, gin = 0.f;
        if constexpr (kMode == 0) {
            den = qs * n + sum_over_groups(zd);
        } else if constexpr (kMode == 1) {
            den = valid ? den_in[(int64_t)(bh / Gv) * N + tok] : 1.f;
        } else {
            const float2 rs = valid ? rowstat[(int64_t)bh * N + tok] : float2{1.f, 0.f};
            den = rs.x;
            gin = rs.y;
        }
        const float inv_den = rcp_f(den);

        // G = round(dO / den) (staged for the R update) and G.P.
        float gy[NY];
        float gp = 0.f;
#pragma unroll
        for (int m = 0; m < DT; ++m) {
            const f32x4 pv = lds4(&s_p[16 * m + 4 * g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gy[4 * m + e] = valid ? to_f32(from_f32<T>(cdo.get(4 * m + e) * inv_den)) : 0.f;
                if constexpr (FM::kSplit) gp += gy[4 * m + e] * pv[e];
            }
            store4(&tG.at(tl, 16 * m + 4 * g), f32x4{gy[4 * m], gy[4 * m + 1], gy[4 * m + 2], gy[4 * m + 3]});
        }
        gp = sum_over_groups(gp);
        // The rows kAhead chunks on (past the segment: row N, zeros without memory traffic).
        const int nxt = c0 + kAhead * kC < tok_end ? c0 + kAhead * kC + 16 * w : N;
        qrow.load(bq, nxt, lane);
        cdo.load(bdo, nxt, lane);

        // (S_E G)_a for this wave's rows (accumulator [a][t]).
        f32x4 accQ[DT];
#pragma unroll
        for (int m = 0; m < DT; ++m) accQ[m] = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += KS) {
            const typename M::frag yg = M::vals_op(gy, k0);
#pragma unroll
            for (int m = 0; m < DT; ++m) accQ[m] = M::mma(M::ld_tr_acc(tSt, k0, 16 * m, lane), yg, accQ[m]);
        }
        // g = -(q_sum (G.P) + phi(Q).(S_E G)) / den.
        float s3 = 0.f;
        if constexpr (kMode != 2) {
#pragma unroll
            for (int m = 0; m < DT; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) s3 += y[4 * m + e] * accQ[m][e];
            s3 = sum_over_groups(s3);
        }
        if constexpr (kMode == 1) {
            // This block's G . num of the row with the head's den.
            if (g == 0 && valid) rowstat[(int64_t)bh * N + tok] = float2{den, s3};
            return;
        }
        const float gt = kMode == 2 ? (valid ? gin : 0.f) : (valid ? -(qs * gp + s3) * inv_den : 0.f);
        if (g == 0) s_g[buf][tl] = gt;

        // dQ = ((S_E G)_a + g z_E[a] + G.P + g N) phi'(Q_a), phi' = min(phi, 1).
        const float bracket = FM::kSplit ? gp + gt * n : 0.f;
#pragma unroll
        for (int m = 0; m < DT; ++m) {
            const int f0 = 16 * m + 4 * g;
            const f32x4 zv = lds4(&s_z[f0]);
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[e] = (accQ[m][e] + zv[e] * gt + bracket) * FM::dphi_at_phi(y[4 * m + e]);
            gstore4<T>(bdq, (uint32_t)(tok * D + f0), x);
        }
        __syncthreads();  // the chunk's phi(Q), G and g are staged

        // R += phi(Q)^T G, r += phi(Q)^T g.
        state_update<T, D, true, false>(stR, vr, vr, tQ, tG, s_g[buf], nullptr, lane, w);
    };
    // LDS buffers alternate by chunk.
    for (int c00 = tok_begin, ci = 0; c00 < tok_end; c00 += kAhead * kC) {
#pragma unroll
        for (int u = 0; u < kAhead; ++u, ++ci) {
            const int c0 = c00 + u * kC;
            if (c0 >= tok_end) break;
            chunk(qb[u], db[u], c0, ci & 1);
        }
    }
    if constexpr (kMode == 1) return;
    // Record [R^T | r | 0].
    float* rr = rrec + ((int64_t)bh * nseg + seg) * Rec<D>::kSize;
    store_state<D>(rr, stR, lane, w);
    store_vec<D>(rr + Rec<D>::kZ, vr, lane, w);
    if (tid < D) rr[Rec<D>::kP + tid] = 0.f;
}

// ---------------------------------------------------------------------------------------
// ncbwd_kv.  (R, r) of the head (the in-order sum of ntotal records) is rounded
// into LDS once; wavefront w then walks key tile 16 w .. of every chunk on its
// own (no barrier in the loop), with K and V of its rows in registers in
// accumulator order (E(K) and phi'(K) from one exp).
template <typename T, int D, class FM = FeatElu>
__global__ __launch_bounds__(kBlock, 2) void ncbwd_kv_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                          T* __restrict__ dk, T* __restrict__ dv,
                                                          const float* __restrict__ rtotal, int ntotal, int N,
                                                          int cps, int BH, int Gv) {
    using M = Mma<T>;
    constexpr int KS = M::KSTEP;
    constexpr int DT = D / 16;
    constexpr int NY = D / 4;
    __shared__ __attribute__((aligned(16))) T sm_rt[D * D];
    __shared__ __attribute__((aligned(16))) float s_r[D];
    // R^T is read as accumulator-order operands (ld_acc) and transposed: bf16 tiles keep
    // those operands' columns together.
    const Tile<T, D, D, std::is_same<T, bf16>::value> tRt{sm_rt};

    const int seg = blockIdx.x / BH, bh = blockIdx.x % BH;
    const int lane = threadIdx.x & 63, w = wave_id(), g = lane >> 4;
    const int64_t hoff = (int64_t)bh * N * D;
    const uint32_t hbytes = (uint32_t)N * D * sizeof(T);
    const GBuf bk(k + hoff, hbytes), bv(v + (int64_t)(bh / Gv) * N * D, hbytes), bdk(dk + hoff, hbytes),
        bdv(dv + hoff, hbytes);
    const int tok_begin = seg * cps * kC;
    const int tok_end = min(N, tok_begin + cps * kC);
    {
        StateAcc<D> stR;
        VecAcc<D> vr, vunused;
        zero_state<D>(stR);
        zero_vec<D>(vr);
        zero_vec<D>(vunused);
        add_records<D, 64, false>(rtotal + (int64_t)bh * ntotal * Rec<D>::kSize, Rec<D>::kSize, ntotal, stR, vr,
                                  vunused, lane, w);
        publish_state<T, D>(stR, tRt, lane, w);
        store_vec<D>(s_r, vr, lane, w);
    }
    // Rows of kAhead chunks are in flight per wave (registers allowing).
    constexpr int kAhead = D * sizeof(T) <= 128 ? 2 : 1;
    RowAcc<T, D> kb[kAhead], vb[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
        const int c = tok_begin + u * kC;
        kb[u].load(bk, c < tok_end ? c + 16 * w : N, lane);  // past the segment: row N, zeros, no traffic
        vb[u].load(bv, c < tok_end ? c + 16 * w : N, lane);
    }
    __syncthreads();

    auto chunk = [&](RowAcc<T, D>& kr, RowAcc<T, D>& vrow, int c0) {
        // For d <= 64 the compiler keeps the R operands in registers across the
        // loop; at d = 128 they would take 256 registers, so they are re-read
        // from LDS every chunk (the fence stops the loads from being hoisted).
        if constexpr (D > 64) __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const int tok = c0 + 16 * w + (lane & 15);
        // Raw K and V of this lane's row; E(K) is formed where the MFMAs take it
        // and phi'(K) in the epilogue (short register lifetimes at d = 128).
        const RowAcc<T, D> kcur = kr, vcur = vrow;
        const int nxt = c0 + kAhead * kC < tok_end ? c0 + kAhead * kC + 16 * w : N;
        kr.load(bk, nxt, lane);
        vrow.load(bv, nxt, lane);

        // dphi(K)^T[a][s] = sum_b R[a][b] V[s][b] (+ r[a]);
        // dV^T[b][s]      = sum_a R[a][b] E[s][a] + sum_a R[a][b].
        f32x4 acck[DT], accv[DT];
#pragma unroll
        for (int m = 0; m < DT; ++m) {
            acck[m] = zero4();
            accv[m] = zero4();
        }
        const typename M::frag one = M::ones();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += KS) {
            if constexpr (D > 64) __atomic_signal_fence(__ATOMIC_SEQ_CST);  // one k-step's operands at a time
            float ke[NY];
#pragma unroll
            for (int i = 0; i < NY; ++i) ke[i] = to_f32(from_f32<T>(FM::e(kcur.get(i))));
            const typename M::frag yv = M::raw_op(vcur.r, k0);
            const typename M::frag ye = M::vals_op(ke, k0);
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                const typename M::frag xr = M::ld_acc(tRt, 16 * m, k0, lane);
                acck[m] = M::mma(M::ld_tr_acc(tRt, k0, 16 * m, lane), yv, acck[m]);
                accv[m] = M::mma(xr, ye, accv[m]);
                if constexpr (FM::kSplit) accv[m] = M::mma(xr, one, accv[m]);  // w = sum_a R[a][.]
            }
        }
#pragma unroll
        for (int m = 0; m < DT; ++m) {
            const int f0 = 16 * m + 4 * g;
            const f32x4 rv = lds4(&s_r[f0]);
            f32x4 xk;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                xk[e] = (acck[m][e] + rv[e]) * (FM::kSplit ? dphi_f(kcur.get(4 * m + e)) : 1.f);
            gstore4<T>(bdk, (uint32_t)(tok * D + f0), xk);
            gstore4<T>(bdv, (uint32_t)(tok * D + f0), accv[m]);
        }
    };
    for (int c00 = tok_begin; c00 < tok_end; c00 += kAhead * kC) {
#pragma unroll
        for (int u = 0; u < kAhead; ++u) {
            const int c0 = c00 + u * kC;
            if (c0 >= tok_end) break;
            chunk(kb[u], vb[u], c0);
        }
    }
}

// ---------------------------------------------------------------------------------------
hipError_t launch_ncbwd_q(int dt, int d, const void* q, const void* dout, void* dq, const float* total, int ntotal,
                          float* rrec, int64_t BH, int64_t N, SegPlan p, hipStream_t s, int feat, int mode, int Gv,
                          const float* den_in, float* rowstat) {
    const dim3 grid((unsigned)(p.nseg * BH));
    if (mode != 0 && feat != kFeatGiven) return hipErrorInvalidValue;
#define LA_NCQ_ARGS(TT) (const TT*)q, (const TT*)dout, (TT*)dq, total, ntotal, rrec, (int)N, p.cps, p.nseg, (int)BH, \
                        Gv, den_in, reinterpret_cast<float2*>(rowstat)
#define LA_NCQ(TT, DD)                                                                                            \
    if (feat != kFeatGiven)                                                                                       \
        hipLaunchKernelGGL((ncbwd_q_kernel<TT, DD>), grid, dim3(kBlock), 0, s, LA_NCQ_ARGS(TT));                 \
    else if (mode == 1)                                                                                           \
        hipLaunchKernelGGL((ncbwd_q_kernel<TT, DD, FeatGiven, 1>), grid, dim3(kBlock), 0, s, LA_NCQ_ARGS(TT));   \
    else if (mode == 2)                                                                                           \
        hipLaunchKernelGGL((ncbwd_q_kernel<TT, DD, FeatGiven, 2>), grid, dim3(kBlock), 0, s, LA_NCQ_ARGS(TT));   \
    else                                                                                                          \
        hipLaunchKernelGGL((ncbwd_q_kernel<TT, DD, FeatGiven>), grid, dim3(kBlock), 0, s, LA_NCQ_ARGS(TT))
    if (dt == kBF16) {
        switch (d) {
            case 32: LA_NCQ(bf16, 32); break;
            case 64: LA_NCQ(bf16, 64); break;
            case 128: LA_NCQ(bf16, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (d) {
            case 32: LA_NCQ(float, 32); break;
            case 64: LA_NCQ(float, 64); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef LA_NCQ
#undef LA_NCQ_ARGS
    return hipGetLastError();
}

hipError_t launch_ncbwd_kv(int dt, int d, const void* k, const void* v, void* dk, void* dv, const float* rtotal,
                           int ntotal, int64_t BH, int64_t N, SegPlan p, hipStream_t s, int feat, int Gv) {
    const dim3 grid((unsigned)(p.nseg * BH));
#define LA_NCKV(TT, DD)                                                                                           \
    if (feat == kFeatGiven)                                                                                       \
        hipLaunchKernelGGL((ncbwd_kv_kernel<TT, DD, FeatGiven>), grid, dim3(kBlock), 0, s, (const TT*)k,         \
                           (const TT*)v, (TT*)dk, (TT*)dv, rtotal, ntotal, (int)N, p.cps, (int)BH, Gv);              \
    else                                                                                                         \
        hipLaunchKernelGGL((ncbwd_kv_kernel<TT, DD>), grid, dim3(kBlock), 0, s, (const TT*)k, (const TT*)v,      \
                           (TT*)dk, (TT*)dv, rtotal, ntotal, (int)N, p.cps, (int)BH, Gv)
    if (dt == kBF16) {
        switch (d) {
            case 32: LA_NCKV(bf16, 32); break;
            case 64: LA_NCKV(bf16, 64); break;
            case 128: LA_NCKV(bf16, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (d) {
            case 32: LA_NCKV(float, 32); break;
            case 64: LA_NCKV(float, 64); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef LA_NCKV
    return hipGetLastError();
}

}  // namespace la
