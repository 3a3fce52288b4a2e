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
// Work decomposition (one workgroup of 4 wavefronts per (segment, head),
// numbered segment-major like the forward's):
//   seg_state (forward kernel, or the forward's saved records): the aggregates
//               (S_E, z_E, P) of every segment;
//   bwd_prefix: starts from the sum of the records before the segment (segment
//               order); chunks in order: den, G, g, dA, dQ; saves den and g per
//               row and the segment's aggregates R = sum phi(Q) G^T, r = sum g phi(Q);
//   bwd_suffix: starts from the sum of the (R, r) records after the segment
//               (reverse segment order); chunks in reverse: dK, dV from the
//               in-chunk terms plus the suffix state.
#include "chunk.h"

namespace la {

// LDS of the two sweeps, carved from one byte buffer so that the fused kernel
// can run both sweeps in the same workgroup over the same bytes.
template <typename T, int D>
struct BwdPrefixLds {
    static constexpr size_t kTile = (size_t)kC * D * sizeof(T), kSt = (size_t)D * D * sizeof(T);
    static constexpr size_t oE = 0, oV = 2 * kTile, oQ = 4 * kTile, oG = 5 * kTile, oSt = 6 * kTile;
    static constexpr size_t oZ = oSt + kSt, oP = oZ + D * 4, oGv = oP + D * 4, kBytes = oGv + kC * 4;
};
template <typename T, int D>
struct BwdSuffixLds {
    // The G tiles sit 256 bytes past a multiple of 512 from the phi(Q) tiles (the bank
    // mapping repeats every 256 bytes): no paired LDS read can then fetch a phi(Q) half
    // and a G half together, which would cost register moves to assemble the operands.
    static constexpr size_t kTile = (size_t)kC * D * sizeof(T), kSt = (size_t)D * D * sizeof(T);
    static constexpr size_t oQ = 0, oG = 2 * kTile + 256, oRt = oG + 2 * kTile + 256, oGv = oRt + 2 * kSt,
                            oR = oGv + 2 * kC * 4;
    static constexpr size_t kBytes = oR + 2 * D * 4;
};

// ---------------------------------------------------------------------------------------
// bwd_prefix.  Wavefront w owns the token tile t = 16 w .. 16 w + 15 of every
// chunk and keeps phi(Q_t) and G_t of its tokens in registers in accumulator
// order, so that B, G V and S_E G come out of MFMAs in the layout the row
// reductions and the dQ epilogue use; dA stays in the accumulators that form it
// and feeds the dQ product directly.  phi(Q) and G are also written to LDS for
// the R update, which contracts over all tokens of the chunk.
// Whether the prefix sweep forms the segment's (R, r) record itself: at d = 128
// the registers of R would make the sweep spill, and the rseg pass forms it.
template <int D>
struct BwdPrefixForms {
    static constexpr bool kRecord = D <= 64;
};

// kCoherentRecord: the segment's (R, r) record is written with agent-coherent
// stores (read by other workgroups of the same launch).
// kRecord: the sweep also forms that record (for d = 128 the registers of R are
// left to the sweep, and rseg forms the record from the saved den and g).
// init / init_n (nullable): the forward's start state in split form and its token
// count, one record and one count per head (the carried state starts from them).
// FM: the feature map (FeatGiven: phi is the identity, E = phi and the rank-1 terms of the
// split vanish: no q_sum, P or n anywhere, and dphi = 1).
// Gv: heads per value head (v, dout, and den_in, of head bh / Gv: feature blocks of one head).
// kMode, for attention split over feature blocks that share one normalization:
//   0: the sweep as stated above;
//   1: statistics: with the denominator den_in of the whole head given, G = round(dO / den),
//      and each row's G . num of this block goes to rowstat (den, G . num); no dQ, no record;
//   2: from given statistics: den and g are read from rowstat (den, g), the rest as in 0.
template <typename T, int D, bool kCoherentRecord, bool kRecord = true, bool kState = false, class FM = FeatElu,
          int kMode = 0>
__device__ __forceinline__ void bwd_prefix_body(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    T* __restrict__ dq, float2* __restrict__ rowstat, float* __restrict__ rrec, const float* __restrict__ rec, int N,
    int cps, int nseg, int prefixed, int seg, int bh, char* lds, const float* __restrict__ init,
    const float* __restrict__ init_n, int Gv = 1, const float* __restrict__ den_in = nullptr) {
    using M = Mma<T>;
    constexpr int KS = M::KSTEP;
    constexpr int DT = D / 16;
    constexpr int NY = D / 4;  // row values per lane in accumulator order
    constexpr bool kFormsRecord = kRecord && kMode != 1;
    // E(K) and V are read after the mid-chunk barrier and are double-buffered;
    // phi(Q), G and g are written after the first barrier and read before the
    // next chunk's first barrier; S_E^T, z_E and P are read before the second.
    using L = BwdPrefixLds<T, D>;
    T(*const sm_e)[kC * D] = reinterpret_cast<T(*)[kC * D]>(lds + L::oE);
    T(*const sm_v)[kC * D] = reinterpret_cast<T(*)[kC * D]>(lds + L::oV);
    T* const sm_q = reinterpret_cast<T*>(lds + L::oQ);
    T* const sm_g = reinterpret_cast<T*>(lds + L::oG);
    T* const sm_st = reinterpret_cast<T*>(lds + L::oSt);
    float* const s_z = reinterpret_cast<float*>(lds + L::oZ);
    float* const s_p = reinterpret_cast<float*>(lds + L::oP);
    float* const s_g = reinterpret_cast<float*>(lds + L::oGv);
    const Tile<T, kC, D> tQ{sm_q}, tG{sm_g};
    const Tile<T, D, D> tSt{sm_st};

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 4;
    const int64_t hoff = (int64_t)bh * N * D, voff = (int64_t)(bh / Gv) * N * D;
    const uint32_t hbytes = (uint32_t)N * D * sizeof(T);
    const GBuf bq(q + hoff, hbytes), bk(k + hoff, hbytes), bv(v + voff, hbytes), bdo(dout + voff, hbytes);
    const GBuf bdq(dq + hoff, hbytes), brs(rowstat + (int64_t)bh * N, (uint32_t)N * 8);
    const int tok_begin = seg * cps * kC;
    const int tok_end = min(N, tok_begin + cps * kC);

    // Prefix state (S_E, z_E, P) at the start of the segment: the records of the
    // segments before it, summed in order; segment aggregates from zero.
    // The first chunk's loads are in flight while the records arrive.
    ChunkRegs<T, D> ck, cv;
    ChunkRegs<T, D, true> cq;
    RowAcc<T, D> cdo;
    ck.load(bk, tok_begin, tid);
    cv.load(bv, tok_begin, tid);
    cq.load(bq, tok_begin + 16 * w, tid);
    cdo.load(bdo, tok_begin + 16 * w, lane);
    StateAcc<D> stS, stR;
    VecAcc<D> vz, vp, vr;
    float n = (float)tok_begin;
    constexpr int kRecRegs = 192 - 4 * (int)(sizeof(ChunkRegs<T, D>) / 4);
    if constexpr (kState) {
        carried_state<D, kRecRegs>(rec + (int64_t)bh * nseg * Rec<D>::kSize, Rec<D>::kSize, seg, prefixed != 0, stS,
                                   vz, vp, lane, w, init != nullptr ? init + (int64_t)bh * Rec<D>::kSize : nullptr);
        if (init_n != nullptr) n += init_n[bh];
    } else {
        carried_state<D, kRecRegs>(rec + (int64_t)bh * nseg * Rec<D>::kSize, Rec<D>::kSize, seg, prefixed != 0, stS,
                                   vz, vp, lane, w);
    }
    zero_state<D>(stR);
    zero_vec<D>(vr);
    // Whether the segment's key features hold an inf or NaN: the dQ product over the
    // k-step holding the diagonal tile then takes E(K) with non-finite entries replaced
    // by 0 (a masked dA is an exact zero, but 0 * inf = NaN would reach earlier rows);
    // rows t >= s still become NaN through their den, formed from the unreplaced tile.
    // The segment's own forward record holds z_E = the sum of its E(K), non-finite
    // exactly then (running-sum records: the next one stands in; the last segment of
    // such a plan always takes the path).
    bool ebad;
    {
        const int own = prefixed ? seg + 1 : seg;
        bool bad = own >= nseg;
        if (!bad) {
            const float* p = rec + ((int64_t)bh * nseg + own) * Rec<D>::kSize + Rec<D>::kZ;
#pragma unroll
            for (int i = 0; i < (D + kWave - 1) / kWave; ++i)
                if (i * kWave + lane < D) bad = bad || !finite_f(p[i * kWave + lane]);
        }
        ebad = __builtin_amdgcn_ballot_w64(bad) != 0;
    }

    // Wavefront w takes token tile tt = (w + ci) mod 4 of chunk ci: the causal
    // mask leaves tt + 1 key tiles, and the rotation spreads that work evenly
    // over the SIMDs.

    int buf = 0, ci = 0;
    for (int c0 = tok_begin; c0 < tok_end; c0 += kC, buf ^= 1, ++ci) {
        const Tile<T, kC, D> tE{sm_e[buf]}, tV{sm_v[buf]};
        const int tt = (w + ci) & 3, tt_next = (w + ci + 1) & 3;
        const int tl = 16 * tt + (lane & 15);
        publish_state<T, D>(stS, tSt, lane, w);
        store_vec<D>(s_z, vz, lane, w);
        store_vec<D>(s_p, vp, lane, w);
        stage_elu<T, D, FM>(ck, tE, tid);
        stage_raw<T, D>(cv, tV, tid);
        // Loads past the segment are aimed at row N: out of the buffer's range,
        // they return zeros without touching memory, and the loop stays branch free.
        const int nxt = c0 + kC < tok_end ? c0 + kC : N;
        ck.load(bk, nxt, tid);
        cv.load(bv, nxt, tid);
        const int tok = c0 + tl;
        const bool valid = tok < N;
        __syncthreads();

        // phi(Q) of this wave's rows: staged (for the R update) and read back in
        // accumulator order where it is used (short register lifetimes).
        stage_phi<T, D, true, FM>(cq, tQ, tid, 16 * tt);
        cq.load(bq, nxt < N ? nxt + 16 * tt_next : N, tid);
        wave_lds_sync();
        auto read_y = [&](float* y) {
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                const f32x4 x = lds4(&tQ.at(tl, 16 * m + 4 * g));
#pragma unroll
                for (int e = 0; e < 4; ++e) y[4 * m + e] = x[e];
            }
        };

        // (1) B_ts = phi(Q_t).E(K_s) for s <= t (accumulator [s][t]), q_sum_t, den_t.
        f32x4 accB[4];
        float qs_t, rowB = 0.f, zd = 0.f;
        {
            float y[NY];
            read_y(y);
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                const f32x4 zv = lds4(&s_z[16 * m + 4 * g]);
#pragma unroll
                for (int e = 0; e < 4; ++e) zd += y[4 * m + e] * zv[e];
            }
            const typename M::frag one = M::ones();
            f32x4 accq = zero4();
#pragma unroll
            for (int j = 0; j < 4; ++j) accB[j] = zero4();
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += KS) {
                const typename M::frag yq = M::vals_op(y, k0);
                if constexpr (FM::kSplit) accq = M::mma(one, yq, accq);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (j <= tt) accB[j] = M::mma(M::ld_acc(tE, 16 * j, k0, lane), yq, accB[j]);
            }
            qs_t = FM::kSplit ? accq[0] : 0.f;  // no rank-1 parts when unsplit
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j < tt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) rowB += accB[j][e];
                } else if (j == tt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float b = (4 * g + e) <= (lane & 15) ? accB[j][e] : 0.f;
                        accB[j][e] = b;
                        rowB += b;
                    }
                }
            }
        }
        float den = qs_t * (n + (float)(tl + 1)) + sum_over_groups(rowB) + sum_over_groups(zd);
        if constexpr (kMode == 1) den = valid ? den_in[(int64_t)(bh / Gv) * N + tok] : 1.f;
        if constexpr (kMode == 2) den = valid ? brs.ld4f((uint32_t)tok * 8) : 1.f;
        const float inv_den = rcp_f(den);

        // (2)+(3) G_t = round(dO_t / den_t) of this wave's rows (staged for the R
        //     update), G_t.P, G_t.V_s (accumulator [s][t]) and (S_E G_t)_a (accumulator [a][t]).
        f32x4 accGV[4], accQ[DT];
        float gp = 0.f;
        {
            float gy[NY];
            // bf16: G rounded once and kept packed for the staged tile and the MFMA operands.
            // Rows past the head read dO = 0; with the elu map their den is positive, so G = 0
            // there without a select (a given map can leave den = 0 there).
            T gb[NY];
#pragma unroll
            for (int i = 0; i < NY; ++i) {
                float x = cdo.get(i) * inv_den;
                if (!FM::kSplit || sizeof(T) != 2) x = valid ? x : 0.f;
                gb[i] = from_f32<T>(x);
                gy[i] = to_f32(gb[i]);
            }
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                if constexpr (sizeof(T) == 2)
                    *reinterpret_cast<uint2*>(&tG.at(tl, 16 * m + 4 * g)) = *reinterpret_cast<const uint2*>(&gb[4 * m]);
                else
                    store4(&tG.at(tl, 16 * m + 4 * g), f32x4{gy[4 * m], gy[4 * m + 1], gy[4 * m + 2], gy[4 * m + 3]});
                if constexpr (FM::kSplit) {
                    const f32x4 pv = lds4(&s_p[16 * m + 4 * g]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) gp += gy[4 * m + e] * pv[e];
                }
            }
            cdo.load(bdo, nxt < N ? nxt + 16 * tt_next : N, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) accGV[j] = zero4();
#pragma unroll
            for (int m = 0; m < DT; ++m) accQ[m] = zero4();
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += KS) {
                typename M::frag yg;
                if constexpr (sizeof(T) == 2)
                    yg = *reinterpret_cast<const typename M::frag*>(&gb[k0 / 4]);
                else
                    yg = M::vals_op(gy, k0);
#pragma unroll
                for (int m = 0; m < DT; ++m) accQ[m] = M::mma(M::ld_tr_acc(tSt, k0, 16 * m, lane), yg, accQ[m]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (j <= tt) accGV[j] = M::mma(M::ld_acc(tV, 16 * j, k0, lane), yg, accGV[j]);
            }
        }
        gp = sum_over_groups(gp);

        // (4) g_t = -(G_t . num_t) / den_t with
        //     G_t . num_t = sum_{s<=t} A_ts (G_t.V_s) + q_sum_t (G_t.P) + phi(Q_t).(S_E G_t).
        float s1 = 0.f, s3 = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < tt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) s1 += (qs_t + accB[j][e]) * accGV[j][e];
            } else if (j == tt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) s1 += (4 * g + e) <= (lane & 15) ? (qs_t + accB[j][e]) * accGV[j][e] : 0.f;
            }
        }
        float y[NY];
        read_y(y);
#pragma unroll
        for (int m = 0; m < DT; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) s3 += y[4 * m + e] * accQ[m][e];
        float gt;
        if constexpr (kMode == 0)
            gt = valid ? -(sum_over_groups(s1) + qs_t * gp + sum_over_groups(s3)) * inv_den : 0.f;
        else if constexpr (kMode == 1)  // this block's G . num
            gt = valid ? sum_over_groups(s1) + qs_t * gp + sum_over_groups(s3) : 0.f;
        else
            gt = valid ? brs.ld4f((uint32_t)tok * 8 + 4) : 0.f;
        if (g == 0) {
            s_g[tl] = gt;
            if constexpr (kMode != 2) brs.st8((uint32_t)tok * 8, make_uint2(__float_as_uint(den), __float_as_uint(gt)));
        }
        if constexpr (kMode != 1) {

        // (5) dA_ts = G_t.V_s + g_t for s <= t, in place; its row sums.
        float rowdA = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < tt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    accGV[j][e] += gt;
                    rowdA += accGV[j][e];
                }
            } else if (j == tt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a = (4 * g + e) <= (lane & 15) ? accGV[j][e] + gt : 0.f;
                    accGV[j][e] = a;
                    rowdA += a;
                }
            }
        }
        rowdA = sum_over_groups(rowdA);

        // (6) dphi(Q)^T[a][t] = (S_E G_t)_a + sum_s E[s][a] dA[t][s] + z_E[a] g_t + bracket_t;
        //     dQ = dphi(Q) phi'(Q) with phi'(Q) = min(phi(Q), 1).
#pragma unroll
        for (int k0 = 0; k0 < kC; k0 += KS) {
            if (k0 / 16 <= tt) {
                const typename M::frag yd = M::acc_op(accGV, k0);
                auto step = [&](auto san) {
#pragma unroll
                    for (int m = 0; m < DT; ++m) {
                        typename M::frag ef = M::ld_tr_acc(tE, k0, 16 * m, lane);
                        if constexpr (decltype(san)::value) ef = finite_or_zero(ef);
                        accQ[m] = M::mma(ef, yd, accQ[m]);
                    }
                };
                if (ebad && (k0 + KS - 1) / 16 >= tt)  // the k-step reaching the diagonal tile
                    step(std::true_type{});
                else
                    step(std::false_type{});
            }
        }
        {
            const float bracket = FM::kSplit ? rowdA + gp + gt * n : 0.f;
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
        }
        }  // kMode != 1
        __syncthreads();  // all rows of phi(Q), G and g are staged; S_E^T, z_E, P are no longer read

        // (7) State S_E += E^T V, z_E, P; segment aggregates R += phi(Q)^T G, r += phi(Q)^T g.
        state_update<T, D, true, true>(stS, vz, vp, tE, tV, nullptr, nullptr, lane, w);
        if constexpr (kFormsRecord) state_update<T, D, true, false>(stR, vr, vr, tQ, tG, s_g, nullptr, lane, w);
        n += (float)min(kC, N - c0);
    }
    // The record's last vector is unused (w = sum over a of R is formed from R where it is used).
    if constexpr (!kFormsRecord) {
    } else if constexpr (kCoherentRecord) {
        const GBuf brr(rrec + (int64_t)bh * nseg * Rec<D>::kSize, (uint32_t)(nseg * Rec<D>::kSize * 4));
        store_record_coherent<D>(brr, (int64_t)seg * Rec<D>::kSize, stR, vr, nullptr, lane, w);
    } else {
        float* rr = rrec + ((int64_t)bh * nseg + seg) * Rec<D>::kSize;
        store_state<D>(rr, stR, lane, w);
        store_vec<D>(rr + Rec<D>::kZ, vr, lane, w);
        if (tid < D) rr[Rec<D>::kP + tid] = 0.f;
    }
}

template <typename T, int D, bool kState = false, class FM = FeatElu, int kMode = 0>
__global__ __launch_bounds__(kBlock, LA_HEAVY_WAVES_PER_SIMD) void bwd_prefix_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    T* __restrict__ dq, float2* __restrict__ rowstat, float* __restrict__ rrec, const float* __restrict__ rec, int N,
    int cps, int nseg, int BH, int prefixed, const float* __restrict__ init, const float* __restrict__ init_n, int Gv,
    const float* __restrict__ den_in) {
    __shared__ __attribute__((aligned(16))) char lds[BwdPrefixLds<T, D>::kBytes];
    // Later segments sum more records: they are dispatched first, since a CU's
    // older workgroup issues ahead of its younger one.
    const int seg = nseg - 1 - (int)(blockIdx.x / BH), bh = blockIdx.x % BH;
    bwd_prefix_body<T, D, false, BwdPrefixForms<D>::kRecord, kState, FM, kMode>(
        q, k, v, dout, dq, rowstat, rrec, rec, N, cps, nseg, prefixed, seg, bh, lds, init, init_n, Gv, den_in);
}

// ---------------------------------------------------------------------------------------
// rseg: per (segment, head) the suffix-state aggregates R = sum phi(Q) G^T and
// r = sum g phi(Q) of the segment's tokens, with G = round(dO / den) and g from
// the per-row statistics the prefix sweep saved: the same operands, chunk order
// and products as the prefix sweep's own update, so the record is bitwise the
// same.  Used where the prefix sweep does not form the record (d = 128).
template <typename T, int D, class FM = FeatElu>
__global__ __launch_bounds__(kBlock, 2) void rseg_kernel(const T* __restrict__ q, const T* __restrict__ dout,
                                                      const float2* __restrict__ rowstat, float* __restrict__ rrec,
                                                      int N, int cps, int nseg, int BH, int Gv) {
    using CR = ChunkRegs<T, D>;
    __shared__ __attribute__((aligned(16))) T sm_q[2][kC * D];
    __shared__ __attribute__((aligned(16))) T sm_g[2][kC * D];
    __shared__ __attribute__((aligned(16))) float s_g[2][kC];
    const int seg = blockIdx.x / BH, bh = blockIdx.x % BH;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int64_t hoff = (int64_t)bh * N * D, voff = (int64_t)(bh / Gv) * N * D;
    const uint32_t hbytes = (uint32_t)N * D * sizeof(T);
    const GBuf bq(q + hoff, hbytes), bdo(dout + voff, hbytes), brs(rowstat + (int64_t)bh * N, (uint32_t)N * 8);
    const int tok_begin = seg * cps * kC;
    const int tok_end = min(N, tok_begin + cps * kC);

    StateAcc<D> stR;
    VecAcc<D> vr;
    zero_state<D>(stR);
    zero_vec<D>(vr);
    CR cq, cdo;
    float dn[CR::NV];
    float gv = 0.f;
    auto load_chunk = [&](int c) {
        cq.load(bq, c, tid);
        cdo.load(bdo, c, tid);
#pragma unroll
        for (int i = 0; i < CR::NV; ++i) dn[i] = brs.ld4f((uint32_t)(c + CR::row(i, tid)) * 8);
        gv = brs.ld4f((uint32_t)(c + (tid & (kC - 1))) * 8 + 4);
    };
    load_chunk(tok_begin);
    int buf = 0;
    for (int c0 = tok_begin; c0 < tok_end; c0 += kC, buf ^= 1) {
        const Tile<T, kC, D> tQ{sm_q[buf]}, tG{sm_g[buf]};
        stage_phi<T, D, false, FM>(cq, tQ, tid);
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
        if (tid < kC) s_g[buf][tid] = gv;
        load_chunk(c0 + kC < tok_end ? c0 + kC : N);  // past the segment: zeros, no memory traffic
        __syncthreads();
        state_update<T, D, true, false>(stR, vr, vr, tQ, tG, s_g[buf], nullptr, lane, w);
    }
    float* rr = rrec + ((int64_t)bh * nseg + seg) * Rec<D>::kSize;
    store_state<D>(rr, stR, lane, w);
    store_vec<D>(rr + Rec<D>::kZ, vr, lane, w);
    if (tid < D) rr[Rec<D>::kP + tid] = 0.f;
}

// ---------------------------------------------------------------------------------------
// bwd_suffix.  Wavefront w owns key tile st = (w + it) mod 4 of the it-th chunk
// it visits (the causal mask leaves 4 - st token tiles; the rotation spreads
// that work evenly over the SIMDs); its K and V rows stay in registers in accumulator order (E(K) and
// phi'(K) share one exp), while phi(Q), G and the rounded R^T are staged in LDS
// (double-buffered, one barrier per chunk).  A and dA for the wave's keys stay
// in the accumulators that form them and feed the dV and dK products directly;
// w = sum_a R[a][b] comes from the same R^T operands against a ones operand.
// kCoherentRecords: the (R, r) records of the later segments are read with
// agent-coherent loads (written by other workgroups of the same launch), each batch
// of them once records_ready(s0, s1) has confirmed segments s0 .. s1-1 (false: they
// could not be confirmed, and the results are made NaN).
// rinit (nullable): per head, a record [dS_N^T | dz_N | 0] of upstream gradients of
// the final state, which every suffix sum starts from.  dS0, dz0 (nullable): the
// first segment writes the suffix state at the first token there, the gradient of
// the start state (S [a][b], z [a] layouts).
template <typename T, int D, bool kCoherentRecords, bool kState = false, class FM = FeatElu, class Wait>
__device__ __forceinline__ void bwd_suffix_body(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    T* __restrict__ dk, T* __restrict__ dv, const float2* __restrict__ rowstat, const float* __restrict__ rrec, int N,
    int cps, int nseg, int prefixed, int seg, int bh, Wait&& records_ready, char* lds, const float* __restrict__ rinit,
    float* __restrict__ dS0, float* __restrict__ dz0, int Gv = 1) {
    using M = Mma<T>;
    using CR = ChunkRegs<T, D>;
    constexpr int KS = M::KSTEP;
    constexpr int DT = D / 16;
    constexpr int NY = D / 4;
    using L = BwdSuffixLds<T, D>;
    T(*const sm_q)[kC * D] = reinterpret_cast<T(*)[kC * D]>(lds + L::oQ);
    T(*const sm_g)[kC * D] = reinterpret_cast<T(*)[kC * D]>(lds + L::oG);
    T(*const sm_rt)[D * D] = reinterpret_cast<T(*)[D * D]>(lds + L::oRt);
    float(*const s_g)[kC] = reinterpret_cast<float(*)[kC]>(lds + L::oGv);
    float(*const s_r)[D] = reinterpret_cast<float(*)[D]>(lds + L::oR);

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 4;
    const int64_t hoff = (int64_t)bh * N * D, voff = (int64_t)(bh / Gv) * N * D;
    const uint32_t hbytes = (uint32_t)N * D * sizeof(T);
    const GBuf bq(q + hoff, hbytes), bk(k + hoff, hbytes), bv(v + voff, hbytes), bdo(dout + voff, hbytes);
    const GBuf bdk(dk + hoff, hbytes), bdv(dv + hoff, hbytes), brs(rowstat + (int64_t)bh * N, (uint32_t)N * 8);
    const int tok_begin = seg * cps * kC;
    const int tok_end = min(N, tok_begin + cps * kC);
    const int nch = (tok_end - tok_begin + kC - 1) / kC;

    CR cq, cdo;
    RowAcc<T, D> kr, vrow;
    float dn[CR::NV];
    float gv = 0.f;
    auto load_chunk = [&](int c, int st) {
        cq.load(bq, c, tid);
        cdo.load(bdo, c, tid);
        kr.load(bk, c < N ? c + 16 * st : N, lane);
        vrow.load(bv, c < N ? c + 16 * st : N, lane);
        // den of the rows this thread stages, g of token tid (rows past the head read as 0)
#pragma unroll
        for (int i = 0; i < CR::NV; ++i) dn[i] = brs.ld4f((uint32_t)(c + CR::row(i, tid)) * 8);
        gv = brs.ld4f((uint32_t)(c + (tid & (kC - 1))) * 8 + 4);
    };
    // The first chunk's loads are in flight while the later segments' records are
    // awaited and read.
    load_chunk(tok_begin + (nch - 1) * kC, w);
    constexpr int kRecRegs = 192 - (int)((2 * sizeof(CR) + 2 * sizeof(RowAcc<T, D>)) / 4) - 8;

    // Suffix state (R, r): the records of the segments after this one, last segment first.
    StateAcc<D> stR;
    VecAcc<D> vr, vunused;
    const float* ri = kState && rinit != nullptr ? rinit + (int64_t)bh * Rec<D>::kSize : nullptr;
    if constexpr (kCoherentRecords) {
        const GBuf brr(rrec + (int64_t)bh * nseg * Rec<D>::kSize, (uint32_t)(nseg * Rec<D>::kSize * 4));
        if (ri != nullptr) {
            load_state<D>(ri, stR, lane, w);
            load_vec<D>(ri + Rec<D>::kZ, vr, lane, w);
        } else {
            zero_state<D>(stR);
            zero_vec<D>(vr);
        }
        zero_vec<D>(vunused);
        // Record j is segment nseg-1-j: the last segments' records (their workgroups
        // were dispatched first) are summed while the nearer ones are still on their way.
        bool poison = false;
        add_records_from<D, kRecRegs>(RecCoherent{brr}, (int64_t)(nseg - 1) * Rec<D>::kSize,
                                      -(int64_t)Rec<D>::kSize, nseg - 1 - seg, stR, vr, vunused, lane, w,
                                      [&](int j0, int j1) { poison = !records_ready(nseg - j1, nseg - j0) || poison; });
        if (poison) {
            using ST = StateTiles<D>;
            const float nan = __builtin_nanf("");
#pragma unroll
            for (int ia = 0; ia < ST::NAT; ++ia)
#pragma unroll
                for (int ib = 0; ib < ST::NBT; ++ib) stR[ia][ib] = splat4(nan);
        }
    } else {
        carried_state<D, kRecRegs>(rrec + ((int64_t)bh * nseg + nseg - 1) * Rec<D>::kSize, -(int64_t)Rec<D>::kSize,
                                   nseg - 1 - seg, prefixed != 0, stR, vr, vunused, lane, w, ri);
    }

    int buf = 0;
    for (int ci = nch - 1, it = 0; ci >= 0; --ci, ++it, buf ^= 1) {
        const int c0 = tok_begin + ci * kC;
        const int st = (w + it) & 3;
        const int sl = 16 * st + (lane & 15);  // this lane's key
        const Tile<T, kC, D> tQ{sm_q[buf]}, tG{sm_g[buf]};
        // R^T is read as accumulator-order operands (ld_acc) and transposed: bf16 tiles
        // keep those operands' columns together.
        const Tile<T, D, D, std::is_same<T, bf16>::value> tRt{sm_rt[buf]};
        publish_state<T, D>(stR, tRt, lane, w);
        store_vec<D>(s_r[buf], vr, lane, w);
        stage_phi<T, D, false, FM>(cq, tQ, tid);
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
        if (tid < kC) s_g[buf][tid] = gv;
        // This wave's keys: E(K) and phi'(K) from one exp; V stays raw.
        // E(K) rounded once to the operand type (bf16: kept packed as the MFMA operands).
        T ke[NY];
        float dphik[NY];
#pragma unroll
        for (int i = 0; i < NY; ++i) {
            const float x = kr.get(i);
            if constexpr (FM::kSplit) {
                const float c = expn_f(x);  // NaN for NaN, so phi'(K) carries it into dK
                ke[i] = from_f32<T>(__builtin_elementwise_maximum(x, c - 1.f));
                dphik[i] = c;
            } else {
                ke[i] = from_f32<T>(FM::e(x));
                dphik[i] = 1.f;
            }
        }
        // Operand of k-step k0 from ke (value k0 / 4 + e at position e, the order of vals_op).
        auto ke_op = [&](int k0) {
            if constexpr (sizeof(T) == 2) {
                return *reinterpret_cast<const typename M::frag*>(&ke[k0 / 4]);
            } else {
                return M::vals_op(reinterpret_cast<const float*>(ke), k0);
            }
        };
        const RowAcc<T, D> vcur = vrow;
        load_chunk(ci > 0 ? c0 - kC : N, (w + it + 1) & 3);  // past the head: zeros, no memory traffic
        const int tok = c0 + sl;
        __syncthreads();
        // Rows t of the k-steps that reach the diagonal key tile mix masked (t < s)
        // and live weights in the dK and dV products.  If one of them holds an inf or
        // NaN (phi(Q_t) or G_t, then g_t too: den_t or G_t . num_t is not finite), those
        // products take phi(Q) and G with non-finite entries replaced by 0 (0 * inf =
        // NaN would reach later keys), and the live weights of such rows carry the NaN
        // back: dA through g_t, A as A_ts + 0 g_t.
        constexpr int KSPAN = KS >= 16 ? 2 * 16 : 16;  // rows of the k-steps that reach tile st
        const int r0 = KS >= 16 ? 32 * (st >> 1) : 16 * st;
        const bool rbad = __builtin_amdgcn_ballot_w64(!finite_f(s_g[buf][r0 + (lane & (KSPAN - 1))])) != 0;

        // (1) dA_ts = G_t.V_s + g_t and A_ts = q_sum_t + phi(Q_t).E(K_s) for s <= t
        //     (accumulators [t][s], all four token tiles, branch free).
        f32x4 dA[4], A[4];
        {
            const typename M::frag one = M::ones();
            typename M::frag yv[D / KS], ye[D / KS];
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += KS) {
                yv[k0 / KS] = M::raw_op(vcur.r, k0);
                ye[k0 / KS] = ke_op(k0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dA[i] = zero4();
                A[i] = zero4();
                if (i >= st) {
                    f32x4 acc_d = zero4(), acc_b = zero4(), acc_q = zero4();
#pragma unroll
                    for (int k0 = 0; k0 < D; k0 += KS) {
                        const typename M::frag xq = M::ld_acc(tQ, 16 * i, k0, lane);
                        acc_d = M::mma(M::ld_acc(tG, 16 * i, k0, lane), yv[k0 / KS], acc_d);
                        acc_b = M::mma(xq, ye[k0 / KS], acc_b);
                        if constexpr (FM::kSplit) acc_q = M::mma(xq, one, acc_q);
                    }
                    const f32x4 gt4 = lds4(&s_g[buf][16 * i + 4 * g]);
                    // A_ts + 0 g_t: bitwise A_ts, or NaN where g_t is not finite.
                    if (i > st) {
                        dA[i] = acc_d + gt4;
#pragma unroll
                        for (int e = 0; e < 4; ++e) A[i][e] = __builtin_fmaf(gt4[e], 0.f, acc_b[e]) + acc_q[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const bool live = (lane & 15) <= 4 * g + e;
                            dA[i][e] = live ? acc_d[e] + gt4[e] : 0.f;
                            A[i][e] = live ? __builtin_fmaf(gt4[e], 0.f, acc_b[e]) + acc_q[e] : 0.f;
                        }
                    }
                }
            }
        }

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
            if ((k0 + KS - 1) / 16 >= st) {
                const typename M::frag yd = M::acc_op(dA, k0);
                const typename M::frag ya = M::acc_op(A, k0);
                auto step = [&](auto san) {
#pragma unroll
                    for (int m = 0; m < DT; ++m) {
                        typename M::frag qf = M::ld_tr_acc(tQ, k0, 16 * m, lane);
                        typename M::frag gf = M::ld_tr_acc(tG, k0, 16 * m, lane);
                        if constexpr (decltype(san)::value) {
                            qf = finite_or_zero(qf);
                            gf = finite_or_zero(gf);
                        }
                        acck[m] = M::mma(qf, yd, acck[m]);
                        accv[m] = M::mma(gf, ya, accv[m]);
                    }
                };
                if (rbad && k0 / 16 <= st)
                    step(std::true_type{});
                else
                    step(std::false_type{});
            }
        }
        {
            const typename M::frag one = M::ones();
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += KS) {
                const typename M::frag yv = M::raw_op(vcur.r, k0);
                const typename M::frag ye = ke_op(k0);
#pragma unroll
                for (int m = 0; m < DT; ++m) {
                    const typename M::frag xr = M::ld_acc(tRt, 16 * m, k0, lane);
                    acck[m] = M::mma(M::ld_tr_acc(tRt, k0, 16 * m, lane), yv, acck[m]);
                    accv[m] = M::mma(xr, ye, accv[m]);
                    if constexpr (FM::kSplit) accv[m] = M::mma(xr, one, accv[m]);  // w = sum_a R[a][.]
                }
            }
        }
#pragma unroll
        for (int m = 0; m < DT; ++m) {
            const int f0 = 16 * m + 4 * g;
            const f32x4 rv = lds4(&s_r[buf][f0]);
            f32x4 xk;
#pragma unroll
            for (int e = 0; e < 4; ++e) xk[e] = (acck[m][e] + rv[e]) * dphik[4 * m + e];
            gstore4<T>(bdk, (uint32_t)(tok * D + f0), xk);
            gstore4<T>(bdv, (uint32_t)(tok * D + f0), accv[m]);
        }

        // (3) Suffix state: R += phi(Q)^T G, r += phi(Q)^T g.
        state_update<T, D, true, false>(stR, vr, vr, tQ, tG, s_g[buf], nullptr, lane, w);
    }
    if (kState && seg == 0 && dS0 != nullptr) {  // R at the first token: the start state's gradient
        using ST = StateTiles<D>;
        float* o = dS0 + (int64_t)bh * D * D;
#pragma unroll
        for (int ia = 0; ia < ST::NAT; ++ia)
#pragma unroll
            for (int ib = 0; ib < ST::NBT; ++ib)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[(int64_t)((ST::at0(w) + ia) * 16 + 4 * g + e) * D + (ST::bt0(w) + ib) * 16 + (lane & 15)] =
                        stR[ia][ib][e];
    }
    if (kState && seg == 0 && dz0 != nullptr && StateTiles<D>::owns_vec(w) && (lane & 15) == 0) {
#pragma unroll
        for (int x = 0; x < StateTiles<D>::NVT; ++x)
#pragma unroll
            for (int e = 0; e < 4; ++e) dz0[(int64_t)bh * D + (StateTiles<D>::vt0(w) + x) * 16 + 4 * g + e] = vr[x][e];
    }
}

template <typename T, int D, bool kState = false, class FM = FeatElu>
__global__ __launch_bounds__(kBlock, LA_HEAVY_WAVES_PER_SIMD) void bwd_suffix_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    T* __restrict__ dk, T* __restrict__ dv, const float2* __restrict__ rowstat, const float* __restrict__ rrec, int N,
    int cps, int nseg, int BH, int prefixed, const float* __restrict__ rinit, float* __restrict__ dS0,
    float* __restrict__ dz0, int Gv) {
    __shared__ __attribute__((aligned(16))) char lds[BwdSuffixLds<T, D>::kBytes];
    const int seg = blockIdx.x / BH, bh = blockIdx.x % BH;
    bwd_suffix_body<T, D, false, kState, FM>(q, k, v, dout, dk, dv, rowstat, rrec, N, cps, nseg, prefixed, seg, bh,
                                             [] { return true; }, lds, rinit, dS0, dz0, Gv);
}

// ---------------------------------------------------------------------------------------
// bwd_fused: both sweeps of one (segment, head) in one workgroup, for plans whose
// consumers sum the segment records themselves.  After the prefix sweep the
// workgroup publishes its (R, r) record (agent-coherent stores, then its flag)
// and waits for the flags of the later segments of its head, whose workgroups
// were dispatched before it (segments run last to first); then the suffix sweep
// starts from their records.  The suffix sweep's cold start (records, first
// chunk) overlaps other workgroups' prefix sweeps instead of following a kernel
// boundary.  den and g per row stay with the workgroup that wrote them.
template <typename T, int D, bool kState = false, class FM = FeatElu>
__global__ __launch_bounds__(kBlock, LA_HEAVY_WAVES_PER_SIMD) void bwd_fused_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv, float2* __restrict__ rowstat,
    float* __restrict__ rrec, const float* __restrict__ rec, unsigned long long* __restrict__ flags,
    unsigned* __restrict__ giveups, unsigned long long epoch, int wait_limit, int N, int cps, int nseg, int BH,
    const float* __restrict__ init,
    const float* __restrict__ init_n, const float* __restrict__ rinit, float* __restrict__ dS0,
    float* __restrict__ dz0) {
    constexpr size_t kP = BwdPrefixLds<T, D>::kBytes, kS = BwdSuffixLds<T, D>::kBytes;
    __shared__ __attribute__((aligned(16))) char lds[kP > kS ? kP : kS];
    const int seg = nseg - 1 - (int)(blockIdx.x / BH), bh = blockIdx.x % BH;
    if (threadIdx.x == 0) giveups[(int64_t)bh * nseg + seg] = 0u;  // ordered before any wave's give-up by the barriers below
    bwd_prefix_body<T, D, true, true, kState, FM>(q, k, v, dout, dq, rowstat, rrec, rec, N, cps, nseg, 0, seg, bh, lds,
                                                  init, init_n);
    // Every wave's record stores (and den, g rows) are complete before the flag.
    wait_all_memory();
    __syncthreads();
    unsigned long long* hf = flags + (int64_t)bh * nseg;
    if (threadIdx.x == 0) post_flag(&hf[seg], epoch);
    // Each wave confirms the flags of the records it is about to read (segments s0 .. s1-1).
    bool all_ok = true;
    auto records_ready = [&](int s0, int s1) {
        bool ok = true;
        if ((threadIdx.x & 63) == 0)
            for (int j = s0; j < s1; ++j) ok = ok && await_flag(&hf[j], epoch, wait_limit);
        ok = __builtin_amdgcn_readfirstlane((int)ok) != 0;
        all_ok = all_ok && ok;
        return ok;
    };
    // The first half of the segments (dispatched last, so usually the younger of the
    // two workgroups on a CU, the one the SIMDs serve second) sum the most records
    // and start their suffix sweeps last: they take the higher wave priority for it.
    if (2 * seg < nseg) __builtin_amdgcn_s_setprio(1);
    bwd_suffix_body<T, D, true, kState, FM>(q, k, v, dout, dk, dv, rowstat, rrec, N, cps, nseg, 0, seg, bh,
                                            records_ready, lds, rinit, dS0, dz0);
    // The host reads these counts back (la_wait_failures): a give-up leaves NaN rows
    // that must not pass for a result of the data.  Thread 0 cleared the count before
    // the prefix sweep; any wave that gave up sets it.
    if ((threadIdx.x & 63) == 0 && !all_ok) atomicOr(&giveups[(int64_t)bh * nseg + seg], 1u);
}

// ---------------------------------------------------------------------------------------
hipError_t launch_bwd_prefix(int dt, int d, const void* q, const void* k, const void* v, const void* dout, void* dq,
                             float* rowstat, float* rrec, const float* rec, int64_t BH, int64_t N, SegPlan p,
                             hipStream_t s, const float* init, const float* init_n, int feat, int mode, int Gv,
                             const float* den_in) {
    const dim3 grid((unsigned)(p.nseg * BH));
#define LA_BWDP_GIVEN(TT, DD, MODE)                                                                               \
    hipLaunchKernelGGL((bwd_prefix_kernel<TT, DD, false, FeatGiven, MODE>), grid, dim3(kBlock), 0, s, (const TT*)q, \
                       (const TT*)k, (const TT*)v, (const TT*)dout, (TT*)dq, (float2*)rowstat, rrec, rec, (int)N,     \
                       p.cps, p.nseg, (int)BH, (int)p.scan, nullptr, nullptr, Gv, den_in)
#define LA_BWDP(TT, DD)                                                                                           \
    if (feat == kFeatGiven && mode == 1)                                                                          \
        LA_BWDP_GIVEN(TT, DD, 1);                                                                                 \
    else if (feat == kFeatGiven && mode == 2)                                                                     \
        LA_BWDP_GIVEN(TT, DD, 2);                                                                                 \
    else if (feat == kFeatGiven)                                                                                  \
        LA_BWDP_GIVEN(TT, DD, 0);                                                                                 \
    else if (init != nullptr || init_n != nullptr)                                                                \
        hipLaunchKernelGGL((bwd_prefix_kernel<TT, DD, true>), grid, dim3(kBlock), 0, s, (const TT*)q, (const TT*)k, \
                           (const TT*)v, (const TT*)dout, (TT*)dq, (float2*)rowstat, rrec, rec, (int)N, p.cps, p.nseg, \
                           (int)BH, (int)p.scan, init, init_n, 1, nullptr);                                          \
    else                                                                                                         \
        hipLaunchKernelGGL((bwd_prefix_kernel<TT, DD>), grid, dim3(kBlock), 0, s, (const TT*)q, (const TT*)k,    \
                           (const TT*)v, (const TT*)dout, (TT*)dq, (float2*)rowstat, rrec, rec, (int)N, p.cps, p.nseg, \
                           (int)BH, (int)p.scan, nullptr, nullptr, 1, nullptr)
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
#undef LA_BWDP_GIVEN
    return hipGetLastError();
}

hipError_t launch_rseg(int dt, int d, const void* q, const void* dout, const float* rowstat, float* rrec, int64_t BH,
                       int64_t N, SegPlan p, hipStream_t s, int feat, int Gv) {
    const dim3 grid((unsigned)(p.nseg * BH));
#define LA_RSEG(TT, DD)                                                                                           \
    if (feat == kFeatGiven)                                                                                       \
        hipLaunchKernelGGL((rseg_kernel<TT, DD, FeatGiven>), grid, dim3(kBlock), 0, s, (const TT*)q,             \
                           (const TT*)dout, (const float2*)rowstat, rrec, (int)N, p.cps, p.nseg, (int)BH, Gv);      \
    else                                                                                                         \
        hipLaunchKernelGGL((rseg_kernel<TT, DD>), grid, dim3(kBlock), 0, s, (const TT*)q, (const TT*)dout,       \
                           (const float2*)rowstat, rrec, (int)N, p.cps, p.nseg, (int)BH, Gv)
    if (dt == kBF16) {
        switch (d) {
            case 32: LA_RSEG(bf16, 32); break;
            case 64: LA_RSEG(bf16, 64); break;
            case 128: LA_RSEG(bf16, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (d) {
            case 32: LA_RSEG(float, 32); break;
            case 64: LA_RSEG(float, 64); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef LA_RSEG
    return hipGetLastError();
}

hipError_t launch_bwd_fused(int dt, int d, const void* q, const void* k, const void* v, const void* dout, void* dq,
                            void* dk, void* dv, float* rowstat, float* rrec, const float* rec, unsigned long long* flags,
                            unsigned* giveups, unsigned long long epoch, int wait_limit, int64_t BH, int64_t N,
                            SegPlan p, hipStream_t s,
                            const float* init, const float* init_n, const float* rinit, float* dS0, float* dz0,
                            int feat) {
    const dim3 grid((unsigned)(p.nseg * BH));
    const bool state = init != nullptr || init_n != nullptr || rinit != nullptr || dS0 != nullptr || dz0 != nullptr;
#define LA_BWDF(TT, DD)                                                                                           \
    if (feat == kFeatGiven)                                                                                       \
        hipLaunchKernelGGL((bwd_fused_kernel<TT, DD, false, FeatGiven>), grid, dim3(kBlock), 0, s, (const TT*)q,   \
                           (const TT*)k, (const TT*)v, (const TT*)dout, (TT*)dq, (TT*)dk, (TT*)dv, (float2*)rowstat, \
                           rrec, rec, flags, giveups, epoch, wait_limit, (int)N, p.cps, p.nseg, (int)BH, nullptr, nullptr, \
                           nullptr, nullptr, nullptr);                                                              \
    else if (state)                                                                                              \
        hipLaunchKernelGGL((bwd_fused_kernel<TT, DD, true>), grid, dim3(kBlock), 0, s, (const TT*)q, (const TT*)k, \
                           (const TT*)v, (const TT*)dout, (TT*)dq, (TT*)dk, (TT*)dv, (float2*)rowstat, rrec, rec,  \
                           flags, giveups, epoch, wait_limit, (int)N, p.cps, p.nseg, (int)BH, init, init_n, rinit, dS0, \
                           dz0);                                                                                     \
    else                                                                                                         \
        hipLaunchKernelGGL((bwd_fused_kernel<TT, DD>), grid, dim3(kBlock), 0, s, (const TT*)q, (const TT*)k,     \
                           (const TT*)v, (const TT*)dout, (TT*)dq, (TT*)dk, (TT*)dv, (float2*)rowstat, rrec, rec,  \
                           flags, giveups, epoch, wait_limit, (int)N, p.cps, p.nseg, (int)BH, nullptr, nullptr, nullptr, \
                           nullptr, nullptr)
    if (dt == kBF16) {
        switch (d) {
            case 32: LA_BWDF(bf16, 32); break;
            case 64: LA_BWDF(bf16, 64); break;
            case 128: LA_BWDF(bf16, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (d) {
            case 32: LA_BWDF(float, 32); break;
            case 64: LA_BWDF(float, 64); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef LA_BWDF
    return hipGetLastError();
}

hipError_t launch_bwd_suffix(int dt, int d, const void* q, const void* k, const void* v, const void* dout, void* dk,
                             void* dv, const float* rowstat, const float* rrec, int64_t BH, int64_t N, SegPlan p,
                             hipStream_t s, const float* rinit, float* dS0, float* dz0, int feat, int Gv) {
    const dim3 grid((unsigned)(p.nseg * BH));
#define LA_BWDS(TT, DD)                                                                                           \
    if (feat == kFeatGiven)                                                                                       \
        hipLaunchKernelGGL((bwd_suffix_kernel<TT, DD, false, FeatGiven>), grid, dim3(kBlock), 0, s, (const TT*)q,  \
                           (const TT*)k, (const TT*)v, (const TT*)dout, (TT*)dk, (TT*)dv, (const float2*)rowstat,   \
                           rrec, (int)N, p.cps, p.nseg, (int)BH, (int)p.scan, nullptr, nullptr, nullptr, Gv);       \
    else if (rinit != nullptr || dS0 != nullptr || dz0 != nullptr)                                                \
        hipLaunchKernelGGL((bwd_suffix_kernel<TT, DD, true>), grid, dim3(kBlock), 0, s, (const TT*)q, (const TT*)k, \
                           (const TT*)v, (const TT*)dout, (TT*)dk, (TT*)dv, (const float2*)rowstat, rrec, (int)N,  \
                           p.cps, p.nseg, (int)BH, (int)p.scan, rinit, dS0, dz0, 1);                                 \
    else                                                                                                         \
        hipLaunchKernelGGL((bwd_suffix_kernel<TT, DD>), grid, dim3(kBlock), 0, s, (const TT*)q, (const TT*)k,    \
                           (const TT*)v, (const TT*)dout, (TT*)dk, (TT*)dv, (const float2*)rowstat, rrec, (int)N,  \
                           p.cps, p.nseg, (int)BH, (int)p.scan, nullptr, nullptr, nullptr, 1)
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
