// fwd.hip -- forward kernels of kernelized linear attention for gfx950.
//
// Method (page "Efficient Transformers Survey", section "Linear Attention",
// Proposition "Linear Attention via Kernel Decomposition"):
//   O_i = phi(Q_i)^T S / phi(Q_i)^T z,  S = sum_j phi(K_j) V_j^T,  z = sum_j phi(K_j),
// with phi = elu + 1 applied elementwise.  The causal form sums over j <= i.
//
// Chunked evaluation.  The associativity of the Intuition paragraph,
// (phi(Q) phi(K)^T) V = phi(Q) (phi(K)^T V), applied blockwise, splits a causal
// row into an in-chunk part (a masked 64 x 64 product) and a carried state.
// The state is kept split around the constant 1 in phi(K) = 1 + E(K):
//   S = 1 P^T + S_E,  z = n 1 + z_E,
// so with q_sum_t = sum_a phi(Q_ta) and A_ts = q_sum_t + phi(Q_t).E(K_s):
//   num_t = q_sum_t P + phi(Q_t) S_E + sum_{s<=t in chunk} A_ts V_s,
//   den_t = q_sum_t n + phi(Q_t) . z_E + sum_{s<=t in chunk} A_ts.
//
// Work decomposition.  One workgroup (4 wavefronts) per (head, segment of
// `cps` chunks).  seg_state reduces each segment's keys to (S_E, z_E, P);
// scan turns those into exclusive prefixes in segment order (fixed order, so
// results are bitwise reproducible) and per-head totals; causal_fwd walks a
// segment's chunks from its prefix.  The non-causal forward is seg_state +
// scan (totals) + noncausal_fwd.
//
// Data layout.  Inputs/outputs [BH][N][d] row-major in HBM.  Per chunk the
// workgroup stages phi(Q), E(K) and V row-major in LDS (bf16 for bf16 inputs,
// fp32 for fp32 inputs); products that contract over tokens read them with the
// transposing LDS load.  The in-chunk weights A and the rounded S_E^T live in
// LDS, S_E itself stays in fp32 MFMA accumulators across chunks; z_E and P are
// accumulated by MFMA against a ones operand.  Segment records are fp32
// [S_E^T | z_E | P].
#include "chunk.h"

namespace la {

// ---------------------------------------------------------------------------------------
// seg_state: per (segment, head) the aggregates (S_E, z_E, P) of the segment's keys.
template <typename T, int D>
__global__ __launch_bounds__(kBlock) void seg_state_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                           float* __restrict__ rec, int N, int cps, int nseg) {
    __shared__ __attribute__((aligned(16))) T sm_e[kC * D];
    __shared__ __attribute__((aligned(16))) T sm_v[kC * D];
    const Tile<T, kC, D> tE{sm_e}, tV{sm_v};

    const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int64_t hoff = (int64_t)bh * N * D;
    const int tok_begin = seg * cps * kC;
    const int tok_end = min(N, tok_begin + cps * kC);

    StateAcc<D> st;
    VecAcc<D> vz, vp;
    zero_state<D>(st);
    zero_vec<D>(vz);
    zero_vec<D>(vp);

    ChunkRegs<T, D> ck, cv;
    ck.load(k + hoff, tok_begin, N, tid);
    cv.load(v + hoff, tok_begin, N, tid);
    for (int c0 = tok_begin; c0 < tok_end; c0 += kC) {
        stage_elu<T, D>(ck, tE, tid);
        stage_raw<T, D>(cv, tV, tid);
        if (c0 + kC < tok_end) {
            ck.load(k + hoff, c0 + kC, N, tid);
            cv.load(v + hoff, c0 + kC, N, tid);
        }
        __syncthreads();
        state_update<T, D, true, true>(st, vz, vp, tE, tV, nullptr, nullptr, lane, w);
        __syncthreads();
    }
    float* r = rec + ((int64_t)bh * nseg + seg) * Rec<D>::kSize;
    store_state<D>(r, st, lane, w);
    store_vec<D>(r + Rec<D>::kZ, vz, lane, w);
    store_vec<D>(r + Rec<D>::kP, vp, lane, w);
}

// ---------------------------------------------------------------------------------------
// scan: per head, replace each segment record by the sum of the records before
// it (in segment order), or after it (reverse order) for the backward's suffix
// records, and/or write the head total.  Records are loaded in batches ahead
// of the running sum.
template <int D>
__global__ __launch_bounds__(kBlock) void scan_kernel(float* __restrict__ rec, float* __restrict__ total, int nseg,
                                                      int write_prefix, int reverse) {
    constexpr int R4 = Rec<D>::kSize / 4;
    constexpr int NBLK = (R4 + kBlock - 1) / kBlock;
    constexpr int BATCH = 16;
    const int e4 = (blockIdx.x % NBLK) * kBlock + threadIdx.x;
    const int bh = blockIdx.x / NBLK;
    if (e4 >= R4) return;
    f32x4* r = reinterpret_cast<f32x4*>(rec) + (int64_t)bh * nseg * R4 + e4;
    f32x4 run = zero4();
    for (int i0 = 0; i0 < nseg; i0 += BATCH) {
        f32x4 x[BATCH];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const int i = i0 + b;
            const int s = reverse ? nseg - 1 - i : i;
            x[b] = i < nseg ? r[(int64_t)s * R4] : zero4();
        }
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const int i = i0 + b;
            const int s = reverse ? nseg - 1 - i : i;
            if (write_prefix && i < nseg) r[(int64_t)s * R4] = run;
            run += x[b];
        }
    }
    if (total != nullptr) reinterpret_cast<f32x4*>(total)[(int64_t)bh * R4 + e4] = run;
}

// ---------------------------------------------------------------------------------------
// causal_fwd: per (segment, head), walk the segment's chunks from its prefix state.
template <typename T, int D>
__global__ __launch_bounds__(kBlock, LA_HEAVY_WAVES_PER_SIMD) void causal_fwd_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                            const T* __restrict__ v, T* __restrict__ o,
                                                            float* __restrict__ den_out, const float* __restrict__ rec,
                                                            int N, int cps, int nseg) {
    using M = Mma<T>;
    constexpr int KS = M::KSTEP;
    constexpr int DT = D / 16;
    __shared__ __attribute__((aligned(16))) T sm_q[kC * D];
    __shared__ __attribute__((aligned(16))) T sm_e[kC * D];
    __shared__ __attribute__((aligned(16))) T sm_v[kC * D];
    __shared__ __attribute__((aligned(16))) T sm_a[kC * kC];
    __shared__ __attribute__((aligned(16))) T sm_st[D * D];
    __shared__ __attribute__((aligned(16))) float s_z[D], s_p[D];
    const Tile<T, kC, D> tQ{sm_q}, tE{sm_e}, tV{sm_v};
    const Tile<T, kC, kC> tA{sm_a};
    const Tile<T, D, D> tSt{sm_st};

    const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 4;
    const int64_t hoff = (int64_t)bh * N * D;
    const int tok_begin = seg * cps * kC;
    const int tok_end = min(N, tok_begin + cps * kC);

    // Starting state: the exclusive prefix of the segments before this one.
    const float* r = rec + ((int64_t)bh * nseg + seg) * Rec<D>::kSize;
    StateAcc<D> st;
    VecAcc<D> vz, vp;
    load_state<D>(r, st, lane, w);
    load_vec<D>(r + Rec<D>::kZ, vz, lane, w);
    load_vec<D>(r + Rec<D>::kP, vp, lane, w);
    float n = (float)tok_begin;

    ChunkRegs<T, D> cq, ck, cv;
    cq.load(q + hoff, tok_begin, N, tid);
    ck.load(k + hoff, tok_begin, N, tid);
    cv.load(v + hoff, tok_begin, N, tid);

    const int t0 = 16 * w;            // this wave's token tile
    const int tl = t0 + (lane & 15);  // this lane's token (accumulator column)

    for (int c0 = tok_begin; c0 < tok_end; c0 += kC) {
        // Publish the state reached so far and stage this chunk.
        publish_state<T, D>(st, tSt, lane, w);
        store_vec<D>(s_z, vz, lane, w);
        store_vec<D>(s_p, vp, lane, w);
        stage_phi<T, D>(cq, tQ, tid);
        stage_elu<T, D>(ck, tE, tid);
        stage_raw<T, D>(cv, tV, tid);
        if (c0 + kC < tok_end) {
            cq.load(q + hoff, c0 + kC, N, tid);
            ck.load(k + hoff, c0 + kC, N, tid);
            cv.load(v + hoff, c0 + kC, N, tid);
        }
        __syncthreads();

        // In-chunk weights A_ts = q_sum_t + phi(Q_t).E(K_s) for s <= t (accumulator [s][t]);
        // every wave forms all four key tiles so the code has no wave-dependent branches.
        float qs_t, den = 0.f;
        {
            const typename M::frag one = M::ones();
            f32x4 acc_a[4], acc_q = zero4();
#pragma unroll
            for (int j = 0; j < 4; ++j) acc_a[j] = zero4();
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += KS) {
                const typename M::frag yf = M::ld(tQ, t0, k0, lane);
                acc_q = M::mma(one, yf, acc_q);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc_a[j] = M::mma(M::ld(tE, 16 * j, k0, lane), yf, acc_a[j]);
            }
            qs_t = acc_q[0];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a = (16 * j + 4 * g + e) <= tl ? qs_t + acc_a[j][e] : 0.f;
                    acc_a[j][e] = a;
                    den += a;
                }
                store_T(tA, 16 * j, t0, acc_a[j], lane);
            }
        }
        den = sum_over_groups(den) + n * qs_t + row_dot_quarters<T, D>(tQ, s_z, tl, lane);
        const float inv = rcp_f(den);
        wave_lds_sync();  // this wave's rows of A

        // num^T[b][t] = sum_s V[s][b] A[t][s] + sum_a S_E^T[b][a] phi(Q)[t][a]
        f32x4 acc[DT];
#pragma unroll
        for (int m = 0; m < DT; ++m) acc[m] = zero4();
#pragma unroll
        for (int k0 = 0; k0 < kC; k0 += KS) {
            const typename M::frag yf = M::ld(tA, t0, k0, lane);
#pragma unroll
            for (int m = 0; m < DT; ++m) acc[m] = M::mma(M::ld_tr(tV, k0, 16 * m, lane), yf, acc[m]);
        }
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += KS) {
            const typename M::frag yf = M::ld(tQ, t0, k0, lane);
#pragma unroll
            for (int m = 0; m < DT; ++m) acc[m] = M::mma(M::ld(tSt, 16 * m, k0, lane), yf, acc[m]);
        }
        const int tok = c0 + tl;
        if (tok < N) {
            T* orow = o + hoff + (int64_t)tok * D;
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                const int b0 = 16 * m + 4 * g;
                const f32x4 p4 = lds4(&s_p[b0]);
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = (acc[m][e] + qs_t * p4[e]) * inv;
                gstore4(orow + b0, x);
            }
            if (den_out != nullptr && g == 0) den_out[(int64_t)bh * N + tok] = den;
        }

        // State update: S_E += E(K)^T V, z_E += colsum E(K), P += colsum V.
        state_update<T, D, true, true>(st, vz, vp, tE, tV, nullptr, nullptr, lane, w);
        n += (float)min(kC, N - c0);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------
// noncausal_fwd: every row reads the head's total state.
template <typename T, int D>
__global__ __launch_bounds__(kBlock) void noncausal_fwd_kernel(const T* __restrict__ q, T* __restrict__ o,
                                                               const float* __restrict__ total, int N, int cps,
                                                               int nseg) {
    using M = Mma<T>;
    constexpr int KS = M::KSTEP;
    constexpr int DT = D / 16;
    __shared__ __attribute__((aligned(16))) T sm_q[kC * D];
    __shared__ __attribute__((aligned(16))) T sm_st[D * D];
    __shared__ __attribute__((aligned(16))) float s_z[D], s_p[D];
    const Tile<T, kC, D> tQ{sm_q};
    const Tile<T, D, D> tSt{sm_st};

    const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 4;
    const int64_t hoff = (int64_t)bh * N * D;
    const int tok_begin = seg * cps * kC;
    const int tok_end = min(N, tok_begin + cps * kC);
    const float* r = total + (int64_t)bh * Rec<D>::kSize;

    {
        StateAcc<D> st;
        load_state<D>(r, st, lane, w);
        publish_state<T, D>(st, tSt, lane, w);
    }
    if (tid < D) s_z[tid] = r[Rec<D>::kZ + tid];
    else if (tid < 2 * D) s_p[tid - D] = r[Rec<D>::kP + tid - D];
    const float n = (float)N;

    ChunkRegs<T, D> cq;
    cq.load(q + hoff, tok_begin, N, tid);
    const int t0 = 16 * w;
    const int tl = t0 + (lane & 15);
    for (int c0 = tok_begin; c0 < tok_end; c0 += kC) {
        stage_phi<T, D>(cq, tQ, tid);
        if (c0 + kC < tok_end) cq.load(q + hoff, c0 + kC, N, tid);
        __syncthreads();
        const float qs_t = tile_row_sums<T, D>(tQ, t0, lane)[0];
        const float inv = rcp_f(n * qs_t + row_dot_quarters<T, D>(tQ, s_z, tl, lane));
        f32x4 acc[DT];
#pragma unroll
        for (int m = 0; m < DT; ++m) acc[m] = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += KS) {
            const typename M::frag yf = M::ld(tQ, t0, k0, lane);
#pragma unroll
            for (int m = 0; m < DT; ++m) acc[m] = M::mma(M::ld(tSt, 16 * m, k0, lane), yf, acc[m]);
        }
        const int tok = c0 + tl;
        if (tok < N) {
            T* orow = o + hoff + (int64_t)tok * D;
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                const int b0 = 16 * m + 4 * g;
                const f32x4 p4 = lds4(&s_p[b0]);
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = (acc[m][e] + qs_t * p4[e]) * inv;
                gstore4(orow + b0, x);
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------
// final_state: S[a][b] = P[b] + S_E[a][b], z[a] = N + z_E[a] from the head totals.
template <int D>
__global__ __launch_bounds__(kBlock) void final_state_kernel(const float* __restrict__ total,
                                                             float* __restrict__ S_out, float* __restrict__ z_out,
                                                             int N) {
    const int bh = blockIdx.x;
    const float* r = total + (int64_t)bh * Rec<D>::kSize;
    if (S_out != nullptr) {
        float* s = S_out + (int64_t)bh * D * D;
        for (int x = threadIdx.x; x < D * D; x += kBlock) {
            const int a = x / D, b = x % D;
            s[x] = r[Rec<D>::kP + b] + r[b * D + a];
        }
    }
    if (z_out != nullptr && threadIdx.x < D)
        z_out[(int64_t)bh * D + threadIdx.x] = (float)N + r[Rec<D>::kZ + threadIdx.x];
}

__global__ __launch_bounds__(kBlock) void fill_zero_kernel(float* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (size_t)gridDim.x * kBlock) p[i] = 0.f;
}

// ---------------------------------------------------------------------------------------
// Host launchers.
SegPlan plan_segments(int64_t BH, int64_t N) {
    const int64_t nchunk = (N + kC - 1) / kC;
    // Aim for about 1024 workgroups (4 per CU) while keeping >= 1 chunk per segment.
    int64_t cps = (BH * nchunk + 1023) / 1024;
    if (cps < 1) cps = 1;
    if (cps > 16) cps = 16;
    SegPlan p;
    p.cps = (int)cps;
    p.nseg = (int)((nchunk + cps - 1) / cps);
    if (p.nseg < 1) p.nseg = 1;
    return p;
}

#define LA_DISPATCH_D(d, ...)                 \
    switch (d) {                              \
        case 32: {                            \
            constexpr int D = 32;             \
            __VA_ARGS__;                      \
        } break;                              \
        case 64: {                            \
            constexpr int D = 64;             \
            __VA_ARGS__;                      \
        } break;                              \
        case 128: {                           \
            constexpr int D = 128;            \
            __VA_ARGS__;                      \
        } break;                              \
        default: return hipErrorInvalidValue; \
    }

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_seg_state(int dt, int d, const void* k, const void* v, float* rec, int64_t BH, int64_t N,
                            SegPlan p, hipStream_t s) {
    const dim3 grid((unsigned)(p.nseg * BH));
    if (dt == kBF16) {
        LA_DISPATCH_D(d, hipLaunchKernelGGL((seg_state_kernel<bf16, D>), grid, dim3(kBlock), 0, s, (const bf16*)k,
                                            (const bf16*)v, rec, (int)N, p.cps, p.nseg));
    } else {
        LA_DISPATCH_D(d, hipLaunchKernelGGL((seg_state_kernel<float, D>), grid, dim3(kBlock), 0, s, (const float*)k,
                                            (const float*)v, rec, (int)N, p.cps, p.nseg));
    }
    return hipGetLastError();
}

static hipError_t scan_launch(int d, float* rec, float* total, int64_t BH, int nseg, bool write_prefix, bool reverse,
                              hipStream_t s) {
    const int r4 = (int)(rec_floats(d) / 4);
    const dim3 grid((unsigned)(((r4 + kBlock - 1) / kBlock) * BH));
    LA_DISPATCH_D(d, hipLaunchKernelGGL((scan_kernel<D>), grid, dim3(kBlock), 0, s, rec, total, nseg,
                                        write_prefix ? 1 : 0, reverse ? 1 : 0));
    return hipGetLastError();
}

hipError_t launch_scan(int d, float* rec, float* total, int64_t BH, int nseg, bool write_prefix, hipStream_t s) {
    return scan_launch(d, rec, total, BH, nseg, write_prefix, false, s);
}

hipError_t launch_rscan(int d, float* rrec, int64_t BH, int nseg, hipStream_t s) {
    return scan_launch(d, rrec, nullptr, BH, nseg, true, true, s);
}

hipError_t launch_causal_fwd(int dt, int d, const void* q, const void* k, const void* v, void* o, float* den_out,
                             const float* rec, int64_t BH, int64_t N, SegPlan p, hipStream_t s) {
    const dim3 grid((unsigned)(p.nseg * BH));
    if (dt == kBF16) {
        LA_DISPATCH_D(d, hipLaunchKernelGGL((causal_fwd_kernel<bf16, D>), grid, dim3(kBlock), 0, s, (const bf16*)q,
                                            (const bf16*)k, (const bf16*)v, (bf16*)o, den_out, rec, (int)N, p.cps,
                                            p.nseg));
    } else {
        switch (d) {
            case 32:
                hipLaunchKernelGGL((causal_fwd_kernel<float, 32>), grid, dim3(kBlock), 0, s, (const float*)q,
                                   (const float*)k, (const float*)v, (float*)o, den_out, rec, (int)N, p.cps, p.nseg);
                break;
            case 64:
                hipLaunchKernelGGL((causal_fwd_kernel<float, 64>), grid, dim3(kBlock), 0, s, (const float*)q,
                                   (const float*)k, (const float*)v, (float*)o, den_out, rec, (int)N, p.cps, p.nseg);
                break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

hipError_t launch_noncausal_fwd(int dt, int d, const void* q, void* o, const float* total, int64_t BH, int64_t N,
                                SegPlan p, hipStream_t s) {
    const dim3 grid((unsigned)(p.nseg * BH));
    if (dt == kBF16) {
        LA_DISPATCH_D(d, hipLaunchKernelGGL((noncausal_fwd_kernel<bf16, D>), grid, dim3(kBlock), 0, s,
                                            (const bf16*)q, (bf16*)o, total, (int)N, p.cps, p.nseg));
    } else {
        LA_DISPATCH_D(d, hipLaunchKernelGGL((noncausal_fwd_kernel<float, D>), grid, dim3(kBlock), 0, s,
                                            (const float*)q, (float*)o, total, (int)N, p.cps, p.nseg));
    }
    return hipGetLastError();
}

hipError_t launch_final_state(int d, const float* total, float* S_out, float* z_out, int64_t BH, int64_t N,
                              hipStream_t s) {
    LA_DISPATCH_D(d, hipLaunchKernelGGL((final_state_kernel<D>), dim3((unsigned)BH), dim3(kBlock), 0, s, total, S_out,
                                        z_out, (int)N));
    return hipGetLastError();
}

}  // namespace la
