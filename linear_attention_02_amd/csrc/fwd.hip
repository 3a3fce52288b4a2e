// fwd.hip -- forward kernels of kernelized linear attention for gfx950.
//
// Method (page "Efficient Transformers Survey", section "Linear Attention",
// Proposition "Linear Attention via Kernel Decomposition"):
//   O_i = phi(Q_i)^T S / phi(Q_i)^T z,  S = sum_j phi(K_j) V_j^T,  z = sum_j phi(K_j),
// with phi = elu + 1 applied elementwise.  The causal form sums over j <= i.
//
// Chunked evaluation.  The associativity of the Intuition paragraph,
// (phi(Q) phi(K)^T) V = phi(Q) (phi(K)^T V), applied blockwise, splits a causal
// row into an in-chunk part (a masked C x C product) and a carried state.  The
// state is kept split around the constant 1 that phi(K) = 1 + E(K) carries:
//   S = 1 P^T + S_E,  P = sum_j V_j,  S_E = sum_j E(K_j) V_j^T,
//   z = n 1 + z_E,    z_E = sum_j E(K_j),  n = number of keys,
// so the MFMA operand E(K) is small and exact-ish in bf16 and the "+1" part
// stays in fp32 rank-1 terms.  With q_sum_t = sum_a phi(Q_ta):
//   num_t = q_sum_t P + phi(Q_t) S_E + sum_{s<=t in chunk} A_ts V_s
//   den_t = q_sum_t n + phi(Q_t) . z_E + sum_{s<=t in chunk} A_ts
//   A_ts  = q_sum_t + phi(Q_t) . E(K_s).
//
// Work decomposition.  One workgroup (4 wavefronts) per (head, segment); a
// segment is `cps` chunks of 64 tokens processed in order.  Three launches:
//   seg_state  : per segment, the aggregates (S_E, z_E, P) of its keys;
//   scan       : per head, exclusive prefix of the aggregates over segments
//                (fixed order, so results are bitwise reproducible) and the total;
//   causal_fwd : per segment, start from the prefix and walk the chunks.
// The non-causal forward uses seg_state + scan (total only) + noncausal_fwd.
//
// Data layout.  Inputs/outputs [BH][N][d] row-major in HBM.  Per chunk the
// workgroup stages phi(Q) and E(K) row-major and E(K)^T, V^T transposed in
// LDS (bf16 for bf16 inputs, fp32 for fp32 inputs); the in-chunk weights A and
// the bf16 copy of S_E^T also live in LDS; S_E itself stays in fp32 MFMA
// accumulators across chunks.  Segment records are fp32 [S_E^T | z_E | P].
#include "chunk.h"

namespace la {

// ---------------------------------------------------------------------------------------
// seg_state: per (segment, head) the aggregates (S_E, z_E, P) of the segment's keys.
template <typename T, int D>
__global__ __launch_bounds__(kBlock) void seg_state_kernel(const T* __restrict__ k,
                                                           const T* __restrict__ v,
                                                           float* __restrict__ rec, int N, int cps,
                                                           int nseg) {
    constexpr int C = kChunk;
    __shared__ __attribute__((aligned(16))) T sm_ekt[D * C];
    __shared__ __attribute__((aligned(16))) T sm_vt[D * C];
    const Tile<T, D, C> tEkt{sm_ekt}, tVt{sm_vt};
    const Tile<T, C, D> tNone{nullptr};

    const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t hoff = (int64_t)bh * N * D;
    const int tok_begin = seg * cps * kChunk;
    const int tok_end = min(N, tok_begin + cps * kChunk);

    StateAcc<D> st;
    zero_state<D>(st);
    float zp = 0.f;  // thread < D: z_E[tid]; D <= thread < 2D: P[tid - D]

    ChunkRegs<T, D, C> ck, cv;
    ck.load(k + hoff, tok_begin, N, tid);
    cv.load(v + hoff, tok_begin, N, tid);
    for (int c0 = tok_begin; c0 < tok_end; c0 += C) {
        stage_e<T, D, C, false, true>(ck, tNone, tEkt, tid);
        stage_raw<T, D, C, false, true>(cv, tNone, tVt, tid);
        if (c0 + C < tok_end) {
            ck.load(k + hoff, c0 + C, N, tid);
            cv.load(v + hoff, c0 + C, N, tid);
        }
        __syncthreads();
        state_mma<T, D, D, C>(st, tEkt, tVt, lane, w);
        if (tid < D) zp += row_sum(tEkt, tid);
        else if (tid < 2 * D) zp += row_sum(tVt, tid - D);
        __syncthreads();
    }
    float* r = rec + ((int64_t)bh * nseg + seg) * Rec<D>::kSize;
    store_state_acc<D>(r, st, lane, w);
    if (tid < D) r[Rec<D>::kZ + tid] = zp;
    else if (tid < 2 * D) r[Rec<D>::kP + tid - D] = zp;
}

// ---------------------------------------------------------------------------------------
// scan: per head, replace each segment record by the sum of the records before it
// (exclusive prefix, summed in segment order; or after it, in reverse order,
// for the backward's suffix records) and/or write the head total.
template <int D>
__global__ __launch_bounds__(kBlock) void scan_kernel(float* __restrict__ rec, float* __restrict__ total,
                                                      int nseg, int write_prefix, int reverse) {
    constexpr int R4 = Rec<D>::kSize / 4;
    constexpr int NBLK = (R4 + kBlock - 1) / kBlock;
    const int e4 = (blockIdx.x % NBLK) * kBlock + threadIdx.x;
    const int bh = blockIdx.x / NBLK;
    if (e4 >= R4) return;
    f32x4* r = reinterpret_cast<f32x4*>(rec) + (int64_t)bh * nseg * R4 + e4;
    f32x4 run = zero4();
    for (int i = 0; i < nseg; ++i) {
        const int s = reverse ? nseg - 1 - i : i;
        const f32x4 x = r[(int64_t)s * R4];
        if (write_prefix) r[(int64_t)s * R4] = run;
        run += x;
    }
    if (total != nullptr) reinterpret_cast<f32x4*>(total)[(int64_t)bh * R4 + e4] = run;
}

// ---------------------------------------------------------------------------------------
// causal_fwd: per (segment, head), walk the segment's chunks from its prefix state.
template <typename T, int D>
__global__ __launch_bounds__(kBlock) void causal_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ o,
    float* __restrict__ den_out, const float* __restrict__ rec, int N, int cps, int nseg) {
    using M = Mma<T>;
    constexpr int C = kChunk;
    constexpr int KS = M::KSTEP;
    constexpr int DT = D / 16;
    __shared__ __attribute__((aligned(16))) T sm_qf[C * D];
    __shared__ __attribute__((aligned(16))) T sm_ek[C * D];
    __shared__ __attribute__((aligned(16))) T sm_ekt[D * C];
    __shared__ __attribute__((aligned(16))) T sm_vt[D * C];
    __shared__ __attribute__((aligned(16))) T sm_a[C * C];
    __shared__ __attribute__((aligned(16))) T sm_st[D * D];
    __shared__ float s_qsum[C], s_z[D], s_p[D];
    const Tile<T, C, D> tQf{sm_qf}, tEk{sm_ek};
    const Tile<T, D, C> tEkt{sm_ekt}, tVt{sm_vt}, tNoneT{nullptr};
    const Tile<T, C, C> tA{sm_a};
    const Tile<T, D, D> tSt{sm_st}, tNoneS{nullptr};

    const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4;
    const int64_t hoff = (int64_t)bh * N * D;
    const int tok_begin = seg * cps * kChunk;
    const int tok_end = min(N, tok_begin + cps * kChunk);

    // Starting state: the exclusive prefix of the segments before this one.
    const float* r = rec + ((int64_t)bh * nseg + seg) * Rec<D>::kSize;
    StateAcc<D> st;
    load_state_acc<D>(r, st, lane, w);
    publish_state<T, D, true, false>(st, tSt, tNoneS, lane, w);
    float zp = 0.f;
    if (tid < D) {
        zp = r[Rec<D>::kZ + tid];
        s_z[tid] = zp;
    } else if (tid < 2 * D) {
        zp = r[Rec<D>::kP + tid - D];
        s_p[tid - D] = zp;
    }
    float n = (float)tok_begin;

    ChunkRegs<T, D, C> cq, ck, cv;
    cq.load(q + hoff, tok_begin, N, tid);
    ck.load(k + hoff, tok_begin, N, tid);
    cv.load(v + hoff, tok_begin, N, tid);

    const int t0 = 16 * w;            // this wave's token tile
    const int tl = t0 + (lane & 15);  // this lane's token (accumulator column)
    const int kend = ((16 * (w + 1) + KS - 1) / KS) * KS;

    for (int c0 = tok_begin; c0 < tok_end; c0 += C) {
        stage_q<T, D, C, false>(cq, tQf, tNoneT, s_qsum, tid);
        stage_e<T, D, C, true, true>(ck, tEk, tEkt, tid);
        stage_raw<T, D, C, false, true>(cv, tQf, tVt, tid);
        if (c0 + C < tok_end) {
            cq.load(q + hoff, c0 + C, N, tid);
            ck.load(k + hoff, c0 + C, N, tid);
            cv.load(v + hoff, c0 + C, N, tid);
        }
        __syncthreads();

        // In-chunk weights A_ts = q_sum_t + phi(Q_t).E(K_s) for s <= t, as A^T tiles.
        f32x4 acc_a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc_a[j] = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += KS) {
            const typename M::frag yf = M::load(tQf, t0, k0, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j <= w) acc_a[j] = M::mma(M::load(tEk, 16 * j, k0, lane), yf, acc_a[j]);
        }
        const float qs_t = s_qsum[tl];
        float den = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j <= w) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 16 * j + 4 * g + e;
                    const float a = s <= tl ? qs_t + acc_a[j][e] : 0.f;
                    acc_a[j][e] = a;
                    den += a;
                }
                store_T(tA, 16 * j, t0, acc_a[j], lane);
            } else if (16 * j < kend) {
                store_T(tA, 16 * j, t0, zero4(), lane);
            }
        }
        den = sum_over_groups(den) + n * qs_t + row_dot_quarters<T, D, C>(tQf, s_z, tl, lane);
        __syncthreads();

        // num^T[b][t] = sum_s V^T[b][s] A[t][s] + sum_a S_E^T[b][a] phi(Q)[t][a]
        f32x4 acc[DT];
#pragma unroll
        for (int m = 0; m < DT; ++m) acc[m] = zero4();
        for (int k0 = 0; k0 < kend; k0 += KS) {
            const typename M::frag yf = M::load(tA, t0, k0, lane);
#pragma unroll
            for (int m = 0; m < DT; ++m) acc[m] = M::mma(M::load(tVt, 16 * m, k0, lane), yf, acc[m]);
        }
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += KS) {
            const typename M::frag yf = M::load(tQf, t0, k0, lane);
#pragma unroll
            for (int m = 0; m < DT; ++m) acc[m] = M::mma(M::load(tSt, 16 * m, k0, lane), yf, acc[m]);
        }
        const int tok = c0 + tl;
        if (tok < N) {
            T* orow = o + hoff + (int64_t)tok * D;
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                const int b0 = 16 * m + 4 * g;
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = (acc[m][e] + qs_t * s_p[b0 + e]) / den;
                gstore4(orow + b0, x);
            }
            if (den_out != nullptr && g == 0) den_out[(int64_t)bh * N + tok] = den;
        }

        // State update: S_E += E(K)^T V, z_E += colsum E(K), P += colsum V.
        state_mma<T, D, D, C>(st, tEkt, tVt, lane, w);
        if (tid < D) zp += row_sum(tEkt, tid);
        else if (tid < 2 * D) zp += row_sum(tVt, tid - D);
        n += (float)min(C, N - c0);
        __syncthreads();
        publish_state<T, D, true, false>(st, tSt, tNoneS, lane, w);
        if (tid < D) s_z[tid] = zp;
        else if (tid < 2 * D) s_p[tid - D] = zp;
    }
}

// ---------------------------------------------------------------------------------------
// noncausal_fwd: every row reads the head's total state.
template <typename T, int D>
__global__ __launch_bounds__(kBlock) void noncausal_fwd_kernel(const T* __restrict__ q, T* __restrict__ o,
                                                               const float* __restrict__ total, int N,
                                                               int cps, int nseg) {
    using M = Mma<T>;
    constexpr int C = kChunk;
    constexpr int KS = M::KSTEP;
    constexpr int DT = D / 16;
    __shared__ __attribute__((aligned(16))) T sm_qf[C * D];
    __shared__ __attribute__((aligned(16))) T sm_st[D * D];
    __shared__ float s_qsum[C], s_z[D], s_p[D];
    const Tile<T, C, D> tQf{sm_qf};
    const Tile<T, D, C> tNoneT{nullptr};
    const Tile<T, D, D> tSt{sm_st}, tNoneS{nullptr};

    const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4;
    const int64_t hoff = (int64_t)bh * N * D;
    const int tok_begin = seg * cps * kChunk;
    const int tok_end = min(N, tok_begin + cps * kChunk);
    const float* r = total + (int64_t)bh * Rec<D>::kSize;

    {
        StateAcc<D> st;
        load_state_acc<D>(r, st, lane, w);
        publish_state<T, D, true, false>(st, tSt, tNoneS, lane, w);
    }
    if (tid < D) s_z[tid] = r[Rec<D>::kZ + tid];
    else if (tid < 2 * D) s_p[tid - D] = r[Rec<D>::kP + tid - D];
    const float n = (float)N;

    ChunkRegs<T, D, C> cq;
    cq.load(q + hoff, tok_begin, N, tid);
    const int t0 = 16 * w;
    const int tl = t0 + (lane & 15);
    for (int c0 = tok_begin; c0 < tok_end; c0 += C) {
        stage_q<T, D, C, false>(cq, tQf, tNoneT, s_qsum, tid);
        if (c0 + C < tok_end) cq.load(q + hoff, c0 + C, N, tid);
        __syncthreads();
        const float qs_t = s_qsum[tl];
        const float den = n * qs_t + row_dot_quarters<T, D, C>(tQf, s_z, tl, lane);
        f32x4 acc[DT];
#pragma unroll
        for (int m = 0; m < DT; ++m) acc[m] = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += KS) {
            const typename M::frag yf = M::load(tQf, t0, k0, lane);
#pragma unroll
            for (int m = 0; m < DT; ++m) acc[m] = M::mma(M::load(tSt, 16 * m, k0, lane), yf, acc[m]);
        }
        const int tok = c0 + tl;
        if (tok < N) {
            T* orow = o + hoff + (int64_t)tok * D;
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                const int b0 = 16 * m + 4 * g;
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = (acc[m][e] + qs_t * s_p[b0 + e]) / den;
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
                                                             float* __restrict__ S_out,
                                                             float* __restrict__ z_out, int N) {
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

// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void fill_zero_kernel(float* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (size_t)gridDim.x * kBlock) p[i] = 0.f;
}

// ---------------------------------------------------------------------------------------
// Host launchers.
SegPlan plan_segments(int64_t BH, int64_t N) {
    const int64_t nchunk = (N + kChunk - 1) / kChunk;
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

#define LA_DISPATCH_D(d, ...)                        \
    switch (d) {                                     \
        case 32: { constexpr int D = 32; __VA_ARGS__; } break; \
        case 64: { constexpr int D = 64; __VA_ARGS__; } break; \
        case 128: { constexpr int D = 128; __VA_ARGS__; } break; \
        default: return hipErrorInvalidValue;        \
    }

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_seg_state(int dt, int d, const void* k, const void* v, float* rec, int64_t BH,
                            int64_t N, SegPlan p, hipStream_t s) {
    const dim3 grid((unsigned)(p.nseg * BH));
    if (dt == kBF16) {
        LA_DISPATCH_D(d, hipLaunchKernelGGL((seg_state_kernel<bf16, D>), grid, dim3(kBlock), 0, s,
                                            (const bf16*)k, (const bf16*)v, rec, (int)N, p.cps, p.nseg));
    } else {
        LA_DISPATCH_D(d, hipLaunchKernelGGL((seg_state_kernel<float, D>), grid, dim3(kBlock), 0, s,
                                            (const float*)k, (const float*)v, rec, (int)N, p.cps, p.nseg));
    }
    return hipGetLastError();
}

hipError_t launch_scan(int d, float* rec, float* total, int64_t BH, int nseg, bool write_prefix,
                       hipStream_t s) {
    const int r4 = (int)(rec_floats(d) / 4);
    const dim3 grid((unsigned)(((r4 + kBlock - 1) / kBlock) * BH));
    LA_DISPATCH_D(d, hipLaunchKernelGGL((scan_kernel<D>), grid, dim3(kBlock), 0, s, rec, total, nseg,
                                        write_prefix ? 1 : 0, 0));
    return hipGetLastError();
}

hipError_t launch_causal_fwd(int dt, int d, const void* q, const void* k, const void* v, void* o,
                             float* den_out, const float* rec, int64_t BH, int64_t N, SegPlan p,
                             hipStream_t s) {
    const dim3 grid((unsigned)(p.nseg * BH));
    if (dt == kBF16) {
        LA_DISPATCH_D(d, hipLaunchKernelGGL((causal_fwd_kernel<bf16, D>), grid, dim3(kBlock), 0, s,
                                            (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o,
                                            den_out, rec, (int)N, p.cps, p.nseg));
    } else {
        switch (d) {
            case 32: hipLaunchKernelGGL((causal_fwd_kernel<float, 32>), grid, dim3(kBlock), 0, s,
                                        (const float*)q, (const float*)k, (const float*)v, (float*)o,
                                        den_out, rec, (int)N, p.cps, p.nseg); break;
            case 64: hipLaunchKernelGGL((causal_fwd_kernel<float, 64>), grid, dim3(kBlock), 0, s,
                                        (const float*)q, (const float*)k, (const float*)v, (float*)o,
                                        den_out, rec, (int)N, p.cps, p.nseg); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

hipError_t launch_noncausal_fwd(int dt, int d, const void* q, void* o, const float* total,
                                int64_t BH, int64_t N, SegPlan p, hipStream_t s) {
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

hipError_t launch_final_state(int d, const float* total, float* S_out, float* z_out, int64_t BH,
                              int64_t N, hipStream_t s) {
    LA_DISPATCH_D(d, hipLaunchKernelGGL((final_state_kernel<D>), dim3((unsigned)BH), dim3(kBlock), 0, s,
                                        total, S_out, z_out, (int)N));
    return hipGetLastError();
}

}  // namespace la

namespace la {
hipError_t launch_rscan(int d, float* rrec, int64_t BH, int nseg, hipStream_t s) {
    const int r4 = (int)(rec_floats(d) / 4);
    const dim3 grid((unsigned)(((r4 + kBlock - 1) / kBlock) * BH));
    LA_DISPATCH_D(d, hipLaunchKernelGGL((scan_kernel<D>), grid, dim3(kBlock), 0, s, rrec, (float*)nullptr,
                                        nseg, 1, 1));
    return hipGetLastError();
}
}  // namespace la
