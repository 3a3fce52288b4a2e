// favor.hip -- FAVOR+ positive random features for gfx950.
//
// Performer section of the page "Efficient Transformers Survey": the softmax
// kernel exp(q.k) is the expectation over w ~ N(0, I_d) of
// exp(w.q - |q|^2/2) exp(w.k - |k|^2/2), so the features
// phi(x)_i = m^{-1/2} exp(w_i.x - |x|^2/2), i < m, estimate it without bias and
// stay positive.  Here m is a multiple of d, and the constant m^{-1/2} is left out: it scales
// every weight of a row equally, so num / den does not see it (states and
// denominators carry the factor m).  Left out, the features average 1 over the
// draw of w, which suits the split phi = 1 + E the linear-attention kernels carry.
// The exponent needs fp32 accuracy (exp turns an absolute error in w.x into a
// relative one), so X Omega^T runs on the fp32 MFMA (v_mfma_f32_16x16x4_f32)
// with x widened exactly; one exp per feature finishes it.
#include "chunk.h"

namespace la {

// One workgroup takes CPB chunks of 64 rows.  Omega is staged in LDS once; each
// chunk's rows are prefetched into registers one chunk ahead, staged into LDS
// with their squared norms reduced by shuffles on the way (the D/4 threads of a
// row are adjacent lanes), and every wavefront forms the [D features x 16 rows]
// tile of Omega X^T for its 16 rows on MFMA.  bf16 rows are exact in bf16, so
// Omega is split into bf16 hi + lo parts and two bf16 MFMAs with fp32
// accumulation give the exponent to about 2^-17 of sum |w_i x_i| (a sixteenth
// of the fp32 MFMA's cost per product); fp32 rows use the fp32 MFMA.
// Feature block j = blockIdx.y (directions omega[j D .. j D + D - 1]) of row r = h N + t
// goes to row (h KF + j) N + t of out: with KF = m / D blocks, each head's features
// are KF contiguous [N][D] matrices (KF = 1: out is [rows][D] like x).
template <typename T, int D>
__global__ __launch_bounds__(kBlock) void favor_features_kernel(const T* __restrict__ x,
                                                                const float* __restrict__ omega, T* __restrict__ out,
                                                                int64_t rows, int64_t N, int KF) {
    constexpr bool kBF = sizeof(T) == 2;
    using M = Mma<T>;
    constexpr int DT = D / 16;
    constexpr int CPB = 4;                 // chunks of 64 rows per workgroup
    constexpr int TPR = D / 4;             // threads per row (4 elements each)
    constexpr int NI = kC * TPR / kBlock;  // 4-element groups per thread per chunk
    static_assert(NI >= 1 && kC * TPR % kBlock == 0 && TPR <= kWave, "rows must tile the workgroup");
    typedef typename std::conditional<kBF, uint2, uint4>::type word;
    __shared__ __attribute__((aligned(16))) T s_om[kBF ? 2 : 1][D * D];  // bf16: hi, lo; fp32: omega
    __shared__ __attribute__((aligned(16))) T s_x[2][kC * D];
    __shared__ float s_n[2][kC];
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 4;
    const int jb = blockIdx.y;
    omega += (int64_t)jb * D * D;

    for (int i = tid; i < D * D / 4; i += kBlock) {
        const int r = (4 * i) / D, c = (4 * i) % D;
        const f32x4 om = reinterpret_cast<const f32x4*>(omega)[i];
        if constexpr (kBF) {
            f32x4 hi;
#pragma unroll
            for (int e = 0; e < 4; ++e) hi[e] = (float)(bf16)om[e];
            store4(&Tile<T, D, D>{s_om[0]}.at(r, c), hi);
            store4(&Tile<T, D, D>{s_om[kBF ? 1 : 0]}.at(r, c), om - hi);
        } else {
            store4(&Tile<T, D, D>{s_om[0]}.at(r, c), om);
        }
    }
    // Group j of this thread: row (4 (tid + kBlock j)) / D of the chunk, columns 4 (tid mod TPR) ..
    auto load = [&](word* xr, int64_t r0) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int i = tid + kBlock * j;
            const int64_t row = r0 + (4 * i) / D;
            xr[j] = row < rows ? *reinterpret_cast<const word*>(x + row * D + (4 * i) % D) : word{};
        }
    };
    const int64_t base = (int64_t)blockIdx.x * CPB * kC;
    word xr[NI];
    load(xr, base);
    for (int cb = 0; cb < CPB; ++cb) {
        const int64_t r0 = base + (int64_t)cb * kC;
        if (r0 >= rows) break;
        const Tile<T, kC, D> tX{s_x[cb & 1]};
        float* sn = s_n[cb & 1];
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int i = tid + kBlock * j;
            *reinterpret_cast<word*>(&tX.at((4 * i) / D, (4 * i) % D)) = xr[j];  // as loaded
            const T* h = reinterpret_cast<const T*>(&xr[j]);
            float nrm = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) nrm += to_f32(h[e]) * to_f32(h[e]);
            nrm = sum_lanes<TPR>(nrm);
            if ((4 * i) % D == 0) sn[(4 * i) / D] = nrm;
        }
        load(xr, r0 + kC);  // the next chunk (past the rows: nothing is read)
        __syncthreads();    // rows and norms staged (and omega, for the first chunk)
        // acc[m]: the accumulator tile [feature 16 m + 4 g + e][row 16 w + (lane & 15)] of Omega X^T.
        f32x4 acc[DT];
#pragma unroll
        for (int m = 0; m < DT; ++m) acc[m] = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += M::KSTEP) {
            const typename M::frag xf = M::ld(tX, 16 * w, k0, lane);
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                acc[m] = M::mma(M::ld(Tile<T, D, D>{s_om[0]}, 16 * m, k0, lane), xf, acc[m]);
                if constexpr (kBF) acc[m] = M::mma(M::ld(Tile<T, D, D>{s_om[kBF ? 1 : 0]}, 16 * m, k0, lane), xf, acc[m]);
            }
        }
        const int t = 16 * w + (lane & 15);
        const int64_t row = r0 + t;
        if (row < rows) {
            const int64_t hh = row / N;
            const int64_t orow = (hh * KF + jb) * N + (row - hh * N);
            const float half_n = 0.5f * sn[t];
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = __builtin_amdgcn_exp2f((acc[m][e] - half_n) * 1.4426950408889634f);
                store4(out + orow * D + 16 * m + 4 * g, y);
            }
        }
        // The next chunk stages into the other LDS buffer; the barrier after that
        // staging keeps this chunk's buffer intact until every wave has read it.
    }
}

hipError_t launch_favor_features(int dt, int d, const void* x, const float* omega, void* out, int64_t rows,
                                 hipStream_t s, int64_t N, int KF) {
    if (rows == 0) return hipSuccess;
    if (N <= 0) N = rows;
    const dim3 grid((unsigned)((rows + 4 * kC - 1) / (4 * kC)), (unsigned)KF);
#define LA_FAV(TT, DD)                                                                                        \
    hipLaunchKernelGGL((favor_features_kernel<TT, DD>), grid, dim3(kBlock), 0, s, (const TT*)x, omega, (TT*)out, \
                       rows, N, KF)
    if (dt == kBF16) {
        switch (d) {
            case 32: LA_FAV(bf16, 32); break;
            case 64: LA_FAV(bf16, 64); break;
            case 128: LA_FAV(bf16, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (d) {
            case 32: LA_FAV(float, 32); break;
            case 64: LA_FAV(float, 64); break;
            case 128: LA_FAV(float, 128); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef LA_FAV
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// favor_features_bwd: the gradient through the features.  F_i = exp(w_i.x - |x|^2/2)
// has dF_i/dx = F_i (w_i - x), so for an upstream gradient dF of a row
//   dx = Omega^T u - x sum_i u_i,  u = dF * F   (elementwise, from the saved F).
// Omega^T u for 16 rows per wavefront is one MFMA contraction over the features i
// against Omega staged in LDS.  bf16 rows: u of two bf16 values has 16 significant
// bits, so u = u_hi + u_lo exactly in bf16, Omega is split the same way, and three
// bf16 MFMAs (hi hi, hi lo, lo hi) give the product to about 2^-16 relative; fp32 rows
// use the fp32 MFMA.  One workgroup takes CPB chunks of 64 rows.
template <typename T, int D>
__global__ __launch_bounds__(kBlock) void favor_features_bwd_kernel(const T* __restrict__ x,
                                                                    const float* __restrict__ omega,
                                                                    const T* __restrict__ F, const T* __restrict__ dF,
                                                                    T* __restrict__ dx, int64_t rows) {
    constexpr bool kBF = sizeof(T) == 2;
    using M = Mma<T>;
    constexpr int DT = D / 16;
    constexpr int CPB = 4;
    constexpr int TPR = D / 4;
    constexpr int NI = kC * TPR / kBlock;
    static_assert(NI >= 1 && kC * TPR % kBlock == 0 && TPR <= kWave, "rows must tile the workgroup");
    typedef typename std::conditional<kBF, uint2, uint4>::type word;
    __shared__ __attribute__((aligned(16))) T s_om[kBF ? 2 : 1][D * D];  // bf16: hi, lo; fp32: omega
    __shared__ __attribute__((aligned(16))) T s_u[kBF ? 2 : 1][kC * D];  // bf16: u hi, lo; fp32: u
    __shared__ float s_s[kC];
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 4;

    for (int i = tid; i < D * D / 4; i += kBlock) {
        const int r = (4 * i) / D, c = (4 * i) % D;
        const f32x4 om = reinterpret_cast<const f32x4*>(omega)[i];
        if constexpr (kBF) {
            f32x4 hi;
#pragma unroll
            for (int e = 0; e < 4; ++e) hi[e] = (float)(bf16)om[e];
            store4(&Tile<T, D, D>{s_om[0]}.at(r, c), hi);
            store4(&Tile<T, D, D>{s_om[kBF ? 1 : 0]}.at(r, c), om - hi);
        } else {
            store4(&Tile<T, D, D>{s_om[0]}.at(r, c), om);
        }
    }
    const int64_t base = (int64_t)blockIdx.x * CPB * kC;
    // F and dF words of chunk cb for this thread's groups of 4 (zeros past the rows); the next
    // chunk's are loaded while the current chunk's MFMAs run.
    word pf[NI], pg[NI];
    auto load_chunk = [&](int cb) {
        const int64_t r0 = base + (int64_t)cb * kC;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int i = tid + kBlock * j;
            const int64_t row = r0 + (4 * i) / D;
            pf[j] = word{};
            pg[j] = word{};
            if (row < rows) {
                pf[j] = *reinterpret_cast<const word*>(F + row * D + (4 * i) % D);
                pg[j] = *reinterpret_cast<const word*>(dF + row * D + (4 * i) % D);
            }
        }
    };
    load_chunk(0);
#pragma unroll
    for (int cb = 0; cb < CPB; ++cb) {
        const int64_t r0 = base + (int64_t)cb * kC;
        if (r0 >= rows) break;
        if (cb > 0) __syncthreads();  // every wave has read the previous chunk's u
        // u = dF * F of this thread's groups of 4, split hi + lo, and the row sums of u.
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int i = tid + kBlock * j;
            const int rr = (4 * i) / D, c = (4 * i) % D;
            const word fw = pf[j], gw = pg[j];
            const T* fh = reinterpret_cast<const T*>(&fw);
            const T* gh = reinterpret_cast<const T*>(&gw);
            f32x4 u;
            float su = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u[e] = to_f32(fh[e]) * to_f32(gh[e]);
                su += u[e];
            }
            if constexpr (kBF) {
                f32x4 hi;
#pragma unroll
                for (int e = 0; e < 4; ++e) hi[e] = (float)(bf16)u[e];
                store4(&Tile<T, kC, D>{s_u[0]}.at(rr, c), hi);
                store4(&Tile<T, kC, D>{s_u[kBF ? 1 : 0]}.at(rr, c), u - hi);
            } else {
                store4(&Tile<T, kC, D>{s_u[0]}.at(rr, c), u);
            }
            su = sum_lanes<TPR>(su);
            if (c == 0) s_s[rr] = su;
        }
        if (cb + 1 < CPB && r0 + kC < rows) load_chunk(cb + 1);
        raw_barrier();  // u and its row sums staged (and omega, for the first chunk); loads stay in flight
        // acc[m]: [feature 16 m + 4 g + e][row 16 w + (lane & 15)] of Omega^T u.
        f32x4 acc[DT];
#pragma unroll
        for (int m = 0; m < DT; ++m) acc[m] = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += M::KSTEP) {
            const typename M::frag uh = M::ld(Tile<T, kC, D>{s_u[0]}, 16 * w, k0, lane);
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                const typename M::frag oh = M::ld_tr(Tile<T, D, D>{s_om[0]}, k0, 16 * m, lane);
                acc[m] = M::mma(oh, uh, acc[m]);
                if constexpr (kBF) {
                    const typename M::frag ul = M::ld(Tile<T, kC, D>{s_u[kBF ? 1 : 0]}, 16 * w, k0, lane);
                    acc[m] = M::mma(oh, ul, acc[m]);
                    acc[m] = M::mma(M::ld_tr(Tile<T, D, D>{s_om[kBF ? 1 : 0]}, k0, 16 * m, lane), uh, acc[m]);
                }
            }
        }
        const int t = 16 * w + (lane & 15);
        const int64_t row = r0 + t;
        if (row < rows) {
            const float su = s_s[t];
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                const int c = 16 * m + 4 * g;
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = acc[m][e] - su * to_f32(x[row * D + c + e]);
                store4(dx + row * D + c, y);
            }
        }
    }
}

// KF feature blocks (m = KF d; omega [KF d][d], F and dF [heads][KF][N][d] for x [heads][N][d]):
// the map is linear in u, so dx = sum_j (Omega_j^T u_j - x sum(u_j)).  Blocks are the outer
// loop, so each Omega_j is staged once per workgroup; the MFMA accumulators and row sums of
// the workgroup's CPB chunks carry over the blocks.  The F and dF words of the next (block,
// chunk) step are loaded into registers while the current step's MFMAs run.  Omega and u
// as in the kernel above.
template <int D>
constexpr int favor_bwd_blocks_cpb() { return D > 64 ? 1 : 4; }
template <typename T, int D>
__global__ __launch_bounds__(kBlock) void favor_features_bwd_blocks_kernel(
    const T* __restrict__ x, const float* __restrict__ omega, const T* __restrict__ F, const T* __restrict__ dF,
    T* __restrict__ dx, int64_t rows, int64_t N, int KF) {
    constexpr bool kBF = sizeof(T) == 2;
    using M = Mma<T>;
    constexpr int DT = D / 16;
    constexpr int CPB = favor_bwd_blocks_cpb<D>();
    constexpr int TPR = D / 4;
    constexpr int NI = kC * TPR / kBlock;
    static_assert(NI >= 1 && kC * TPR % kBlock == 0 && TPR <= kWave, "rows must tile the workgroup");
    typedef typename std::conditional<kBF, uint2, uint4>::type word;
    __shared__ __attribute__((aligned(16))) T s_om[kBF ? 2 : 1][D * D];
    __shared__ __attribute__((aligned(16))) T s_u[kBF ? 2 : 1][kC * D];
    __shared__ float s_s[CPB][kC];
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 4;
    const int64_t base = (int64_t)blockIdx.x * CPB * kC;

    // F and dF words of step (jb, cb) for this thread's groups of 4 (zeros past the rows).
    word pf[NI], pg[NI];
    auto load_step = [&](int jb, int cb) {
        const int64_t r0 = base + (int64_t)cb * kC;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int i = tid + kBlock * j;
            const int rr = (4 * i) / D, c = (4 * i) % D;
            const int64_t row = r0 + rr;
            pf[j] = word{};
            pg[j] = word{};
            if (row < rows) {
                const int64_t hh = row / N;
                const int64_t frow = (hh * KF + jb) * N + (row - hh * N);
                pf[j] = *reinterpret_cast<const word*>(F + frow * D + c);
                pg[j] = *reinterpret_cast<const word*>(dF + frow * D + c);
            }
        }
    };
    load_step(0, 0);

    f32x4 acc[CPB][DT];
#pragma unroll
    for (int cb = 0; cb < CPB; ++cb)
#pragma unroll
        for (int m = 0; m < DT; ++m) acc[cb][m] = zero4();
    for (int jb = 0; jb < KF; ++jb) {
        if (jb > 0) __syncthreads();  // every wave has read Omega_{j-1} and the last u
        const f32x4* ob = reinterpret_cast<const f32x4*>(omega + (int64_t)jb * D * D);
        for (int i = tid; i < D * D / 4; i += kBlock) {
            const int r = (4 * i) / D, c = (4 * i) % D;
            const f32x4 om = ob[i];
            if constexpr (kBF) {
                f32x4 hi;
#pragma unroll
                for (int e = 0; e < 4; ++e) hi[e] = (float)(bf16)om[e];
                store4(&Tile<T, D, D>{s_om[0]}.at(r, c), hi);
                store4(&Tile<T, D, D>{s_om[kBF ? 1 : 0]}.at(r, c), om - hi);
            } else {
                store4(&Tile<T, D, D>{s_om[0]}.at(r, c), om);
            }
        }
#pragma unroll
        for (int cb = 0; cb < CPB; ++cb) {
            const int64_t r0 = base + (int64_t)cb * kC;
            if (r0 >= rows) break;
            if (cb > 0) __syncthreads();  // every wave has read the previous chunk's u
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int i = tid + kBlock * j;
                const int rr = (4 * i) / D, c = (4 * i) % D;
                const word fw = pf[j], gw = pg[j];
                const T* fh = reinterpret_cast<const T*>(&fw);
                const T* gh = reinterpret_cast<const T*>(&gw);
                f32x4 u;
                float su = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    u[e] = to_f32(fh[e]) * to_f32(gh[e]);
                    su += u[e];
                }
                if constexpr (kBF) {
                    f32x4 hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e) hi[e] = (float)(bf16)u[e];
                    store4(&Tile<T, kC, D>{s_u[0]}.at(rr, c), hi);
                    store4(&Tile<T, kC, D>{s_u[kBF ? 1 : 0]}.at(rr, c), u - hi);
                } else {
                    store4(&Tile<T, kC, D>{s_u[0]}.at(rr, c), u);
                }
                su = sum_lanes<TPR>(su);
                if (c == 0) s_s[cb][rr] = jb == 0 ? su : s_s[cb][rr] + su;
            }
            // The next step's words: the next chunk of this block, else the first chunk of the next block.
            if (cb + 1 < CPB && r0 + kC < rows)
                load_step(jb, cb + 1);
            else if (jb + 1 < KF)
                load_step(jb + 1, 0);
            raw_barrier();  // u, its row sums and Omega_j staged (the next step's loads stay in flight)
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += M::KSTEP) {
                const typename M::frag uh = M::ld(Tile<T, kC, D>{s_u[0]}, 16 * w, k0, lane);
#pragma unroll
                for (int m = 0; m < DT; ++m) {
                    const typename M::frag oh = M::ld_tr(Tile<T, D, D>{s_om[0]}, k0, 16 * m, lane);
                    acc[cb][m] = M::mma(oh, uh, acc[cb][m]);
                    if constexpr (kBF) {
                        const typename M::frag ul = M::ld(Tile<T, kC, D>{s_u[kBF ? 1 : 0]}, 16 * w, k0, lane);
                        acc[cb][m] = M::mma(oh, ul, acc[cb][m]);
                        acc[cb][m] =
                            M::mma(M::ld_tr(Tile<T, D, D>{s_om[kBF ? 1 : 0]}, k0, 16 * m, lane), uh, acc[cb][m]);
                    }
                }
            }
        }
    }
    // s_s of the last block was written before the last barrier; each row's own lanes read it.
#pragma unroll
    for (int cb = 0; cb < CPB; ++cb) {
        const int t = 16 * w + (lane & 15);
        const int64_t row = base + (int64_t)cb * kC + t;
        if (row < rows) {
            const float su = s_s[cb][t];
#pragma unroll
            for (int m = 0; m < DT; ++m) {
                const int c = 16 * m + 4 * g;
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = acc[cb][m][e] - su * to_f32(x[row * D + c + e]);
                store4(dx + row * D + c, y);
            }
        }
    }
}

hipError_t launch_favor_features_bwd(int dt, int d, const void* x, const float* omega, const void* F, const void* dF,
                                     void* dx, int64_t rows, hipStream_t s, int64_t N, int KF) {
    if (KF < 1 || (KF > 1 && N <= 0)) return hipErrorInvalidValue;
    if (rows == 0) return hipSuccess;
    const int cpb = KF == 1 ? 4 : (d > 64 ? favor_bwd_blocks_cpb<128>() : favor_bwd_blocks_cpb<64>());
    const dim3 grid((unsigned)((rows + cpb * kC - 1) / (cpb * kC)));
#define LA_FAVB(TT, DD)                                                                                         \
    if (KF > 1)                                                                                                 \
        hipLaunchKernelGGL((favor_features_bwd_blocks_kernel<TT, DD>), grid, dim3(kBlock), 0, s, (const TT*)x,  \
                           omega, (const TT*)F, (const TT*)dF, (TT*)dx, rows, N, KF);                           \
    else                                                                                                        \
        hipLaunchKernelGGL((favor_features_bwd_kernel<TT, DD>), grid, dim3(kBlock), 0, s, (const TT*)x, omega,  \
                           (const TT*)F, (const TT*)dF, (TT*)dx, rows)
    if (dt == kBF16) {
        switch (d) {
            case 32: LA_FAVB(bf16, 32); break;
            case 64: LA_FAVB(bf16, 64); break;
            case 128: LA_FAVB(bf16, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (d) {
            case 32: LA_FAVB(float, 32); break;
            case 64: LA_FAVB(float, 64); break;
            case 128: LA_FAVB(float, 128); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef LA_FAVB
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// combine_blocks: attention over KF feature blocks of one head, each computed as its own
// head (o_j = num_j / den_j, den_j), put together: num = sum_j num_j and den = sum_j den_j,
// so o = sum_j den_j o_j / sum_j den_j.  ob [BH][KF][N][D] in T, db [BH][KF][N] fp32;
// o [BH][N][D], den_out (nullable) [BH][N].  One thread per 4 elements of a row.
template <typename T, int D>
__global__ __launch_bounds__(kBlock) void combine_blocks_kernel(const T* __restrict__ ob, const float* __restrict__ db,
                                                                T* __restrict__ o, float* __restrict__ den_out,
                                                                int64_t rows, int64_t N, int KF) {
    constexpr int TPR = D / 4;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t row = i / TPR;
    if (row >= rows) return;
    const int c = 4 * (int)(i % TPR);
    const int64_t hh = row / N, t = row - hh * N;
    f32x4 acc = zero4();
    float den = 0.f;
    for (int j = 0; j < KF; ++j) {
        const int64_t br = (hh * KF + j) * N + t;
        const float dj = db != nullptr ? db[br] : 1.f;
        const T* p = ob + br * D + c;
        den += dj;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += dj * to_f32(p[e]);
    }
    if (db == nullptr) {  // a plain sum over the blocks (the value gradient)
        store4(o + row * D + c, acc);
        return;
    }
    const float inv = rcp_f(den);
    store4(o + row * D + c, acc * inv);
    if (den_out != nullptr && c == 0) den_out[row] = den;
}

// ---------------------------------------------------------------------------------------
// combine_stats: the backward's row statistics over KF feature blocks that share one
// normalization.  rowstat [heads][KF][N] holds (den, G . num_j) per block from the
// statistics sweep (den: the whole head's); every block's entry becomes (den, g) with
// g = -(sum_j G . num_j) / den, the g of the whole head (same reciprocal as the sweeps).
__global__ __launch_bounds__(kBlock) void combine_stats_kernel(float2* __restrict__ rowstat, int64_t rows, int64_t N,
                                                               int KF) {
    const int64_t row = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (row >= rows) return;
    const int64_t hh = row / N, t = row - hh * N;
    float h = 0.f;
    for (int j = 0; j < KF; ++j) h += rowstat[(hh * KF + j) * N + t].y;
    const float den = rowstat[hh * KF * N + t].x;
    const float g = -h * rcp_f(den);
    for (int j = 0; j < KF; ++j) rowstat[(hh * KF + j) * N + t] = make_float2(den, g);
}

// stats_from_output: the same row statistics from the forward's output O of each head row
// instead of a statistics sweep: G . num_j summed over the blocks is G . O den, so
// g = -G . O with G = dO / den rounded to the operand type as the sweeps round it (same
// reciprocal).  dout, o [heads][N][D]; den [heads][N]; every block's entry of rowstat
// [heads][KF][N] gets (den, g).  D / 4 adjacent lanes per row, 4 elements each.
template <typename T, int D>
__global__ __launch_bounds__(kBlock) void stats_from_output_kernel(const T* __restrict__ dout, const T* __restrict__ o,
                                                                   const float* __restrict__ den,
                                                                   float2* __restrict__ rowstat, int64_t rows,
                                                                   int64_t N, int KF) {
    constexpr int TPR = D / 4;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t row = i / TPR;
    const int c = 4 * (int)(i % TPR);
    const bool valid = row < rows;
    const float dn = valid ? den[row] : 1.f;
    const float inv = rcp_f(dn);
    // One 4-element word of dO and of O per thread (8 bytes for bf16, 16 for fp32).
    typedef typename std::conditional<sizeof(T) == 2, uint2, uint4>::type word;
    word dw{}, ow{};
    if (valid) {
        dw = *reinterpret_cast<const word*>(dout + row * D + c);
        ow = *reinterpret_cast<const word*>(o + row * D + c);
    }
    const T* dh = reinterpret_cast<const T*>(&dw);
    const T* oh = reinterpret_cast<const T*>(&ow);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) s += to_f32(from_f32<T>(to_f32(dh[e]) * inv)) * to_f32(oh[e]);
    s = sum_lanes<TPR>(s);
    if (valid && c == 0) {
        const int64_t hh = row / N, t = row - hh * N;
        for (int j = 0; j < KF; ++j) rowstat[(hh * KF + j) * N + t] = make_float2(dn, -s);
    }
}

hipError_t launch_stats_from_output(int dt, int d, const void* dout, const void* o, const float* den, float* rowstat,
                                    int64_t rows, int64_t N, int KF, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((rows * (d / 4) + kBlock - 1) / kBlock));
#define LA_SFO(TT, DD)                                                                                          \
    hipLaunchKernelGGL((stats_from_output_kernel<TT, DD>), grid, dim3(kBlock), 0, s, (const TT*)dout,          \
                       (const TT*)o, den, reinterpret_cast<float2*>(rowstat), rows, N, KF)
    if (dt == kBF16) {
        switch (d) {
            case 32: LA_SFO(bf16, 32); break;
            case 64: LA_SFO(bf16, 64); break;
            case 128: LA_SFO(bf16, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (d) {
            case 32: LA_SFO(float, 32); break;
            case 64: LA_SFO(float, 64); break;
            case 128: LA_SFO(float, 128); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef LA_SFO
    return hipGetLastError();
}

hipError_t launch_combine_stats(float* rowstat, int64_t rows, int64_t N, int KF, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(combine_stats_kernel, dim3((unsigned)((rows + kBlock - 1) / kBlock)), dim3(kBlock), 0, s,
                       reinterpret_cast<float2*>(rowstat), rows, N, KF);
    return hipGetLastError();
}

hipError_t launch_combine_blocks(int dt, int d, const void* ob, const float* db, void* o, float* den_out,
                                 int64_t rows, int64_t N, int KF, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((rows * (d / 4) + kBlock - 1) / kBlock));
#define LA_CMB(TT, DD)                                                                                         \
    hipLaunchKernelGGL((combine_blocks_kernel<TT, DD>), grid, dim3(kBlock), 0, s, (const TT*)ob, db, (TT*)o,    \
                       den_out, rows, N, KF)
    if (dt == kBF16) {
        switch (d) {
            case 32: LA_CMB(bf16, 32); break;
            case 64: LA_CMB(bf16, 64); break;
            case 128: LA_CMB(bf16, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (d) {
            case 32: LA_CMB(float, 32); break;
            case 64: LA_CMB(float, 64); break;
            case 128: LA_CMB(float, 128); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef LA_CMB
    return hipGetLastError();
}

}  // namespace la
