// decode.hip -- one recurrent decode step of kernelized linear attention (gfx950).
//
// Per (b, h), in place ("Why It Matters" of the linear-attention proposition on
// the page "Efficient Transformers Survey": process tokens one by one, updating
// S and z incrementally, with constant memory per step):
//   S += phi(k) v^T,  z += phi(k),  o = phi(q)^T S / phi(q)^T z.
// The step is a rank-1 update plus a vector-matrix product over the fp32 d x d
// state: 8 bytes of HBM traffic per 2 flops, so it is pure streaming.  MFMA
// has nothing to do here; the kernel reads and writes each state row once with
// 16-byte vector accesses and keeps every load of the workgroup in flight
// before the first use.
#include "common.h"
#include "launch.h"

namespace la {

template <typename T, int D>
__global__ __launch_bounds__(kBlock) void decode_kernel(float* __restrict__ S, float* __restrict__ z,
                                                        const T* __restrict__ q, const T* __restrict__ k,
                                                        const T* __restrict__ v, T* __restrict__ o) {
    constexpr int F4 = D / 4;              // float4 per state row
    constexpr int RPP = kBlock / F4;       // rows per pass
    constexpr int NP = D / RPP;            // passes
    static_assert(kBlock % F4 == 0 && D % RPP == 0, "state rows must tile the workgroup");
    __shared__ float s_qf[D], s_kf[D], s_v[D];
    __shared__ float s_red[RPP][D];
    __shared__ float s_den[kBlock / kWave];

    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int rg = tid / F4, cq = tid % F4;
    f32x4* Sh = reinterpret_cast<f32x4*>(S + (int64_t)bh * D * D);

    // Issue the state loads first: every one is independent.
    f32x4 srow[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) srow[p] = Sh[(rg + RPP * p) * F4 + cq];

    float zn = 0.f;
    if (tid < D) {
        const int64_t off = (int64_t)bh * D + tid;
        const float kf = phi_f(to_f32(k[off]));
        const float qf = phi_f(to_f32(q[off]));
        s_kf[tid] = kf;
        s_qf[tid] = qf;
        s_v[tid] = to_f32(v[off]);
        zn = z[off] + kf;
        z[off] = zn;
        zn *= qf;  // this feature's share of phi(q)^T z
    }
    // denominator: block reduction of phi(q)_a z_a
    zn = sum_lanes<kWave>(zn);
    if ((tid & (kWave - 1)) == 0) s_den[tid / kWave] = zn;
    __syncthreads();

    const f32x4 v4 = *reinterpret_cast<const f32x4*>(&s_v[4 * cq]);
    f32x4 acc = zero4();
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int a = rg + RPP * p;
        const float kf = s_kf[a], qf = s_qf[a];
        f32x4 x = srow[p];
        x += kf * v4;
        Sh[a * F4 + cq] = x;
        acc += qf * x;
    }
    *reinterpret_cast<f32x4*>(&s_red[rg][4 * cq]) = acc;
    __syncthreads();
    if (tid < D) {
        float num = 0.f;
#pragma unroll
        for (int r = 0; r < RPP; ++r) num += s_red[r][tid];
        float den = 0.f;
#pragma unroll
        for (int w = 0; w < kBlock / kWave; ++w) den += s_den[w];
        o[(int64_t)bh * D + tid] = from_f32<T>(num / den);
    }
}

// ---------------------------------------------------------------------------------------
// decode_steps: T recurrent steps per (b, key/value head) in one pass over the
// state, for G = H / Hkv query heads sharing that head's state (G = 1: one state
// per query head).  Per token t: S += phi(k_t) v_t^T, z += phi(k_t) once, then
// each of the G query heads reads o = phi(q)^T S / phi(q)^T z.  The d x d state is
// held in registers across the call (thread (rg, cq) owns columns 4 cq .. 4 cq + 3
// of rows NP rg .. NP rg + NP - 1: its feature values come in 16-byte LDS reads), so
// it moves through HBM once per call instead of once per
// token, and once per group instead of once per query head.
// With KF feature blocks (features m = KF d, block layout), the state of block j of
// key/value head kv is a state of its own (flat index kv KF + j) that reads the
// head's values; q, o are the block layout's [B][H][KF][T][d] and den_out (nullable)
// gets each row's denominator, for the combine over blocks.
// Work goes in rows (t, h), token-major: a block of RB rows stages phi(q) of each
// row and, on the row that opens a token (h = 0), phi(k) and v of that token
// (zeros elsewhere, so z sums each token once); per row each thread applies the
// token's rank-1 update where the row opens one, then forms its part of
// phi(q)^T S, reduced over the row groups with shuffles inside a wavefront and
// through LDS across the four.
template <typename T, int D, class FM = FeatElu, bool kBlocks = false>
__global__ __launch_bounds__(kBlock) void decode_steps_kernel(float* __restrict__ S, float* __restrict__ z,
                                                              const T* __restrict__ q, const T* __restrict__ k,
                                                              const T* __restrict__ v, T* __restrict__ o, int ntok,
                                                              int G, int KFb, float* __restrict__ den_out) {
    const int KF = kBlocks ? KFb : 1;  // feature blocks (compiled out for one)
    constexpr int F4 = D / 4;         // float4 per state row
    constexpr int RPP = kBlock / F4;  // row groups
    constexpr int NP = D / RPP;       // rows per thread: rows NP rg .. NP rg + NP - 1
    constexpr int VW = NP % 4 == 0 ? 4 : 1;  // feature values per LDS read
    constexpr int NW = kBlock / kWave;
    constexpr int RB = D <= 64 ? 16 : 8;  // (token, query head) rows per block
    static_assert(kBlock % F4 == 0 && D % RPP == 0 && F4 <= kWave, "state rows must tile the workgroup");
    __shared__ __attribute__((aligned(16))) float s_qf[RB][D], s_kf[RB][D], s_v[RB][D];
    __shared__ __attribute__((aligned(16))) float s_red[RB][NW][D];
    __shared__ float s_den[RB][NW];

    const int kvh = blockIdx.x;  // flat (b, key/value head, feature block)
    const int64_t bkv = kvh / KF, jb = kvh - bkv * KF;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    const int rg = tid / F4, cq = tid % F4;
    f32x4* Sh = reinterpret_cast<f32x4*>(S + (int64_t)kvh * D * D);
    const int64_t krow0 = (int64_t)kvh * ntok;        // first token row of this state's keys
    const int64_t vrow0 = bkv * ntok;                 // ... and of its head's values
    // Row t of query head h of the group: ((bkv G + h) KF + jb) ntok + t in q, o.
    auto qrow = [&](int64_t t, int64_t h) { return ((bkv * G + h) * KF + jb) * ntok + t; };
    const int64_t nrows = (int64_t)G * ntok;

    f32x4 x[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) x[p] = Sh[(NP * rg + p) * F4 + cq];
    float zn = tid < D ? z[(int64_t)kvh * D + tid] : 0.f;

    for (int64_t r0 = 0; r0 < nrows; r0 += RB) {
        const int nb = (int)min((int64_t)RB, nrows - r0);
        // Stage the block: row i is token t = (r0 + i) / G of query head h = (r0 + i) % G.
        // Rows past the end and rows that do not open a token carry phi(k) = 0, v = 0.
        for (int i = tid; i < RB * D; i += kBlock) {
            const int ri = i / D, a = i % D;
            float qf = 1.f, kf = 0.f, vv = 0.f;
            if (ri < nb) {
                const int64_t r = r0 + ri;
                const int64_t t = r / G, h = r % G;
                qf = FM::phi(to_f32(q[qrow(t, h) * D + a]));
                if (h == 0) {
                    kf = FM::phi(to_f32(k[(krow0 + t) * D + a]));
                    vv = to_f32(v[(vrow0 + t) * D + a]);
                }
            }
            s_qf[ri][a] = qf;
            s_kf[ri][a] = kf;
            s_v[ri][a] = vv;
        }
        __syncthreads();
        // z and each row's denominator phi(q)^T z (feature a = tid).
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            float dp = 0.f;
            if (tid < D) {
                zn += s_kf[i][tid];
                dp = s_qf[i][tid] * zn;
            }
            dp = sum_lanes<kWave>(dp);
            if (lane == 0) s_den[i][w] = dp;
        }
        // Rank-1 update where a row opens a token, then phi(q)^T S, row by row.
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const bool opens = i < nb && (r0 + i) % G == 0;  // uniform over the workgroup
            if (opens) {
                const f32x4 v4 = *reinterpret_cast<const f32x4*>(&s_v[i][4 * cq]);
#pragma unroll
                for (int p4 = 0; p4 < NP; p4 += VW) {
                    float kf4[VW];
                    if constexpr (VW == 4) *reinterpret_cast<f32x4*>(kf4) = *reinterpret_cast<const f32x4*>(&s_kf[i][NP * rg + p4]);
                    else kf4[0] = s_kf[i][NP * rg + p4];
#pragma unroll
                    for (int e = 0; e < VW; ++e) x[p4 + e] += kf4[e] * v4;
                }
            }
            f32x4 acc = zero4();
#pragma unroll
            for (int p4 = 0; p4 < NP; p4 += VW) {
                float qf4[VW];
                if constexpr (VW == 4) *reinterpret_cast<f32x4*>(qf4) = *reinterpret_cast<const f32x4*>(&s_qf[i][NP * rg + p4]);
                else qf4[0] = s_qf[i][NP * rg + p4];
#pragma unroll
                for (int e = 0; e < VW; ++e) acc += qf4[e] * x[p4 + e];
            }
#pragma unroll
            for (int off = F4; off < kWave; off <<= 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], off, kWave);
            }
            if (lane < F4) *reinterpret_cast<f32x4*>(&s_red[i][w][4 * cq]) = acc;
        }
        __syncthreads();
        for (int i = tid; i < nb * D; i += kBlock) {
            const int ri = i / D, b = i % D;
            const int64_t r = r0 + ri;
            const int64_t t = r / G, h = r % G;
            float num = 0.f, den = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                num += s_red[ri][ww][b];
                den += s_den[ri][ww];
            }
            o[qrow(t, h) * D + b] = from_f32<T>(num / den);
            if (kBlocks && den_out != nullptr && b == 0) den_out[qrow(t, h)] = den;
        }
        __syncthreads();  // the block's LDS is free for the next one
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) Sh[(NP * rg + p) * F4 + cq] = x[p];
    if (tid < D) z[(int64_t)kvh * D + tid] = zn;
}

template <class FM>
static hipError_t launch_decode_steps_fm(int dt, int d, float* S, float* z, const void* q, const void* k,
                                         const void* v, void* o, int64_t BHkv, int64_t T, int64_t G, hipStream_t s,
                                         int KF, float* den_out) {
    const dim3 grid((unsigned)(BHkv * KF));
#define LA_DECS(TT, DD)                                                                                    \
    do {                                                                                                   \
        if (KF > 1)                                                                                        \
            hipLaunchKernelGGL((decode_steps_kernel<TT, DD, FM, true>), grid, dim3(kBlock), 0, s, S, z,    \
                               (const TT*)q, (const TT*)k, (const TT*)v, (TT*)o, (int)T, (int)G, KF, den_out); \
        else                                                                                               \
            hipLaunchKernelGGL((decode_steps_kernel<TT, DD, FM, false>), grid, dim3(kBlock), 0, s, S, z,   \
                               (const TT*)q, (const TT*)k, (const TT*)v, (TT*)o, (int)T, (int)G, 1, nullptr); \
    } while (0)
    if (dt == kBF16) {
        switch (d) {
            case 32: LA_DECS(bf16, 32); break;
            case 64: LA_DECS(bf16, 64); break;
            case 128: LA_DECS(bf16, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (d) {
            case 32: LA_DECS(float, 32); break;
            case 64: LA_DECS(float, 64); break;
            case 128: LA_DECS(float, 128); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef LA_DECS
    return hipGetLastError();
}

hipError_t launch_decode_steps(int dt, int d, float* S, float* z, const void* q, const void* k, const void* v,
                               void* o, int64_t BHkv, int64_t T, int64_t G, hipStream_t s, int feat, int KF,
                               float* den_out) {
    return feat == kFeatGiven ? launch_decode_steps_fm<FeatGiven>(dt, d, S, z, q, k, v, o, BHkv, T, G, s, KF, den_out)
                              : launch_decode_steps_fm<FeatElu>(dt, d, S, z, q, k, v, o, BHkv, T, G, s, KF, den_out);
}

hipError_t launch_decode(int dt, int d, float* S, float* z, const void* q, const void* k,
                         const void* v, void* o, int64_t BH, hipStream_t s) {
    const dim3 grid((unsigned)BH);
#define LA_DEC(TT, DD)                                                                              \
    hipLaunchKernelGGL((decode_kernel<TT, DD>), grid, dim3(kBlock), 0, s, S, z, (const TT*)q, (const TT*)k, \
                       (const TT*)v, (TT*)o)
    if (dt == kBF16) {
        switch (d) {
            case 32: LA_DEC(bf16, 32); break;
            case 64: LA_DEC(bf16, 64); break;
            case 128: LA_DEC(bf16, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (d) {
            case 32: LA_DEC(float, 32); break;
            case 64: LA_DEC(float, 64); break;
            case 128: LA_DEC(float, 128); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef LA_DEC
    return hipGetLastError();
}

}  // namespace la
