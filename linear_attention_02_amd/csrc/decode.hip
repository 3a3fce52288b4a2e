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
