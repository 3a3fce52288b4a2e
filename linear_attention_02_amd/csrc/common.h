// common.h -- device helpers shared by the gfx950 linear-attention kernels.
//
// Everything here is written for CDNA4 (gfx950): 64-lane wavefronts, the
// v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x4_f32 matrix instructions, and
// LDS tiles with an XOR swizzle on 16-byte granules.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---- scalar conversions ------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// Round a float through the operand type and back (the value the MFMA sees).
template <typename OT>
__device__ __forceinline__ float round_to(float x) { return to_f32(from_f32<OT>(x)); }

// ---- feature map phi(x) = elu(x) + 1 -------------------------------------------------
// phi(x) = x + 1 (x > 0), exp(x) (x <= 0).  E(x) = phi(x) - 1 = elu(x).
__device__ __forceinline__ float phi_f(float x) { return x > 0.f ? x + 1.f : __expf(x); }
__device__ __forceinline__ float elu_f(float x) { return x > 0.f ? x : expm1f(x); }
// phi'(x) = 1 (x > 0), exp(x) (x <= 0).
__device__ __forceinline__ float dphi_f(float x) { return x > 0.f ? 1.f : __expf(x); }

// ---- 16-byte vectors of input elements -------------------------------------------------
template <typename T>
struct Vec16 {
    static constexpr int EV = 16 / (int)sizeof(T);  // elements per 16 bytes
    uint4 raw;
    __device__ __forceinline__ float get(int e) const {
        const T* p = reinterpret_cast<const T*>(&raw);
        return to_f32(p[e]);
    }
    __device__ __forceinline__ void set(int e, float x) {
        T* p = reinterpret_cast<T*>(&raw);
        p[e] = from_f32<T>(x);
    }
};

template <typename T>
__device__ __forceinline__ uint4 load16(const T* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// ---- swizzled LDS tiles ----------------------------------------------------------------
// ROWS x COLS elements of OT, row-major, with the 16-byte granule index of each
// row XOR-ed by a row-dependent value.  MFMA operand reads (16 rows x one
// granule) and transposed scalar writes (8 rows x one column) then spread over
// the LDS banks.
template <typename OT, int ROWS, int COLS>
struct Tile {
    static constexpr int EV = 16 / (int)sizeof(OT);
    static constexpr int G = COLS / EV;
    static_assert(COLS % EV == 0, "tile width must be whole granules");
    static_assert(G >= 4 && (G & (G - 1)) == 0, "granules per row must be a power of two >= 4");
    static constexpr int kElems = ROWS * COLS;
    OT* p;
    __device__ __forceinline__ static int swz(int r) { return (r + (r >> 3)) & (G - 1); }
    __device__ __forceinline__ int off(int r, int c) const {
        return r * COLS + (((c / EV) ^ swz(r)) * EV) + (c % EV);
    }
    __device__ __forceinline__ OT* granule(int r, int gi) const {
        return p + r * COLS + ((gi ^ swz(r)) * EV);
    }
    __device__ __forceinline__ OT& at(int r, int c) const { return p[off(r, c)]; }
};

// ---- MFMA ------------------------------------------------------------------------------
// 16x16 output tile D[i][j] += sum_k X[i][k] * Y[j][k].  Lane l supplies row
// (l & 15) of X and of Y; the k values it supplies are the same for X and Y,
// so the result does not depend on how the hardware orders k within a step.
// The accumulator holds D[4 * (l >> 4) + r][l & 15] in element r.
template <typename OT>
struct Mma;

template <>
struct Mma<bf16> {
    static constexpr int KSTEP = 32;
    typedef bf16x8 frag;
    template <int ROWS, int COLS>
    __device__ __forceinline__ static frag load(const Tile<bf16, ROWS, COLS>& t, int row0, int k0,
                                                int lane) {
        return *reinterpret_cast<const frag*>(t.granule(row0 + (lane & 15), (k0 >> 3) + (lane >> 4)));
    }
    __device__ __forceinline__ static f32x4 mma(frag x, frag y, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
    }
};

template <>
struct Mma<float> {
    static constexpr int KSTEP = 4;
    typedef float frag;
    template <int ROWS, int COLS>
    __device__ __forceinline__ static frag load(const Tile<float, ROWS, COLS>& t, int row0, int k0,
                                                int lane) {
        return t.at(row0 + (lane & 15), k0 + (lane >> 4));
    }
    __device__ __forceinline__ static f32x4 mma(frag x, frag y, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, c, 0, 0, 0);
    }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Write an accumulator tile transposed: element (i, j) goes to dst[col0 + j][row0 + i].
// Each lane writes 4 consecutive elements of one destination row (8 bytes for
// bf16, 16 bytes for fp32; row0 is a multiple of 16, so they share a granule).
__device__ __forceinline__ void store4(bf16* p, f32x4 a) {
    bf16 h[4] = {(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
    *reinterpret_cast<uint2*>(p) = *reinterpret_cast<const uint2*>(h);
}
__device__ __forceinline__ void store4(float* p, f32x4 a) { *reinterpret_cast<f32x4*>(p) = a; }

template <typename OT, int ROWS, int COLS>
__device__ __forceinline__ void store_T(const Tile<OT, ROWS, COLS>& dst, int row0, int col0, f32x4 acc,
                                        int lane) {
    store4(&dst.at(col0 + (lane & 15), row0 + 4 * (lane >> 4)), acc);
}

// Write an accumulator tile in place: element (i, j) goes to dst[row0 + i][col0 + j].
template <typename OT, int ROWS, int COLS>
__device__ __forceinline__ void store_N(const Tile<OT, ROWS, COLS>& dst, int row0, int col0, f32x4 acc,
                                        int lane) {
    const int c = col0 + (lane & 15);
    const int r = row0 + 4 * (lane >> 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) dst.at(r + e, c) = from_f32<OT>(acc[e]);
}

// ---- wave reductions -------------------------------------------------------------------
// Sum over the four 16-lane groups (lanes with the same l & 15).
__device__ __forceinline__ float sum_over_groups(float x) {
    x += __shfl_xor(x, 16, kWave);
    x += __shfl_xor(x, 32, kWave);
    return x;
}

// Sum over aligned groups of `width` consecutive lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float sum_lanes(float x) {
#pragma unroll
    for (int o = 1; o < WIDTH; o <<= 1) x += __shfl_xor(x, o, kWave);
    return x;
}

}  // namespace la
