// chunk.h -- chunk staging and state helpers shared by the forward and backward kernels.
//
// A chunk is C consecutive tokens of one head (C = 64, or 32 where LDS is
// short).  Its [C][d] input tiles are read from HBM with coalesced 16-byte
// loads into registers one chunk ahead, then staged into swizzled LDS tiles
// (row-major and/or transposed) for the MFMA products.  The carried state is
// split around the constant part of phi(K) = 1 + E(K) (E = elu):
//   S = 1 P^T + S_E, z = n 1 + z_E with P = sum V, S_E = sum E(K) V^T, z_E = sum E(K).
#pragma once

#include "common.h"
#include "launch.h"

namespace la {

// Segment record (fp32): S_E^T[b][a] (d*d), then z_E[a] (d), then P[b] (d).
// The backward's suffix records use the same layout for R^T, r and w.
template <int D>
struct Rec {
    static constexpr int kSt = 0;
    static constexpr int kZ = D * D;
    static constexpr int kP = D * D + D;
    static constexpr int kSize = D * D + 2 * D;
};

// Coalesced loader of one [C][D] chunk: each thread holds NV 16-byte vectors;
// vector i covers row row(i), granule gran(i).  Rows at or beyond N read as 0.
template <typename T, int D, int C>
struct ChunkRegs {
    static constexpr int EV = 16 / (int)sizeof(T);
    static constexpr int VPR = D / EV;  // vectors per row (held by consecutive lanes)
    static constexpr int NV = C * VPR / kBlock;
    static_assert(NV >= 1 && (C * VPR) % kBlock == 0, "chunk must split evenly over the block");
    static_assert(VPR <= kWave, "a row must sit inside one wavefront");
    uint4 r[NV];
    __device__ __forceinline__ static int row(int i, int tid) { return (tid + kBlock * i) / VPR; }
    __device__ __forceinline__ static int gran(int i, int tid) { return (tid + kBlock * i) % VPR; }
    __device__ __forceinline__ void load(const T* head, int tok0, int N, int tid) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int tok = tok0 + row(i, tid);
            r[i] = tok < N ? load16(head + (int64_t)tok * D + gran(i, tid) * EV) : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ float get(int i, int e) const {
        return to_f32(reinterpret_cast<const T*>(&r[i])[e]);
    }
    __device__ __forceinline__ T raw(int i, int e) const { return reinterpret_cast<const T*>(&r[i])[e]; }
};

// Stage phi(Q) row-major (and optionally transposed) and the row sums q_sum_t
// of the values as rounded for the MFMA.
template <typename T, int D, int C, bool kTransposed>
__device__ __forceinline__ void stage_q(const ChunkRegs<T, D, C>& cq, const Tile<T, C, D>& tQf,
                                        const Tile<T, D, C>& tQft, float* s_qsum, int tid) {
    using CR = ChunkRegs<T, D, C>;
#pragma unroll
    for (int i = 0; i < CR::NV; ++i) {
        const int t = CR::row(i, tid), gi = CR::gran(i, tid);
        uint4 packed;
        T* pk = reinterpret_cast<T*>(&packed);
        float qs = 0.f;
#pragma unroll
        for (int e = 0; e < CR::EV; ++e) {
            const T f = from_f32<T>(phi_f(cq.get(i, e)));
            pk[e] = f;
            qs += to_f32(f);
            if (kTransposed) tQft.at(gi * CR::EV + e, t) = f;
        }
        *reinterpret_cast<uint4*>(tQf.granule(t, gi)) = packed;
        qs = sum_lanes<CR::VPR>(qs);
        if (gi == 0) s_qsum[t] = qs;
    }
}

// Stage E(K) = elu(K) row-major and/or transposed.
template <typename T, int D, int C, bool kRow, bool kTransposed>
__device__ __forceinline__ void stage_e(const ChunkRegs<T, D, C>& ck, const Tile<T, C, D>& tEk,
                                        const Tile<T, D, C>& tEkt, int tid) {
    using CR = ChunkRegs<T, D, C>;
#pragma unroll
    for (int i = 0; i < CR::NV; ++i) {
        const int t = CR::row(i, tid), gi = CR::gran(i, tid);
        uint4 packed;
        T* pk = reinterpret_cast<T*>(&packed);
#pragma unroll
        for (int e = 0; e < CR::EV; ++e) {
            const T ev = from_f32<T>(elu_f(ck.get(i, e)));
            pk[e] = ev;
            if (kTransposed) tEkt.at(gi * CR::EV + e, t) = ev;
        }
        if (kRow) *reinterpret_cast<uint4*>(tEk.granule(t, gi)) = packed;
    }
}

// Stage a raw input chunk row-major and/or transposed.
template <typename T, int D, int C, bool kRow, bool kTransposed>
__device__ __forceinline__ void stage_raw(const ChunkRegs<T, D, C>& cx, const Tile<T, C, D>& tX,
                                          const Tile<T, D, C>& tXt, int tid) {
    using CR = ChunkRegs<T, D, C>;
#pragma unroll
    for (int i = 0; i < CR::NV; ++i) {
        const int t = CR::row(i, tid), gi = CR::gran(i, tid);
        if (kTransposed) {
#pragma unroll
            for (int e = 0; e < CR::EV; ++e) tXt.at(gi * CR::EV + e, t) = cx.raw(i, e);
        }
        if (kRow) *reinterpret_cast<uint4*>(tX.granule(t, gi)) = cx.r[i];
    }
}

// Sum of one row of an LDS tile, in fixed order.
template <typename T, int ROWS, int COLS>
__device__ __forceinline__ float row_sum(const Tile<T, ROWS, COLS>& t, int r) {
    constexpr int EV = Tile<T, ROWS, COLS>::EV;
    float s = 0.f;
#pragma unroll
    for (int gi = 0; gi < COLS / EV; ++gi) {
        const uint4 g = *reinterpret_cast<const uint4*>(t.granule(r, gi));
        const T* p = reinterpret_cast<const T*>(&g);
#pragma unroll
        for (int e = 0; e < EV; ++e) s += to_f32(p[e]);
    }
    return s;
}

// Weighted sum of one row of an LDS tile: sum_c t[r][c] * wgt[c], fixed order.
template <typename T, int ROWS, int COLS>
__device__ __forceinline__ float row_dot(const Tile<T, ROWS, COLS>& t, int r, const float* wgt) {
    constexpr int EV = Tile<T, ROWS, COLS>::EV;
    float s = 0.f;
#pragma unroll
    for (int gi = 0; gi < COLS / EV; ++gi) {
        const uint4 g = *reinterpret_cast<const uint4*>(t.granule(r, gi));
        const T* p = reinterpret_cast<const T*>(&g);
#pragma unroll
        for (int e = 0; e < EV; ++e) s += to_f32(p[e]) * wgt[gi * EV + e];
    }
    return s;
}

// Tiles of a d x d state owned by one of the 4 wavefronts: NAT row tiles
// (features a) from at0, NBT column tiles (values b) from bt0.
template <int D>
struct StateTiles {
    static constexpr int DT = D / 16;
    static constexpr int TPW = DT * DT / 4;
    static constexpr int NAT = TPW >= DT ? TPW / DT : 1;
    static constexpr int NBT = TPW >= DT ? DT : TPW;
    __device__ __forceinline__ static int at0(int w) { return (w * TPW) / DT; }
    __device__ __forceinline__ static int bt0(int w) { return (w * TPW) % DT; }
};

template <int D>
using StateAcc = f32x4[StateTiles<D>::NAT][StateTiles<D>::NBT];

// The lane's 4 values of state tile (a-tile at, b-tile bt) inside a record's
// transposed d x d block X^T[b][a].
template <int D>
__device__ __forceinline__ int rec_st_off(int at, int bt, int lane) {
    return (bt * 16 + (lane & 15)) * D + at * 16 + 4 * (lane >> 4);
}

template <int D>
__device__ __forceinline__ void zero_state(StateAcc<D>& st) {
#pragma unroll
    for (int ia = 0; ia < StateTiles<D>::NAT; ++ia)
#pragma unroll
        for (int ib = 0; ib < StateTiles<D>::NBT; ++ib) st[ia][ib] = zero4();
}

template <int D>
__device__ __forceinline__ void load_state_acc(const float* r, StateAcc<D>& st, int lane, int w) {
    using ST = StateTiles<D>;
#pragma unroll
    for (int ia = 0; ia < ST::NAT; ++ia)
#pragma unroll
        for (int ib = 0; ib < ST::NBT; ++ib)
            st[ia][ib] = *reinterpret_cast<const f32x4*>(r + rec_st_off<D>(ST::at0(w) + ia, ST::bt0(w) + ib, lane));
}

template <int D>
__device__ __forceinline__ void store_state_acc(float* r, const StateAcc<D>& st, int lane, int w) {
    using ST = StateTiles<D>;
#pragma unroll
    for (int ia = 0; ia < ST::NAT; ++ia)
#pragma unroll
        for (int ib = 0; ib < ST::NBT; ++ib)
            *reinterpret_cast<f32x4*>(r + rec_st_off<D>(ST::at0(w) + ia, ST::bt0(w) + ib, lane)) = st[ia][ib];
}

// Rounded copies of the state in LDS: X^T[b][a] (transposed) and/or X[a][b].
template <typename T, int D, bool kT, bool kN>
__device__ __forceinline__ void publish_state(const StateAcc<D>& st, const Tile<T, D, D>& tXt,
                                              const Tile<T, D, D>& tX, int lane, int w) {
    using ST = StateTiles<D>;
#pragma unroll
    for (int ia = 0; ia < ST::NAT; ++ia)
#pragma unroll
        for (int ib = 0; ib < ST::NBT; ++ib) {
            const int a0 = (ST::at0(w) + ia) * 16, b0 = (ST::bt0(w) + ib) * 16;
            if (kT) store_T(tXt, a0, b0, st[ia][ib], lane);
            if (kN) store_N(tX, a0, b0, st[ia][ib], lane);
        }
}

// acc += X^T Y over k in [k0, k1) for the wave's state tiles, X^T from tX
// (rows a, k contiguous) and Y from tY (rows b, k contiguous).
template <typename T, int D, int R, int K>
__device__ __forceinline__ void state_mma(StateAcc<D>& st, const Tile<T, R, K>& tX, const Tile<T, R, K>& tY,
                                          int lane, int w) {
    using M = Mma<T>;
    using ST = StateTiles<D>;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += M::KSTEP) {
        typename M::frag xf[ST::NAT];
#pragma unroll
        for (int ia = 0; ia < ST::NAT; ++ia) xf[ia] = M::load(tX, (ST::at0(w) + ia) * 16, k0, lane);
#pragma unroll
        for (int ib = 0; ib < ST::NBT; ++ib) {
            const typename M::frag yf = M::load(tY, (ST::bt0(w) + ib) * 16, k0, lane);
#pragma unroll
            for (int ia = 0; ia < ST::NAT; ++ia) st[ia][ib] = M::mma(xf[ia], yf, st[ia][ib]);
        }
    }
}

// phi(Q_t) . wgt over all d features for the lane's token row t (each 16-lane
// group covers a quarter of the features; the result is summed over groups).
template <typename T, int D, int C>
__device__ __forceinline__ float row_dot_quarters(const Tile<T, C, D>& tQf, const float* wgt, int t, int lane) {
    constexpr int EV = Tile<T, C, D>::EV;
    constexpr int GPQ = D / 4 / EV;
    static_assert(GPQ >= 1, "a quarter of the features must be whole granules");
    const int g = lane >> 4;
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < GPQ; ++x) {
        const int gi = g * GPQ + x;
        const uint4 raw = *reinterpret_cast<const uint4*>(tQf.granule(t, gi));
        const T* p = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int e = 0; e < EV; ++e) s += to_f32(p[e]) * wgt[gi * EV + e];
    }
    return sum_over_groups(s);
}

// Store / load 4 consecutive elements of a global row.
__device__ __forceinline__ void gstore4(float* p, f32x4 a) { *reinterpret_cast<f32x4*>(p) = a; }
__device__ __forceinline__ void gstore4(bf16* p, f32x4 a) {
    bf16 h[4] = {(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
    *reinterpret_cast<uint2*>(p) = *reinterpret_cast<const uint2*>(h);
}
__device__ __forceinline__ f32x4 gload4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 gload4(const bf16* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    const bf16* h = reinterpret_cast<const bf16*>(&u);
    return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}
// 4 consecutive elements of an LDS tile row as fp32.
template <typename T, int R, int K>
__device__ __forceinline__ f32x4 lds_load4(const Tile<T, R, K>& t, int r, int c) {
    const T* p = &t.at(r, c);
    return f32x4{to_f32(p[0]), to_f32(p[1]), to_f32(p[2]), to_f32(p[3])};
}

// Fragment of the lower-triangular ones matrix L[t][s] = (s <= t) for MFMA
// operand row t (lane & 15 of the tile at row0) and k-step k0.
template <typename T>
struct OnesFrag;
template <>
struct OnesFrag<bf16> {
    __device__ __forceinline__ static bf16x8 lower(int t, int k0, int lane) {
        const int s0 = k0 + 8 * (lane >> 4);
        bf16x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (bf16)(s0 + e <= t ? 1.f : 0.f);
        return f;
    }
};
template <>
struct OnesFrag<float> {
    __device__ __forceinline__ static float lower(int t, int k0, int lane) {
        return (k0 + (lane >> 4)) <= t ? 1.f : 0.f;
    }
};

}  // namespace la
