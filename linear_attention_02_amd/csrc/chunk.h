// chunk.h -- chunk staging and carried-state helpers shared by the forward and
// backward kernels.
//
// A chunk is kChunk = 64 consecutive tokens of one head.  Its [64][d] input
// tiles are read from HBM with coalesced 16-byte loads into registers one
// chunk ahead, transformed (phi, elu, 1/den), and staged row-major into
// swizzled LDS tiles; operands that contract over tokens are read back with
// the transposing LDS load.  The carried state is split around the constant
// part of phi(K) = 1 + E(K) (E = elu):
//   S = 1 P^T + S_E, z = n 1 + z_E, with P = sum V, S_E = sum E(K) V^T, z_E = sum E(K).
#pragma once

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace la {

constexpr int kC = kChunk;

// Segment record (fp32): X^T[b][a] (d*d), then two d-vectors.  Forward
// records hold (S_E, z_E, P); the backward's suffix records (R, r, w).
template <int D>
struct Rec {
    static constexpr int kSt = 0;
    static constexpr int kZ = D * D;
    static constexpr int kP = D * D + D;
    static constexpr int kSize = D * D + 2 * D;
};

// Coalesced loader of one [64][D] chunk: each thread holds NV 16-byte vectors;
// vector i covers row row(i), granule gran(i).  Rows past the head's range read as 0.
// kWaveRows = false: the block's threads cover the 64 rows in order;
// kWaveRows = true : each wavefront covers 16 rows (a token tile) from tok0.
template <typename T, int D, bool kWaveRows = false>
struct ChunkRegs {
    static constexpr int EV = 16 / (int)sizeof(T);
    static constexpr int VPR = D / EV;  // vectors per row (held by consecutive lanes)
    static_assert((kC * VPR) % kBlock == 0 && (16 * VPR) % kWave == 0, "rows must split evenly over the threads");
    static_assert(VPR <= kWave, "a row must sit inside one wavefront");
    static constexpr int ROWS = kWaveRows ? 16 : kC;
    static constexpr int NV = ROWS * VPR / (kWaveRows ? kWave : kBlock);
    __device__ __forceinline__ static int row(int i, int tid) {
        return kWaveRows ? ((tid & 63) + kWave * i) / VPR : (tid + kBlock * i) / VPR;
    }
    __device__ __forceinline__ static int gran(int i, int tid) {
        return kWaveRows ? ((tid & 63) + kWave * i) % VPR : (tid + kBlock * i) % VPR;
    }
    uint4 r[NV];
    __device__ __forceinline__ void load(const GBuf& b, int tok0, int tid) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            r[i] = b.ld16((uint32_t)((tok0 + row(i, tid)) * D + gran(i, tid) * EV) * (uint32_t)sizeof(T));
    }
    __device__ __forceinline__ float get(int i, int e) const { return to_f32(reinterpret_cast<const T*>(&r[i])[e]); }
};

// One 16-row token tile of a [N][D] input held in registers in MFMA operand
// layout: lane l holds row (l & 15), 16-byte vector x at elements (4 x + g) EV
// with g = l >> 4 -- for bf16 the k values of step 32 x, for fp32 those of the
// steps 16 x + 4 e (element e), matching Mma's k order.  Rows past the head read as 0.
template <typename T, int D>
struct RowFrag {
    using M = Mma<T>;
    static constexpr int EV = 16 / (int)sizeof(T);
    static constexpr int NR = D / (4 * EV);
    static constexpr int NF = D / M::KSTEP;
    static_assert(NR >= 1, "a row must cover the four lane groups");
    uint4 r[NR];
    __device__ __forceinline__ static int col(int x, int lane) { return (4 * x + (lane >> 4)) * EV; }
    __device__ __forceinline__ void load(const GBuf& b, int tok0, int lane) {
        const int tok = tok0 + (lane & 15);
#pragma unroll
        for (int x = 0; x < NR; ++x) r[x] = b.ld16((uint32_t)(tok * D + col(x, lane)) * (uint32_t)sizeof(T));
    }
    // f[k0 / KSTEP] = phi of the held elements as operands; returns the lane's
    // part of sum_a phi(x_a) wgt[a] (fp32 weights in LDS).
    template <class FM = FeatElu>
    __device__ __forceinline__ float phi_ops(typename M::frag* f, const float* wgt, int lane) const {
        float dot = 0.f;
#pragma unroll
        for (int x = 0; x < NR; ++x) {
            const T* h = reinterpret_cast<const T*>(&r[x]);
            const int c = col(x, lane);
            float y[EV];
#pragma unroll
            for (int e = 0; e < EV; e += 4) {
                const f32x4 wv = *reinterpret_cast<const f32x4*>(wgt + c + e);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    y[e + u] = FM::phi(to_f32(h[e + u]));
                    dot += y[e + u] * wv[u];
                }
            }
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int e = 0; e < EV; ++e) f[x][e] = (T)y[e];
            } else {
#pragma unroll
                for (int e = 0; e < EV; ++e) f[4 * x + e] = y[e];
            }
        }
        return dot;
    }
    // f[k0 / KSTEP] = phi of the held elements as operands.
    template <class FM = FeatElu>
    __device__ __forceinline__ void phi_ops(typename M::frag* f) const {
#pragma unroll
        for (int x = 0; x < NR; ++x) {
            const T* h = reinterpret_cast<const T*>(&r[x]);
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int e = 0; e < EV; ++e) f[x][e] = (T)FM::phi(to_f32(h[e]));
            } else {
#pragma unroll
                for (int e = 0; e < EV; ++e) f[4 * x + e] = FM::phi(h[e]);
            }
        }
    }
};

// One token row per lane in accumulator order: lane l holds row tok0 + (l & 15),
// elements 16 m + 4 (l >> 4) + 0..3 in word m (the order of an accumulator
// tile's rows).  Rows past the head read as 0.
template <typename T, int D>
struct RowAcc {
    typedef typename std::conditional<sizeof(T) == 2, uint2, uint4>::type word;
    static constexpr int NW = D / 16;
    word r[NW];
    __device__ __forceinline__ void load(const GBuf& b, int tok0, int lane) {
        const uint32_t base = (uint32_t)((tok0 + (lane & 15)) * D + 4 * (lane >> 4)) * (uint32_t)sizeof(T);
#pragma unroll
        for (int m = 0; m < NW; ++m) {
            if constexpr (sizeof(T) == 2) r[m] = b.ld8(base + 32 * m);
            else r[m] = b.ld16(base + 64 * m);
        }
    }
    __device__ __forceinline__ float get(int i) const { return to_f32(reinterpret_cast<const T*>(r)[i]); }
};

// Direct-to-LDS fill of a swizzled [64][D] tile from rows tok0.. of a head: each
// wavefront issues PER_WAVE buffer loads whose 64 lanes land 16 bytes apiece on
// consecutive LDS granules; the global address of each lane is chosen so that
// the granule lands at its swizzled place.  Rows past the head's range fill
// with zeros and move no bytes.  Completion is tracked by the vector-memory
// count (PER_WAVE per tile per wavefront).
typedef __attribute__((address_space(3))) void lds_void;
template <typename T, int D>
struct TileDma {
    static constexpr int EV = 16 / (int)sizeof(T);
    static constexpr int G = D / EV;
    static constexpr int PER_WAVE = kC * G / (kWave * (kBlock / kWave));
    static_assert(PER_WAVE >= 1 && kC * G % kBlock == 0, "a tile must split evenly over the wavefronts");
    __device__ __forceinline__ static void issue(const GBuf& b, int tok0, T* tile, int w, int lane) {
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int slot0 = (w * PER_WAVE + i) * kWave;
            const int sl = slot0 + lane;
            const int r = sl / G, p = sl % G;
            const int gi = p ^ Tile<T, kC, D>::swz(r);
            const uint32_t off = (uint32_t)((tok0 + r) * D + gi * EV) * (uint32_t)sizeof(T);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(b.r, (lds_void*)(tile + slot0 * EV), 16, off, 0, 0, 0);
        }
    }
};

// phi(Q) row-major into LDS (phi of the feature map FM).
// (kWaveRows: the wavefront's rows go to tile rows row0 ..)
template <typename T, int D, bool kWaveRows = false, class FM = FeatElu>
__device__ __forceinline__ void stage_phi(const ChunkRegs<T, D, kWaveRows>& cq, const Tile<T, kC, D>& tQ, int tid,
                                          int row0 = 0) {
    using CR = ChunkRegs<T, D, kWaveRows>;
#pragma unroll
    for (int i = 0; i < CR::NV; ++i) {
        uint4 packed;
        T* pk = reinterpret_cast<T*>(&packed);
#pragma unroll
        for (int e = 0; e < CR::EV; ++e) pk[e] = from_f32<T>(FM::phi(cq.get(i, e)));
        *reinterpret_cast<uint4*>(tQ.granule(row0 + CR::row(i, tid), CR::gran(i, tid))) = packed;
    }
}

// E(K) = phi(K) - 1 (elu(K) for the default map) row-major into LDS.
template <typename T, int D, class FM = FeatElu>
__device__ __forceinline__ void stage_elu(const ChunkRegs<T, D>& ck, const Tile<T, kC, D>& tE, int tid) {
    using CR = ChunkRegs<T, D>;
#pragma unroll
    for (int i = 0; i < CR::NV; ++i) {
        uint4 packed;
        T* pk = reinterpret_cast<T*>(&packed);
#pragma unroll
        for (int e = 0; e < CR::EV; ++e) pk[e] = from_f32<T>(FM::e(ck.get(i, e)));
        *reinterpret_cast<uint4*>(tE.granule(CR::row(i, tid), CR::gran(i, tid))) = packed;
    }
}

// A raw chunk row-major into LDS.
template <typename T, int D>
__device__ __forceinline__ void stage_raw(const ChunkRegs<T, D>& cx, const Tile<T, kC, D>& tX, int tid) {
    using CR = ChunkRegs<T, D>;
#pragma unroll
    for (int i = 0; i < CR::NV; ++i) *reinterpret_cast<uint4*>(tX.granule(CR::row(i, tid), CR::gran(i, tid))) = cx.r[i];
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
    // The d-vector tiles a wave owns (vector index = tile of 16): the wave whose
    // tiles start a row block owns that block's vector tiles.
    static constexpr int NVT = DT >= 4 ? DT / 4 : 1;
    __device__ __forceinline__ static bool owns_vec(int w) { return DT >= 4 || (w % (4 / DT)) == 0; }
    __device__ __forceinline__ static int vt0(int w) { return DT >= 4 ? w * (DT / 4) : w / (4 / DT); }
};

template <int D>
using StateAcc = f32x4[StateTiles<D>::NAT][StateTiles<D>::NBT];
template <int D>
using VecAcc = f32x4[StateTiles<D>::NVT];

// Offset of the lane's 4 values of state tile (a-tile at, b-tile bt) inside a
// record's transposed d x d block X^T[b][a].
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
__device__ __forceinline__ void zero_vec(VecAcc<D>& v) {
#pragma unroll
    for (int x = 0; x < StateTiles<D>::NVT; ++x) v[x] = zero4();
}

template <int D>
__device__ __forceinline__ void load_state(const float* r, StateAcc<D>& st, int lane, int w) {
    using ST = StateTiles<D>;
#pragma unroll
    for (int ia = 0; ia < ST::NAT; ++ia)
#pragma unroll
        for (int ib = 0; ib < ST::NBT; ++ib)
            st[ia][ib] = *reinterpret_cast<const f32x4*>(r + rec_st_off<D>(ST::at0(w) + ia, ST::bt0(w) + ib, lane));
}

template <int D>
__device__ __forceinline__ void store_state(float* r, const StateAcc<D>& st, int lane, int w) {
    using ST = StateTiles<D>;
#pragma unroll
    for (int ia = 0; ia < ST::NAT; ++ia)
#pragma unroll
        for (int ib = 0; ib < ST::NBT; ++ib)
            *reinterpret_cast<f32x4*>(r + rec_st_off<D>(ST::at0(w) + ia, ST::bt0(w) + ib, lane)) = st[ia][ib];
}

// Vector accumulators hold v[tile*16 + 4 (l >> 4) + e] in every column; the
// accumulator layout is the MFMA output of X (rows = vector index) times a
// constant operand.
template <int D>
__device__ __forceinline__ void load_vec(const float* v, VecAcc<D>& acc, int lane, int w) {
    using ST = StateTiles<D>;
#pragma unroll
    for (int x = 0; x < ST::NVT; ++x) acc[x] = *reinterpret_cast<const f32x4*>(v + (ST::vt0(w) + x) * 16 + 4 * (lane >> 4));
}

template <int D>
__device__ __forceinline__ void store_vec(float* v, const VecAcc<D>& acc, int lane, int w) {
    using ST = StateTiles<D>;
    if (!ST::owns_vec(w) || (lane & 15) != 0) return;
#pragma unroll
    for (int x = 0; x < ST::NVT; ++x) *reinterpret_cast<f32x4*>(v + (ST::vt0(w) + x) * 16 + 4 * (lane >> 4)) = acc[x];
}

// The same vector tiles rounded to T (operand copies of a vector).
template <typename T, int D>
__device__ __forceinline__ void store_vec_as(T* v, const VecAcc<D>& acc, int lane, int w) {
    using ST = StateTiles<D>;
    if (!ST::owns_vec(w) || (lane & 15) != 0) return;
#pragma unroll
    for (int x = 0; x < ST::NVT; ++x) store4(v + (ST::vt0(w) + x) * 16 + 4 * (lane >> 4), acc[x]);
}

// Sources of segment records (indices in floats from the source's base): plain
// loads through a pointer, or agent-coherent loads through a buffer resource
// (records that other workgroups of the same launch are publishing).
struct RecPtr {
    const float* p;
    __device__ __forceinline__ f32x4 ld4(int64_t i) const { return *reinterpret_cast<const f32x4*>(p + i); }
};
struct RecCoherent {
    GBuf b;
    __device__ __forceinline__ f32x4 ld4(int64_t i) const { return b.ld16c((uint32_t)(i * 4)); }
};

// Add the segment records at base + j * stride of src for j = 0 .. count-1, in
// that order, to the wave's state tiles and vector tiles (fixed order: bitwise
// reproducible).  kRegs: registers the records in flight may take (at most 8
// records per batch).  kVecB false: the records' second vector is not read (vb is
// left as it is), so that more records fit a batch.  ready(j0, j1), called by the
// wave before records j0 .. j1-1 are read (it may wait for them), lets the first
// batches be summed while later records are still being produced.
template <int D, int kRegs, bool kVecB = true, typename Src, typename Ready>
__device__ __forceinline__ void add_records_from(const Src& src, int64_t base, int64_t stride, int count,
                                                 StateAcc<D>& st, VecAcc<D>& va, VecAcc<D>& vb, int lane, int w,
                                                 Ready&& ready) {
    using ST = StateTiles<D>;
    constexpr int PER_REC = 4 * (ST::NAT * ST::NBT + (kVecB ? 2 : 1) * ST::NVT);
    constexpr int B = kRegs / PER_REC >= 8 ? 8 : kRegs / PER_REC >= 1 ? kRegs / PER_REC : 1;
    for (int j0 = 0; j0 < count; j0 += B) {
        ready(j0, j0 + B < count ? j0 + B : count);
        f32x4 xs[B][ST::NAT][ST::NBT], xa[B][ST::NVT], xb[B][ST::NVT];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (j0 + b < count) {
                const int64_t r = base + (int64_t)(j0 + b) * stride;
#pragma unroll
                for (int ia = 0; ia < ST::NAT; ++ia)
#pragma unroll
                    for (int ib = 0; ib < ST::NBT; ++ib)
                        xs[b][ia][ib] = src.ld4(r + rec_st_off<D>(ST::at0(w) + ia, ST::bt0(w) + ib, lane));
#pragma unroll
                for (int x = 0; x < ST::NVT; ++x) {
                    const int o = (ST::vt0(w) + x) * 16 + 4 * (lane >> 4);
                    xa[b][x] = src.ld4(r + Rec<D>::kZ + o);
                    if constexpr (kVecB) xb[b][x] = src.ld4(r + Rec<D>::kP + o);
                }
            }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (j0 + b < count) {
#pragma unroll
                for (int ia = 0; ia < ST::NAT; ++ia)
#pragma unroll
                    for (int ib = 0; ib < ST::NBT; ++ib) st[ia][ib] += xs[b][ia][ib];
#pragma unroll
                for (int x = 0; x < ST::NVT; ++x) {
                    va[x] += xa[b][x];
                    if constexpr (kVecB) vb[x] += xb[b][x];
                }
            }
        }
    }
}

template <int D, int kRegs, bool kVecB = true, typename Src>
__device__ __forceinline__ void add_records_from(const Src& src, int64_t base, int64_t stride, int count,
                                                 StateAcc<D>& st, VecAcc<D>& va, VecAcc<D>& vb, int lane, int w) {
    add_records_from<D, kRegs, kVecB>(src, base, stride, count, st, va, vb, lane, w, [](int, int) {});
}

// The same for records read through a plain pointer: rec[j * stride], j = 0 .. count-1.
template <int D, int kRegs = 192, bool kVecB = true>
__device__ __forceinline__ void add_records(const float* rec, int64_t stride, int count, StateAcc<D>& st,
                                            VecAcc<D>& va, VecAcc<D>& vb, int lane, int w) {
    add_records_from<D, kRegs, kVecB>(RecPtr{rec}, 0, stride, count, st, va, vb, lane, w);
}

// init + the records at base + j * stride of src for j = 0 .. count-1, element by
// element in that order (bitwise what add_records_from forms), by all kThreads
// threads of the workgroup at once, into out (kSize floats, record layout; LDS).
// Every thread keeps a few 16-byte granules of every record of a batch in flight,
// so a batch costs one round trip whatever the number of waves that will use it.
// init (nullable): a record the sum starts from.  ready(j0, j1), called by every
// thread before records j0 .. j1-1 are read (it may wait for them and hold a barrier),
// lets the first batches be summed while later records are still being produced.
template <int D, int kThreads, typename Src, typename Ready>
__device__ __forceinline__ void sum_records_to(const Src& src, int64_t base, int64_t stride, int count,
                                               const float* init, float* out, int tid, Ready&& ready) {
    constexpr int G4 = Rec<D>::kSize / 4;  // 16-byte granules of a record
    static_assert(Rec<D>::kSize % 4 == 0, "records are whole granules");
    constexpr int PER = (G4 + kThreads - 1) / kThreads;
    constexpr int RB = PER <= 2 ? 8 : PER <= 4 ? 4 : 2;  // records per batch
    f32x4 acc[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int g = tid + p * kThreads;
        acc[p] = init != nullptr && g < G4 ? *reinterpret_cast<const f32x4*>(init + 4 * g) : zero4();
    }
    for (int j0 = 0; j0 < count; j0 += RB) {
        ready(j0, j0 + RB < count ? j0 + RB : count);
        f32x4 x[RB][PER];
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                const int g = tid + p * kThreads;
                x[b][p] = j0 + b < count && g < G4 ? src.ld4(base + (int64_t)(j0 + b) * stride + 4 * g) : zero4();
            }
#pragma unroll
        for (int b = 0; b < RB; ++b)
            if (j0 + b < count) {
#pragma unroll
                for (int p = 0; p < PER; ++p) acc[p] += x[b][p];
            }
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int g = tid + p * kThreads;
        if (g < G4) *reinterpret_cast<f32x4*>(out + 4 * g) = acc[p];
    }
}

template <int D, int kThreads, typename Src>
__device__ __forceinline__ void sum_records_to(const Src& src, int64_t base, int64_t stride, int count,
                                               const float* init, float* out, int tid) {
    sum_records_to<D, kThreads>(src, base, stride, count, init, out, tid, [](int, int) {});
}

// One record [X^T | a | b] written with agent-coherent stores through b at float
// index base (b = zeros when vb is null).
template <int D>
__device__ __forceinline__ void store_record_coherent(const GBuf& buf, int64_t base, const StateAcc<D>& st,
                                                      const VecAcc<D>& va, const VecAcc<D>* vb, int lane, int w) {
    using ST = StateTiles<D>;
#pragma unroll
    for (int ia = 0; ia < ST::NAT; ++ia)
#pragma unroll
        for (int ib = 0; ib < ST::NBT; ++ib)
            buf.st16c((uint32_t)((base + rec_st_off<D>(ST::at0(w) + ia, ST::bt0(w) + ib, lane)) * 4), st[ia][ib]);
    if (!ST::owns_vec(w) || (lane & 15) != 0) return;
#pragma unroll
    for (int x = 0; x < ST::NVT; ++x) {
        const int o = (ST::vt0(w) + x) * 16 + 4 * (lane >> 4);
        buf.st16c((uint32_t)((base + Rec<D>::kZ + o) * 4), va[x]);
        buf.st16c((uint32_t)((base + Rec<D>::kP + o) * 4), vb != nullptr ? (*vb)[x] : zero4());
    }
}

// Rounded copy of the state into LDS as X^T[b][a].
// The state carried into a segment from records[0 .. count-1] at first + j * stride.
// prefixed: a scan has already replaced each record by the running sum of the
// ones before it (same order), so the record at first + count * stride is that
// sum; otherwise the records are added here.  Either way the result is bitwise
// the same.  init (nullable): a record the sum starts from (a scan starts from
// it too, so a prefixed record already holds it).
template <int D, int kRegs = 192, bool kVecB = true>
__device__ __forceinline__ void carried_state(const float* first, int64_t stride, int count, bool prefixed,
                                              StateAcc<D>& st, VecAcc<D>& va, VecAcc<D>& vb, int lane, int w,
                                              const float* init = nullptr) {
    if (prefixed) {
        const float* r = first + (int64_t)count * stride;
        load_state<D>(r, st, lane, w);
        load_vec<D>(r + Rec<D>::kZ, va, lane, w);
        load_vec<D>(r + Rec<D>::kP, vb, lane, w);
    } else {
        if (init != nullptr) {
            load_state<D>(init, st, lane, w);
            load_vec<D>(init + Rec<D>::kZ, va, lane, w);
            load_vec<D>(init + Rec<D>::kP, vb, lane, w);
        } else {
            zero_state<D>(st);
            zero_vec<D>(va);
            zero_vec<D>(vb);
        }
        add_records<D, kRegs, kVecB>(first, stride, count, st, va, vb, lane, w);
    }
}

template <typename T, int D, bool A>
__device__ __forceinline__ void publish_state(const StateAcc<D>& st, const Tile<T, D, D, A>& tXt, int lane, int w) {
    using ST = StateTiles<D>;
#pragma unroll
    for (int ia = 0; ia < ST::NAT; ++ia)
#pragma unroll
        for (int ib = 0; ib < ST::NBT; ++ib)
            store_T(tXt, (ST::at0(w) + ia) * 16, (ST::bt0(w) + ib) * 16, st[ia][ib], lane);
}

// st[a][b] += sum_t X[t][a] Y[t][b] over the chunk, X and Y row-major [64][D]
// tiles read with the transposing load; optionally
// va[a] += sum_t X[t][a] * u[t] and vb[b] += sum_t Y[t][b] * v[t] for the
// wave's vector tiles, with u, v either all ones (null pointer) or fp32
// vectors in LDS (split hi + lo in bf16).  The vector tiles a wave owns are
// its own row tiles, so va reuses the X operands.  kEluX: X holds raw keys and
// the operands are E(X) = phi(X) - 1 of the feature map FM, applied after the load.
template <typename T, int D, bool kVecA, bool kVecB, bool kEluX = false, class FM = FeatElu>
__device__ __forceinline__ void state_update(StateAcc<D>& st, VecAcc<D>& va, VecAcc<D>& vb, const Tile<T, kC, D>& tX,
                                             const Tile<T, kC, D>& tY, const float* u, const float* v, int lane,
                                             int w) {
    using M = Mma<T>;
    using ST = StateTiles<D>;
    static_assert(ST::NVT == ST::NAT, "a wave's vector tiles are its row tiles");
    typedef typename M::frag F;
    // All LDS operands of a group of KG k-steps are requested before the first
    // MFMA, so the LDS latency is paid once per group rather than once per product.
    constexpr int FR = (int)(sizeof(F) / 4);
    constexpr int PER_K = ST::NAT + ST::NBT + (kVecB ? ST::NVT : 0);
    constexpr int KSTEPS = kC / M::KSTEP;
    constexpr int KG0 = 48 / (PER_K * FR) > 0 ? 48 / (PER_K * FR) : 1;
    constexpr int KG1 = KG0 < KSTEPS ? KG0 : KSTEPS;
    constexpr int KG = KG1 >= 16 ? 16 : KG1 >= 8 ? 8 : KG1 >= 4 ? 4 : KG1 >= 2 ? 2 : 1;  // a power of two
    static_assert(KSTEPS % KG == 0, "k-step groups must tile the chunk");
    const F one = M::ones();
#pragma unroll
    for (int kg = 0; kg < KSTEPS; kg += KG) {
        F xf[KG][ST::NAT], yf[KG][ST::NBT], yv[KG][kVecB ? ST::NVT : 1];
#pragma unroll
        for (int kk = 0; kk < KG; ++kk) {
            const int k0 = (kg + kk) * M::KSTEP;
#pragma unroll
            for (int ia = 0; ia < ST::NAT; ++ia) xf[kk][ia] = M::ld_tr(tX, k0, (ST::at0(w) + ia) * 16, lane);
#pragma unroll
            for (int ib = 0; ib < ST::NBT; ++ib) yf[kk][ib] = M::ld_tr(tY, k0, (ST::bt0(w) + ib) * 16, lane);
            if (kVecB && ST::owns_vec(w)) {
#pragma unroll
                for (int x = 0; x < ST::NVT; ++x) yv[kk][x] = M::ld_tr(tY, k0, (ST::vt0(w) + x) * 16, lane);
            }
        }
#pragma unroll
        for (int kk = 0; kk < KG; ++kk) {
            const int k0 = (kg + kk) * M::KSTEP;
            if (kEluX) {
#pragma unroll
                for (int ia = 0; ia < ST::NAT; ++ia) xf[kk][ia] = M::template elu_op<FM>(xf[kk][ia]);
            }
#pragma unroll
            for (int ib = 0; ib < ST::NBT; ++ib)
#pragma unroll
                for (int ia = 0; ia < ST::NAT; ++ia) st[ia][ib] = M::mma(xf[kk][ia], yf[kk][ib], st[ia][ib]);
            if (ST::owns_vec(w)) {
                if (kVecA) {
                    F hi = one, lo = one;
                    if (u != nullptr) M::splat(u, k0, lane, hi, lo);
#pragma unroll
                    for (int x = 0; x < ST::NVT; ++x) {
                        va[x] = M::mma(xf[kk][x], hi, va[x]);
                        if (M::kSplitSplat && u != nullptr) va[x] = M::mma(xf[kk][x], lo, va[x]);
                    }
                }
                if (kVecB) {
                    F hi = one, lo = one;
                    if (v != nullptr) M::splat(v, k0, lane, hi, lo);
#pragma unroll
                    for (int x = 0; x < ST::NVT; ++x) {
                        vb[x] = M::mma(yv[kk][x], hi, vb[x]);
                        if (M::kSplitSplat && v != nullptr) vb[x] = M::mma(yv[kk][x], lo, vb[x]);
                    }
                }
            }
        }
    }
}

// q_sum_t = sum_a phi(Q)[t][a] for the token tile t0.. as an MFMA against a
// ones operand: every element of the returned accumulator column t holds q_sum_t.
template <typename T, int D>
__device__ __forceinline__ f32x4 tile_row_sums(const Tile<T, kC, D>& tQ, int t0, int lane) {
    using M = Mma<T>;
    const typename M::frag one = M::ones();
    f32x4 acc = zero4();
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += M::KSTEP) acc = M::mma(one, M::ld(tQ, t0, k0, lane), acc);
    return acc;
}

// phi(Q_t) . wgt over all d features for token row t: each 16-lane group
// covers a quarter of the features; the result is summed over the groups.
template <typename T, int D>
__device__ __forceinline__ float row_dot_quarters(const Tile<T, kC, D>& tQ, const float* wgt, int t, int lane) {
    constexpr int EV = Tile<T, kC, D>::EV;
    constexpr int GPQ = D / 4 / EV;
    static_assert(GPQ >= 1, "a quarter of the features must be whole granules");
    const int g = lane >> 4;
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < GPQ; ++x) {
        const int gi = g * GPQ + x;
        const uint4 raw = *reinterpret_cast<const uint4*>(tQ.granule(t, gi));
        const T* p = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int e = 0; e < EV; ++e) s += to_f32(p[e]) * wgt[gi * EV + e];
    }
    return sum_over_groups(s);
}

// 4 consecutive elements of a head's row at element offset `elem`, rounded to T.
template <typename T>
__device__ __forceinline__ void gstore4(const GBuf& b, uint32_t elem, f32x4 a) {
    if constexpr (sizeof(T) == 2) {
        bf16 h[4] = {(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
        b.st8(elem * 2, *reinterpret_cast<const uint2*>(h));
    } else {
        b.st16(elem * 4, make_uint4(__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]), __float_as_uint(a[3])));
    }
}

}  // namespace la
