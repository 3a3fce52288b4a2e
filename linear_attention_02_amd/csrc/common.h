// common.h -- device helpers shared by the gfx950 linear-attention kernels.
//
// Written for CDNA4 (gfx950): 64-lane wavefronts, v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x4_f32, LDS tiles with an XOR swizzle on 16-byte granules,
// and the transposing LDS load ds_read_b64_tr_b16 for operands whose
// contraction index runs along the tile's rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Wave index as a wave-uniform (scalar) value, so branches on it are scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// LDS writes of this wave become visible to this wave's later LDS reads
// (LDS requests of one wave complete in order; this only stops the compiler
// from reordering across the point and drains the queue).
__device__ __forceinline__ void wave_lds_sync() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- scalar conversions ------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // round to nearest even

// ---- feature map phi(x) = elu(x) + 1 -------------------------------------------------
// phi(x) = x + 1 (x > 0), exp(x) (x <= 0);  E(x) = phi(x) - 1 = elu(x);
// phi'(x) = 1 (x > 0), exp(x) (x <= 0).
// With c(x) = min(exp(x), 1) = exp(min(x, 0)), one exp whose result the hardware
// clamps to [0, 1]: phi'(x) = c(x), and since exp(x) >= 1 + x everywhere and
// c(x) = 1 for x > 0, phi(x) = max(x + 1, c(x)) and E(x) = max(x, c(x) - 1).
// Each costs four VALU operations (mul, exp, add, max) and no compare or select.
// NaN propagates: the maxima are IEEE maximum (v_maximum3_f32, NaN if either
// operand is NaN, same cost as v_max), so phi(NaN) = E(NaN) = NaN even though the
// clamp turns exp(NaN) into 0.  phi(-inf) = 0, E(-inf) = -1, phi(+inf) = +inf.
__device__ __forceinline__ float expc_f(float x) {
    return __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(x * 1.4426950408889634f), 0.f, 1.f);
}
// c(x) as exp(min(x, 0)) without the clamp: NaN for NaN (one more VALU operation),
// 0 for -inf, 1 for +inf.  For phi'(x) where nothing else carries a NaN of x.
__device__ __forceinline__ float expn_f(float x) {
    return __builtin_amdgcn_exp2f(__builtin_elementwise_minimum(x * 1.4426950408889634f, 0.f));
}
__device__ __forceinline__ float phi_f(float x) { return __builtin_elementwise_maximum(x + 1.f, expc_f(x)); }
__device__ __forceinline__ float elu_f(float x) { return __builtin_elementwise_maximum(x, expc_f(x) - 1.f); }
__device__ __forceinline__ float dphi_f(float x) { return expn_f(x); }

// The feature maps kernels are instantiated for.
//   FeatElu: phi = elu + 1 elementwise (the default everywhere).  The kernels
//     carry its sums split around the constant 1 (kSplit): S = 1 P^T + S_E,
//     z = n 1 + z_E, with E(x) = phi(x) - 1 = elu(x) small at the usual input
//     scales, and the rank-1 parts in exact fp32 terms.
//   FeatGiven: the inputs already are positive features computed beforehand
//     (FAVOR+ random features, say): phi(x) = x.  Such features need not sit near
//     1 (FAVOR+ features of unscaled inputs are orders of magnitude below it,
//     where a split around 1 would cancel catastrophically), so they are carried
//     unsplit: E(x) = x and every rank-1 term is dropped.
// Either way E(0) = 0: the zero rows read past a sequence's end add nothing.
// dphi_at_phi(p): phi'(x) from p = phi(x) (the backward's chain factor).
struct FeatElu {
    static constexpr bool kSplit = true;
    __device__ __forceinline__ static float phi(float x) { return phi_f(x); }
    __device__ __forceinline__ static float e(float x) { return elu_f(x); }
    __device__ __forceinline__ static float dphi_at_phi(float p) { return __builtin_elementwise_minimum(p, 1.f); }
};
struct FeatGiven {
    static constexpr bool kSplit = false;
    __device__ __forceinline__ static float phi(float x) { return x; }
    __device__ __forceinline__ static float e(float x) { return x; }
    __device__ __forceinline__ static float dphi_at_phi(float) { return 1.f; }
};

// 1/x to within an ulp: hardware reciprocal refined by one Newton step.
__device__ __forceinline__ float rcp_f(float x) {
    float r = __builtin_amdgcn_rcpf(x);
    return r * (2.f - x * r);
}

// ---- HBM access through buffer resources -----------------------------------------------
// A buffer resource covers one head's range; reads beyond it return 0 and
// writes beyond it are dropped, so sequence tails need no branches and the
// compiler can count outstanding memory operations exactly.  Offsets are bytes.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
struct GBuf {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ GBuf(const void* base, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000)) {}
    __device__ __forceinline__ uint4 ld16(uint32_t off) const {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        return make_uint4(x.x, x.y, x.z, x.w);
    }
    __device__ __forceinline__ uint2 ld8(uint32_t off) const {
        const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        return make_uint2(x.x, x.y);
    }
    __device__ __forceinline__ float ld4f(uint32_t off) const {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    }
    __device__ __forceinline__ void st16(uint32_t off, uint4 v) const {
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, off, 0, 0);
    }
    __device__ __forceinline__ void st8(uint32_t off, uint2 v) const {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, r, off, 0, 0);
    }
    __device__ __forceinline__ void st4f(uint32_t off, float v) const {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
    }
    // Agent-coherent 16-byte load / store (cache policy sc1): served by or written
    // through to the device-wide coherence point, so data that another workgroup
    // of the same launch stores this way is seen without any cache flush.
    __device__ __forceinline__ f32x4 ld16c(uint32_t off) const {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent);
        return f32x4{__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w)};
    }
    __device__ __forceinline__ void st16c(uint32_t off, f32x4 v) const {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)}, r, off, 0,
            kCoherent);
    }
    static constexpr int kCoherent = 16;  // the sc1 bit of the buffer instructions' cache policy
};

// ---- signals between workgroups of one launch -------------------------------------------
// A 64-bit flag word holds the epoch (a value unique to the launch) once its
// producer's data is complete.  The producer writes that data with agent-coherent
// stores and waits for them (s_waitcnt) before the flag store; the consumer polls
// the flag with agent-coherent loads and then reads the data agent-coherently.
// No L2 writeback or invalidation is involved (those would cost every waiting
// workgroup a flush of its XCD's L2).  The wait is bounded: after `limit` polls
// (65536 unless a test lowers it) it gives up and reports failure, so a missing
// producer cannot hang the GPU.
__device__ __forceinline__ void post_flag(unsigned long long* f, unsigned long long epoch) {
    __hip_atomic_store(f, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool await_flag(const unsigned long long* f, unsigned long long epoch, int limit) {
    for (int i = 0; i < limit; ++i) {
        if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) return true;
        __builtin_amdgcn_s_sleep(2);
    }
    return false;
}
// Wait for every outstanding memory operation of this wave (stores acknowledged).
__device__ __forceinline__ void wait_all_memory() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- waits and barriers managed by hand ---------------------------------------------------
// s_waitcnt with only the vector-memory count constrained (gfx9 encoding).
// The signal fences keep the compiler from moving memory operations across
// these points (they emit no instruction).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding direct-to-LDS load): the caller has made the LDS
// data it needs complete with explicit waits.
__device__ __forceinline__ void raw_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS operations are done
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- swizzled LDS tiles ----------------------------------------------------------------
// ROWS x COLS elements of OT, row-major, with the 16-byte granule index of each
// row XOR-ed by a row-dependent value so that 16-row operand reads, 8-row
// granule writes and 4-row transposing reads all spread over the banks.
// kAccCols: within each 32-column block the 4-column groups are stored in the order
// 0 4 1 5 2 6 3 7, so that the k values an accumulator-order operand takes in one lane
// (columns k0 + 4 j .. + 3 and k0 + 16 + 4 j .. + 3) are one 16-byte granule.  Such a
// tile is written 4 columns at a time (store4, store_T) and read by ld_acc and the
// transposing loads; whole-granule writes and Mma::ld do not apply to it.
template <typename OT, int ROWS, int COLS, bool kAccCols = false>
struct Tile {
    static constexpr int EV = 16 / (int)sizeof(OT);
    static constexpr int G = COLS / EV;
    static_assert(COLS % EV == 0, "tile width must be whole granules");
    static_assert(G >= 4 && (G & (G - 1)) == 0, "granules per row must be a power of two >= 4");
    static constexpr int kElems = ROWS * COLS;
    OT* p;
    // 16-byte granule permutation of row r.  With 32 four-byte banks (128 B):
    //  - 16 lanes reading one granule of 16 consecutive rows hit 8 distinct bank
    //    groups per 8 rows (operand loads);
    //  - 16 lanes of a transposing load reading two adjacent granules of 4
    //    consecutive rows hit 8 distinct bank groups;
    //  - 8 (G >= 8) or 4 (G == 4) lanes writing the granules of a row never collide.
    __device__ __forceinline__ static int swz(int r) {
        return G >= 8 ? 2 * (r & 3) + ((r >> 2) & 1) : 2 * ((r >> 1) & 1) + ((r >> 2) & 1);
    }
    __device__ __forceinline__ static int col(int c) {
        if constexpr (kAccCols) {
            static_assert(sizeof(OT) == 2 && COLS % 32 == 0, "acc-order columns are for bf16 tiles of 32-column blocks");
            const int q = (c >> 2) & 7;
            return (c & ~31) | ((2 * (q & 3) + (q >> 2)) << 2) | (c & 3);
        } else {
            return c;
        }
    }
    __device__ __forceinline__ int off(int r, int c) const {
        const int cc = col(c);
        return r * COLS + (((cc / EV) ^ swz(r)) * EV) + (cc % EV);
    }
    __device__ __forceinline__ OT* granule(int r, int gi) const {
        static_assert(!kAccCols, "whole granules of an acc-order tile are not consecutive columns");
        return p + r * COLS + ((gi ^ swz(r)) * EV);
    }
    __device__ __forceinline__ OT& at(int r, int c) const { return p[off(r, c)]; }
};

// ---- MFMA operands ---------------------------------------------------------------------
// A 16x16 output tile D[i][j] += sum_k X[i][k] Y[j][k].  Lane l supplies row
// (l & 15) of X and of Y with the same k values, so the result does not depend
// on how the instruction orders k inside a step.  The accumulator holds
// D[4 (l >> 4) + r][l & 15] in element r.
//
//   ld    : operand rows are tile rows row0.., k runs along the tile's columns;
//   ld_tr : operand rows are tile columns col0.., k runs along the tile's rows
//           (for bf16 two ds_read_b64_tr_b16: within each 16-lane group, lane
//           j of the result holds column col0 + j at 4 consecutive rows);
//   splat : every operand row is the same vector v[k] (from fp32 in LDS).
template <typename OT>
struct Mma;

template <>
struct Mma<bf16> {
    static constexpr int KSTEP = 32;
    typedef bf16x8 frag;
    template <int R, int K>
    __device__ __forceinline__ static frag ld(const Tile<bf16, R, K>& t, int row0, int k0, int lane) {
        return *reinterpret_cast<const frag*>(t.granule(row0 + (lane & 15), (k0 >> 3) + (lane >> 4)));
    }
    template <int R, int K>
    __device__ __forceinline__ static frag ld_tr(const Tile<bf16, R, K>& t, int k0, int col0, int lane) {
        typedef __attribute__((address_space(3))) bf16x4 lds4;
        const int j = lane & 15;
        const int r = k0 + 8 * (lane >> 4) + (j >> 2);
        const int c = col0 + 4 * (j & 3);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(&t.at(r, c)));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(&t.at(r + 4, c)));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // As ld_tr, but lane l takes the k values k0 + 4 (l >> 4) + 0..3 and
    // k0 + 16 + 4 (l >> 4) + 0..3: the rows that accumulator tiles k0/16 and
    // k0/16 + 1 hold in lane l, so that such a pair can be the other operand (acc_op).
    template <int R, int K, bool A>
    __device__ __forceinline__ static frag ld_tr_acc(const Tile<bf16, R, K, A>& t, int k0, int col0, int lane) {
        typedef __attribute__((address_space(3))) bf16x4 lds4;
        const int j = lane & 15;
        const int r = k0 + 4 * (lane >> 4) + (j >> 2);
        const int c = col0 + 4 * (j & 3);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(&t.at(r, c)));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(&t.at(r + 16, c)));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // As ld, in the k order of ld_tr_acc: lane l takes columns k0 + 4 (l >> 4) + 0..3
    // and k0 + 16 + 4 (l >> 4) + 0..3 of its row.
    template <int R, int K, bool A>
    __device__ __forceinline__ static frag ld_acc(const Tile<bf16, R, K, A>& t, int row0, int k0, int lane) {
        const int r = row0 + (lane & 15), c = k0 + 4 * (lane >> 4);
        if constexpr (A) {
            return *reinterpret_cast<const frag*>(&t.at(r, c));  // one granule
        } else {
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(&t.at(r, c));
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(&t.at(r, c + 16));
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }
    // Operand for k-step k0 from per-lane values in accumulator order: y[4 m + e]
    // is the value at k = 16 m + 4 (l >> 4) + e (the layout of an accumulator
    // tile's rows, and of the k order of ld_acc / ld_tr_acc).
    __device__ __forceinline__ static frag vals_op(const float* y, int k0) {
        frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (bf16)y[k0 / 4 + e];
        return f;
    }
    // The same from raw inputs already in that order (4 elements per 8-byte word).
    __device__ __forceinline__ static frag raw_op(const uint2* r, int k0) {
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(&r[k0 / 16]);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(&r[k0 / 16 + 1]);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // E = phi - 1 of every element (elu for the default map), rounded back to bf16.
    template <class FM = FeatElu>
    __device__ __forceinline__ static frag elu_op(frag x) {
        frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (bf16)FM::e((float)x[e]);
        return f;
    }
    // Operand for k-step k0 of a contraction over the row index of accumulator
    // tiles acc[0..]: the column index of the tiles is the operand row.
    __device__ __forceinline__ static frag acc_op(const f32x4* acc, int k0) {
        const f32x4 a = acc[k0 / 16], b = acc[k0 / 16 + 1];
        frag f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[e] = (bf16)a[e];
            f[4 + e] = (bf16)b[e];
        }
        return f;
    }
    // v: fp32 vector in LDS indexed by k; hi/lo split keeps ~16 bits of each value.
    __device__ __forceinline__ static void splat(const float* v, int k0, int lane, frag& hi, frag& lo) {
        const f32x4* p = reinterpret_cast<const f32x4*>(v + k0 + 8 * (lane >> 4));
        const f32x4 a = p[0], b = p[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            hi[e] = (bf16)a[e];
            lo[e] = (bf16)(a[e] - (float)hi[e]);
            hi[4 + e] = (bf16)b[e];
            lo[4 + e] = (bf16)(b[e] - (float)hi[4 + e]);
        }
    }
    __device__ __forceinline__ static frag ones() {
        frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (bf16)1.f;
        return f;
    }
    // Every operand row is the vector v[k] (bf16 in LDS, read as it is stored).
    __device__ __forceinline__ static frag vec_op(const bf16* v, int k0, int lane) {
        return *reinterpret_cast<const frag*>(v + k0 + 8 * (lane >> 4));
    }
    static constexpr bool kSplitSplat = true;
    __device__ __forceinline__ static f32x4 mma(frag x, frag y, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
    }
};

template <>
struct Mma<float> {
    static constexpr int KSTEP = 4;
    typedef float frag;
    // k order inside each block of 16: step k0 = 16 x + 4 e gives lane group g
    // the value 16 x + 4 g + e, which is also the row that accumulator tile x
    // holds in element e of lane group g.  Every operand uses this order, so
    // contraction lengths are multiples of 16.
    __device__ __forceinline__ static int kap(int k0, int lane) { return (k0 & ~15) + 4 * (lane >> 4) + ((k0 & 15) >> 2); }
    template <int R, int K>
    __device__ __forceinline__ static frag ld(const Tile<float, R, K>& t, int row0, int k0, int lane) {
        return t.at(row0 + (lane & 15), kap(k0, lane));
    }
    template <int R, int K>
    __device__ __forceinline__ static frag ld_tr(const Tile<float, R, K>& t, int k0, int col0, int lane) {
        return t.at(kap(k0, lane), col0 + (lane & 15));
    }
    template <int R, int K>
    __device__ __forceinline__ static frag ld_tr_acc(const Tile<float, R, K>& t, int k0, int col0, int lane) {
        return ld_tr(t, k0, col0, lane);
    }
    template <int R, int K>
    __device__ __forceinline__ static frag ld_acc(const Tile<float, R, K>& t, int row0, int k0, int lane) {
        return ld(t, row0, k0, lane);
    }
    __device__ __forceinline__ static frag vals_op(const float* y, int k0) { return y[k0 / 4]; }
    __device__ __forceinline__ static frag raw_op(const uint4* r, int k0) {
        return reinterpret_cast<const float*>(&r[k0 >> 4])[(k0 & 15) >> 2];
    }
    __device__ __forceinline__ static frag acc_op(const f32x4* acc, int k0) { return acc[k0 >> 4][(k0 & 15) >> 2]; }
    template <class FM = FeatElu>
    __device__ __forceinline__ static frag elu_op(frag x) { return FM::e(x); }
    __device__ __forceinline__ static void splat(const float* v, int k0, int lane, frag& hi, frag& lo) {
        hi = v[kap(k0, lane)];
        lo = 0.f;
    }
    __device__ __forceinline__ static frag ones() { return 1.f; }
    __device__ __forceinline__ static frag vec_op(const float* v, int k0, int lane) { return v[kap(k0, lane)]; }
    static constexpr bool kSplitSplat = false;
    __device__ __forceinline__ static f32x4 mma(frag x, frag y, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, c, 0, 0, 0);
    }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ f32x4 splat4(float x) { return f32x4{x, x, x, x}; }

// 0.f that the compiler cannot see through: selecting between a value and it
// keeps the select on the fp32 value (a select against a literal 0 is moved
// past the later bf16 rounding, which then costs a separate pack).
__device__ __forceinline__ float opaque_zero() {
    uint32_t z;
    asm("s_mov_b32 %0, 0" : "=s"(z));
    return __uint_as_float(z);
}
// Lane l of the wavefront reads bit l of the uniform mask m (a select on it
// needs no compare).
__device__ __forceinline__ bool lane_bit(uint64_t m) { return __builtin_amdgcn_inverse_ballot_w64(m); }

// Write an accumulator tile transposed: element (i, j) goes to dst[col0 + j][row0 + i];
// each lane writes 4 consecutive elements of one row (8 bytes in bf16, 16 in fp32).
__device__ __forceinline__ void store4(bf16* p, f32x4 a) {
    bf16 h[4] = {(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
    *reinterpret_cast<uint2*>(p) = *reinterpret_cast<const uint2*>(h);
}
__device__ __forceinline__ void store4(float* p, f32x4 a) { *reinterpret_cast<f32x4*>(p) = a; }

template <typename OT, int ROWS, int COLS, bool A>
__device__ __forceinline__ void store_T(const Tile<OT, ROWS, COLS, A>& dst, int row0, int col0, f32x4 acc, int lane) {
    store4(&dst.at(col0 + (lane & 15), row0 + 4 * (lane >> 4)), acc);
}

// 4 consecutive elements of an LDS tile row as fp32.
__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 lds4(const bf16* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    const bf16* h = reinterpret_cast<const bf16*>(&u);
    return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}

// ---- non-finite operands ----------------------------------------------------------------
// A masked weight is an exact zero, but 0 * inf = NaN: an operand row of a later
// token that holds inf or NaN would reach earlier rows through the masked part of
// an in-chunk product.  Where a segment can hold such a row, the kernels replace
// the non-finite operand values of the products that mix masked and unmasked
// weights by 0 (finite values pass bitwise unchanged) and restore the non-finite
// results of the unmasked rows explicitly.
__device__ __forceinline__ bool finite_f(float x) { return __builtin_isfinite(x); }
__device__ __forceinline__ float finite_or_zero(float x) {
    const uint32_t w = __float_as_uint(x);
    return (w & 0x7f800000u) == 0x7f800000u ? 0.f : x;
}
// Two bf16 in a dword: each half becomes +0 where its exponent is all ones.  With
// h | 0x807f, adding 1 carries into bit 15 (clearing it) exactly when the exponent
// bits are all ones; a packed 16-bit add keeps the halves apart, and an arithmetic
// shift by 15 turns bit 15 into the keep-mask.  Four VALU operations per dword.
__device__ __forceinline__ uint32_t finite_or_zero_bf16x2(uint32_t w) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    typedef short i16x2 __attribute__((ext_vector_type(2)));
    const u16x2 t = __builtin_bit_cast(u16x2, w | 0x807f807fu) + (u16x2){1, 1};
    const i16x2 keep = __builtin_bit_cast(i16x2, t) >> (i16x2){15, 15};
    return w & __builtin_bit_cast(uint32_t, keep);
}
__device__ __forceinline__ bf16x8 finite_or_zero(bf16x8 f) {
    u32x4 w = __builtin_bit_cast(u32x4, f);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = finite_or_zero_bf16x2(w[i]);
    return __builtin_bit_cast(bf16x8, w);
}

// ---- wave reductions -------------------------------------------------------------------
// Sum over the four 16-lane groups (lanes with the same l & 15).
__device__ __forceinline__ float sum_over_groups(float x) {
    x += __shfl_xor(x, 16, kWave);
    x += __shfl_xor(x, 32, kWave);
    return x;
}

// Sum over aligned groups of WIDTH consecutive lanes (WIDTH a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float sum_lanes(float x) {
#pragma unroll
    for (int o = 1; o < WIDTH; o <<= 1) x += __shfl_xor(x, o, kWave);
    return x;
}

}  // namespace la
