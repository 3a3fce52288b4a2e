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

// ---------------------------------------------------------------------------------------
// decode_steps_grouped: the same T steps for G >= 2 query heads per key/value state, with
// every product on MFMA.  The G query heads of a token all read one state, so a block of
// rows (t, h) (token-major, up to 64 rows; 32 for fewer than 4 heads per state) is the causal
// form of the proposition over the block's tokens tau0 .. tau1, chunked:
//   num_r = phi(q_r)^T S_<tau0 + sum_{tau0 <= tau <= t(r)} (phi(q_r).phi(k_tau)) v_tau,
//   den_r = phi(q_r)^T z_<tau0 + sum_{tau0 <= tau <= t(r)} phi(q_r).phi(k_tau),
// and S, z then take the updates of the block's tokens whose rows are all done (a token
// whose rows continue into the next block is that block's first key).  The state term is
// a [rows x d] x [d x d] product, the in-block terms [rows x keys] products, the update a
// rank-(keys) product.  Sums into the state run as fp32 MFMA (v_mfma_f32_16x16x4_f32), so
// the state keeps fp32 arithmetic throughout, as in the one-row kernels; the products with
// phi(q) do too for fp32 inputs, and take bf16 hi + lo splits for bf16 inputs.
// Wave w holds state columns w d/4 .. (w + 1) d/4 - 1 of every feature row in accumulator
// tiles: element i of lane (g, c) of tile (at, bt) is S[16 at + 4 g + i][w d/4 + 16 bt + c].
// Read as the B operand of a product that contracts over features in the order
// 16 at + 4 g + i (the A operand, phi(q), is read from LDS in that order), the tiles need
// no movement; the update accumulates into them.  The state moves through LDS once in
// each direction (16-byte global accesses).  A later token's inf or NaN in v would reach
// earlier rows through the masked zeros of the in-block product (0 * inf = NaN): blocks
// holding one take v with non-finite entries replaced by 0 there, and the rows that do
// read such a token get it back explicitly (num += v - v).
template <typename T>
__device__ __forceinline__ f32x4 gload4(const T* p);
template <>
__device__ __forceinline__ f32x4 gload4<float>(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
template <>
__device__ __forceinline__ f32x4 gload4<bf16>(const bf16* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    const bf16* h = reinterpret_cast<const bf16*>(&u);
    return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}

template <int D>
struct GroupedDecodeCfg {
    static constexpr int RBM = 64;           // rows (token, query head) per block at most
    static constexpr int KM = 16;            // key slots per block: blocks start at multiples of their row count,
                                             // so 64 rows of G >= 4 heads (32 of G = 2, 3) span at most 16 tokens
    static constexpr int DP = D + 4;         // LDS row stride in floats: 16 rows read 16 bytes each without conflicts
    static constexpr int AP = KM + 4;
    static constexpr int DQ = D + 8;         // bf16 row stride of the split phi tiles (16 rows of 8 bytes: no conflicts)
    static constexpr int NAT = D / 16;       // feature tiles of the state
    static constexpr int CPW = D / 4;        // state columns per wave
    static constexpr int NBT = CPW / 16;     // column tiles per wave
};

// Operand of a 16x16x32 bf16 MFMA from row `row` of a bf16 tile (stride ld): columns
// k0 + 4 g .. + 3 and k0 + 16 + 4 g .. + 3, the k order of accumulator-tile pairs.
__device__ __forceinline__ Mma<bf16>::frag ld_pair(const bf16* t, int ld, int row, int k0, int g) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(t + row * ld + k0 + 4 * g);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(t + row * ld + k0 + 16 + 4 * g);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi): 16 significant bits.
__device__ __forceinline__ bf16 split_lo(float x, bf16 hi) { return (bf16)(x - (float)hi); }

template <typename T, int D, class FM>
__global__ __launch_bounds__(kBlock, 2) void decode_steps_grouped_kernel(float* __restrict__ S, float* __restrict__ z,
                                                                      const T* __restrict__ q, const T* __restrict__ k,
                                                                      const T* __restrict__ v, T* __restrict__ o,
                                                                      int ntok, int G) {
    using C = GroupedDecodeCfg<D>;
    constexpr int RBM = C::RBM, KM = C::KM, DP = C::DP, AP = C::AP, NAT = C::NAT, CPW = C::CPW, NBT = C::NBT;
    constexpr int DQ = C::DQ;
    // bf16 inputs: the products with phi(q) (the state term and A) run as three bf16 MFMAs
    // on hi + lo splits of both operands (hi hi + hi lo + lo hi: about 2^-16 relative per
    // product, far below the bf16 rounding of the outputs) at a fifth of the fp32 MFMA's
    // cycles; fp32 inputs keep the fp32 MFMA.  Sums into the state stay fp32 MFMA either way.
    constexpr bool kSplit = sizeof(T) == 2;
    typedef Mma<bf16>::frag BF;
    constexpr int F4 = D / 4;
    static_assert(NBT >= 1 && kBlock == 4 * kWave && RBM % 16 == 0 && D % RBM == 0,
                  "four waves, whole column tiles per wave, the state in whole row buffers");
    // phi(q) of the block's rows (fp32, or bf16 hi and lo tiles); the state; the outputs
    __shared__ __attribute__((aligned(16))) float sQ[RBM * (DP > DQ ? DP : DQ)];
    __shared__ __attribute__((aligned(16))) bf16 sKs[kSplit ? 2 * KM * DQ : 8];  // phi(k) hi, lo tiles
    __shared__ __attribute__((aligned(16))) float sK[KM * DP];   // phi(k) of the block's keys
    __shared__ __attribute__((aligned(16))) float sV[KM * DP];   // v of the block's keys
    __shared__ __attribute__((aligned(16))) float sA[RBM * AP];  // masked phi(q_r).phi(k_tau)
    __shared__ __attribute__((aligned(16))) float sZ[D];
    __shared__ float sDen[RBM];  // 1 / den of each row
    __shared__ int sTok[RBM];    // token of each row of the block

    const int64_t bkv = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave, g = lane >> 4, c16 = lane & 15;
    const int cb0 = w * CPW;
    float* const Sh = S + bkv * D * D;
    const int64_t krow0 = bkv * ntok;
    const int nrows = G * ntok;  // the launcher keeps it below 2^31
    const int rb = G >= 4 ? RBM : RBM / 2;  // at most KM keys per block either way
    const int nrt = rb / 16;
    auto qoff = [&](int t, int h) { return ((bkv * G + h) * ntok + t) * D; };  // row t G + h
    // A thread handles rows tid / F4 + RSTEP j of a block (j = 0, 1, ..): their (token, head)
    // pairs follow from the first by steps of RSTEP rows, one division per block.
    constexpr int RSTEP = kBlock / F4;
    const int tstep = RSTEP / G, hstep = RSTEP - tstep * G;
    auto step_row = [&](int& t, int& h) {
        t += tstep;
        h += hstep;
        if (h >= G) {
            h -= G;
            ++t;
        }
    };

    // The loads of a block's rows and keys go to registers one block ahead: the first
    // block's are in flight during the state passes, each later block's during the
    // products of the block before it.  Rows and keys past a block load a valid row
    // (every load is issued before the first use) and are staged as zeros.
    constexpr int NQ = RBM * F4 / kBlock, NK = KM * F4 / kBlock;
    static_assert(NQ * kBlock == RBM * F4 && NK * kBlock == KM * F4, "whole staging passes");
    f32x4 xq[NQ], xk[NK], xv[NK];
    auto load_block = [&](int rs, int ts, int nbs, int tbks) {
        const int ra = rs + tid / F4, rl = rs + nbs - 1;  // first row, last row of the block
        int t = ra / G, h = ra - t * G;
        const int tl = rl / G, hl = rl - tl * G;
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int i4 = tid + j * kBlock, r = i4 / F4, c = 4 * (i4 % F4);
            xq[j] = gload4<T>(q + (r < nbs ? qoff(t, h) : qoff(tl, hl)) + c);
            step_row(t, h);
        }
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int i4 = tid + j * kBlock, sl = i4 / F4, c = 4 * (i4 % F4);
            const int64_t off = (krow0 + ts + min(sl, tbks - 1)) * D + c;
            xk[j] = gload4<T>(k + off);
            xv[j] = gload4<T>(v + off);
        }
    };
    // Block extent from its first row r0 and first key tau0 = t(r0): nb rows, keys
    // tau0 .. t(r0 + nb - 1) (tbk of them), of which the first tba have all their rows here.
    auto block_nb = [&](int rs) { return min(rb, nrows - rs); };
    auto block_tbk = [&](int rs, int ts) { return (rs + block_nb(rs) - 1) / G - ts + 1; };
    load_block(0, 0, block_nb(0), block_tbk(0, 0));

    f32x4 st[NAT][NBT];
    // 16-byte state loads, RBM rows per pass, the next pass's loads in flight during this one's
    constexpr int NSP = RBM * F4 / kBlock;
    static_assert(NSP * kBlock == RBM * F4, "whole passes");
    f32x4 sld[NSP], snx[NSP];
#pragma unroll
    for (int j = 0; j < NSP; ++j) {
        const int i4 = tid + j * kBlock;
        sld[j] = *reinterpret_cast<const f32x4*>(&Sh[(int64_t)(i4 / F4) * D + 4 * (i4 % F4)]);
    }
#pragma unroll
    for (int a0 = 0; a0 < D; a0 += RBM) {
        if (a0 + RBM < D) {
#pragma unroll
            for (int j = 0; j < NSP; ++j) {
                const int i4 = tid + j * kBlock;
                snx[j] = *reinterpret_cast<const f32x4*>(&Sh[(int64_t)(a0 + RBM + i4 / F4) * D + 4 * (i4 % F4)]);
            }
        }
#pragma unroll
        for (int j = 0; j < NSP; ++j) {
            const int i4 = tid + j * kBlock;
            *reinterpret_cast<f32x4*>(&sQ[(i4 / F4) * DP + 4 * (i4 % F4)]) = sld[j];
        }
        __syncthreads();
#pragma unroll
        for (int at = 0; at < NAT; ++at)
            if (16 * at >= a0 && 16 * at < a0 + RBM)
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) st[at][bt][i] = sQ[(16 * at - a0 + 4 * g + i) * DP + cb0 + 16 * bt + c16];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NSP; ++j) sld[j] = snx[j];
    }
    float zn = 0.f;
    if (tid < D) {
        zn = z[bkv * D + tid];
        sZ[tid] = zn;
    }

    int tau0 = 0;
    for (int r0 = 0; r0 < nrows;) {
        const int nb = block_nb(r0), rend = r0 + nb;
        const int tbk = block_tbk(r0, tau0);            // keys tau0 .. t(rend - 1)
        const int tba = rend % G == 0 ? tbk : tbk - 1;  // keys whose rows are all done
        // Key slot s sits at k index 4 (s % 4) + s / 4 of the in-block products, so the
        // products over the first n keys take ceil(n / 4) of the four MFMA k-steps.
        const int nik = (tbk + 3) / 4, nia = (tba + 3) / 4;

        // Stage phi(q) of the rows (zero past the block), phi(k) and v of the keys (zero past them).
        if (tid < RBM) sTok[tid] = (r0 + tid) / G;
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int i4 = tid + j * kBlock, r = i4 / F4, c = 4 * (i4 % F4);
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = r < nb ? FM::phi(xq[j][e]) : 0.f;
            if constexpr (kSplit) {
                bf16x4 h, l;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[e] = (bf16)x[e];
                    l[e] = split_lo(x[e], h[e]);
                }
                bf16* const qh = reinterpret_cast<bf16*>(sQ);
                *reinterpret_cast<bf16x4*>(qh + r * DQ + c) = h;
                *reinterpret_cast<bf16x4*>(qh + RBM * DQ + r * DQ + c) = l;
            } else {
                *reinterpret_cast<f32x4*>(&sQ[r * DP + c]) = x;
            }
        }
        int bad = 0;
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int i4 = tid + j * kBlock, s = i4 / F4, c = 4 * (i4 % F4);
            f32x4 a, b;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a[e] = s < tbk ? FM::phi(xk[j][e]) : 0.f;
                b[e] = s < tbk ? xv[j][e] : 0.f;
                bad |= !finite_f(b[e]);
            }
            *reinterpret_cast<f32x4*>(&sK[s * DP + c]) = a;
            *reinterpret_cast<f32x4*>(&sV[s * DP + c]) = b;
            if constexpr (kSplit) {
                bf16x4 h, l;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[e] = (bf16)a[e];
                    l[e] = split_lo(a[e], h[e]);
                }
                *reinterpret_cast<bf16x4*>(sKs + s * DQ + c) = h;
                *reinterpret_cast<bf16x4*>(sKs + KM * DQ + s * DQ + c) = l;
            }
        }
        const bool vbad = __syncthreads_or(bad) != 0;
        if (rend < nrows) load_block(rend, tau0 + tba, block_nb(rend), block_tbk(rend, tau0 + tba));

        // A[r][s] = phi(q_r).phi(k_{tau0+s}) for tau0 + s <= t(r), else 0: wave w, row tile w.
        static_assert(KM == 16, "one tile of key slots");
        if (w < nrt) {
            f32x4 acc = zero4();
            if constexpr (kSplit) {
                const bf16* const qh = reinterpret_cast<const bf16*>(sQ);
#pragma unroll
                for (int k0 = 0; k0 < D; k0 += 32) {
                    const BF ah = ld_pair(qh, DQ, 16 * w + c16, k0, g), al = ld_pair(qh + RBM * DQ, DQ, 16 * w + c16, k0, g);
                    const BF bh = ld_pair(sKs, DQ, c16, k0, g), bl = ld_pair(sKs + KM * DQ, DQ, c16, k0, g);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int at = 0; at < NAT; ++at) {
                    const f32x4 xq = lds4(&sQ[(16 * w + c16) * DP + 16 * at + 4 * g]);
                    const f32x4 xk = lds4(&sK[c16 * DP + 16 * at + 4 * g]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xq[i], xk[i], acc, 0, 0, 0);
                }
            }
            const int s = c16, sp = 4 * (s & 3) + (s >> 2);  // slot s at k index sp
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * w + 4 * g + e;
                const bool live = r < nb && s < tbk && tau0 + s <= sTok[r];
                sA[r * AP + sp] = live ? acc[e] : 0.f;
            }
        }
        __syncthreads();

        // den_r = phi(q_r).z + sum_s A[r][s]: four threads per row.
        {
            static_assert(RBM * 4 == kBlock && KM == 16, "four threads per row, four key slots each");
            const int r = tid >> 2, p = tid & 3;
            float dp = 0.f;
            if (r < nb) {
#pragma unroll
                for (int a = p * (D / 4); a < (p + 1) * (D / 4); a += 4) {
                    f32x4 x;
                    if constexpr (kSplit) {
                        const bf16* const qh = reinterpret_cast<const bf16*>(sQ);
                        const bf16x4 h = *reinterpret_cast<const bf16x4*>(qh + r * DQ + a);
                        const bf16x4 l = *reinterpret_cast<const bf16x4*>(qh + RBM * DQ + r * DQ + a);
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = (float)h[e] + (float)l[e];
                    } else {
                        x = lds4(&sQ[r * DP + a]);
                    }
                    const f32x4 zz = lds4(&sZ[a]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dp += x[e] * zz[e];
                }
                const f32x4 x = lds4(&sA[r * AP + 4 * p]);
                dp += (x[0] + x[1]) + (x[2] + x[3]);
            }
            dp += __shfl_xor(dp, 1, kWave);
            dp += __shfl_xor(dp, 2, kWave);
            if (p == 0 && r < nb) sDen[r] = rcp_f(dp);  // 1 / den
        }

        // num = phi(Q) S + A V for this wave's columns, every row tile of the buffer (rows past
        // the block are zeros): the row tiles' accumulators are independent chains, so the
        // products of one feature step go to the MFMA unit back to back.
        constexpr int NRT = RBM / 16;
        f32x4 num[NRT][NBT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) num[rt][bt] = zero4();
        if constexpr (kSplit) {
            const bf16* const qh = reinterpret_cast<const bf16*>(sQ);
#pragma unroll
            for (int at = 0; at < NAT; at += 2) {  // k-step over features 16 at .. 16 at + 31
                BF sh[NBT], sl[NBT];
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sh[bt][e] = (bf16)st[at][bt][e];
                        sl[bt][e] = split_lo(st[at][bt][e], sh[bt][e]);
                        sh[bt][4 + e] = (bf16)st[at + 1][bt][e];
                        sl[bt][4 + e] = split_lo(st[at + 1][bt][e], sh[bt][4 + e]);
                    }
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) {
                    const BF ah = ld_pair(qh, DQ, 16 * rt + c16, 16 * at, g);
                    const BF al = ld_pair(qh + RBM * DQ, DQ, 16 * rt + c16, 16 * at, g);
#pragma unroll
                    for (int bt = 0; bt < NBT; ++bt) {
                        num[rt][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, sh[bt], num[rt][bt], 0, 0, 0);
                        num[rt][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, sl[bt], num[rt][bt], 0, 0, 0);
                        num[rt][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, sh[bt], num[rt][bt], 0, 0, 0);
                    }
                }
            }
        } else {
#pragma unroll
            for (int at = 0; at < NAT; ++at) {
                f32x4 xq[NRT];
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) xq[rt] = lds4(&sQ[(16 * rt + c16) * DP + 16 * at + 4 * g]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                        for (int bt = 0; bt < NBT; ++bt)
                            num[rt][bt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xq[rt][i], st[at][bt][i], num[rt][bt], 0, 0, 0);
            }
        }
        {
            f32x4 xa[NRT];
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) xa[rt] = lds4(&sA[(16 * rt + c16) * AP + 4 * g]);  // slots g, 4 + g, ..
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < nik) {
                    float yv[NBT];
#pragma unroll
                    for (int bt = 0; bt < NBT; ++bt) {
                        yv[bt] = sV[(4 * i + g) * DP + cb0 + 16 * bt + c16];
                        if (vbad) yv[bt] = finite_or_zero(yv[bt]);
                    }
#pragma unroll
                    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                        for (int bt = 0; bt < NBT; ++bt)
                            num[rt][bt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[rt][i], yv[bt], num[rt][bt], 0, 0, 0);
                }
            }
        }
        __syncthreads();  // den is ready; phi(q) is no longer read

        // o = num / den into the row buffer; the rows that read a non-finite v get it back.
#pragma unroll
        for (int rt = 0; rt < RBM / 16; ++rt) {
            if (rt < nrt) {
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) {
                    const int b = cb0 + 16 * bt + c16;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 16 * rt + 4 * g + e;
                        if (r < nb) {
                            float x = num[rt][bt][e];
                            if (vbad) {
                                const int last = sTok[r] - tau0;  // keys tau0 .. tau0 + last
                                for (int s = 0; s <= last; ++s) {
                                    const float y = sV[s * DP + b];
                                    if (!finite_f(y)) x += y - y;
                                }
                            }
                            sQ[r * DP + b] = x * sDen[r];
                        }
                    }
                }
            }
        }
        // S += sum over the finished keys of phi(k) v^T (fp32 MFMA into the state tiles).
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < nia) {
                const int s = 4 * i + g;
                float yv[NBT];
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) yv[bt] = s < tba ? sV[s * DP + cb0 + 16 * bt + c16] : 0.f;
#pragma unroll
                for (int at = 0; at < NAT; ++at) {
                    const float xk = s < tba ? sK[s * DP + 16 * at + c16] : 0.f;
#pragma unroll
                    for (int bt = 0; bt < NBT; ++bt)
                        st[at][bt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xk, yv[bt], st[at][bt], 0, 0, 0);
                }
            }
        }
        __syncthreads();  // the outputs are in the row buffer

        {
            const int ra = r0 + tid / F4;
            int t = ra / G, h = ra - t * G;
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const int i4 = tid + j * kBlock, r = i4 / F4, c = 4 * (i4 % F4);
                if (r < nb) store4(o + qoff(t, h) + c, lds4(&sQ[r * DP + c]));
                step_row(t, h);
            }
        }
        if (tid < D) {  // z over the finished keys, token by token
            for (int s = 0; s < tba; ++s) zn += sK[s * DP + tid];
            sZ[tid] = zn;
        }
        __syncthreads();  // the block's buffers are free for the next one
        r0 = rend;
        tau0 += tba;
    }

    // Write the state back through the row buffer (16-byte global stores).
#pragma unroll
    for (int a0 = 0; a0 < D; a0 += RBM) {
#pragma unroll
        for (int at = 0; at < NAT; ++at)
            if (16 * at >= a0 && 16 * at < a0 + RBM)
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sQ[(16 * at - a0 + 4 * g + i) * DP + cb0 + 16 * bt + c16] = st[at][bt][i];
        __syncthreads();
        for (int i4 = tid; i4 < RBM * F4; i4 += kBlock) {
            const int r = i4 / F4, c = 4 * (i4 % F4);
            *reinterpret_cast<f32x4*>(&Sh[(int64_t)(a0 + r) * D + c]) = lds4(&sQ[r * DP + c]);
        }
        __syncthreads();
    }
    if (tid < D) z[bkv * D + tid] = zn;
}

template <class FM>
static hipError_t launch_decode_steps_fm(int dt, int d, float* S, float* z, const void* q, const void* k,
                                         const void* v, void* o, int64_t BHkv, int64_t T, int64_t G, hipStream_t s,
                                         int KF, float* den_out) {
    const dim3 grid((unsigned)(BHkv * KF));
    // Several query heads per state: the MFMA kernel (d = 64 and 128, one feature block).
    if (KF == 1 && G >= 2 && (d == 64 || d == 128) && G * T <= INT32_MAX) {
#define LA_DECG(TT, DD)                                                                                     \
    hipLaunchKernelGGL((decode_steps_grouped_kernel<TT, DD, FM>), grid, dim3(kBlock), 0, s, S, z, (const TT*)q, \
                       (const TT*)k, (const TT*)v, (TT*)o, (int)T, (int)G)
        if (dt == kBF16) {
            if (d == 64) LA_DECG(bf16, 64);
            else LA_DECG(bf16, 128);
        } else {
            if (d == 64) LA_DECG(float, 64);
            else LA_DECG(float, 128);
        }
#undef LA_DECG
        return hipGetLastError();
    }
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
