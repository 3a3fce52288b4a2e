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
// Work decomposition.  One workgroup (4 wavefronts; 8 for causal_fwd, in two
// roles) per (segment of `cps` chunks, head), numbered segment-major so that with the round-robin
// placement of workgroups on the 8 XCDs all segments of a head share an XCD
// (and its L2) whenever the head count is a multiple of 8.  seg_state reduces
// each segment's keys to (S_E, z_E, P); causal_fwd starts a segment from the
// sum of the records before it, added in segment order (fixed order, so the
// results are bitwise reproducible), and walks its chunks.  The non-causal
// forward is seg_state + per-head totals (total, beyond two segments) + noncausal_fwd.
//
// Data layout.  Inputs/outputs [BH][N][d] row-major in HBM.  Per chunk the
// workgroup stages E(K) and V row-major in LDS (bf16 for bf16 inputs, fp32 for
// fp32 inputs, double-buffered so one barrier per chunk suffices); each output
// wavefront keeps phi(Q) of its own 16 tokens in registers in MFMA operand
// layout, and the in-chunk weights A stay in the accumulators that produce them
// and feed the A V product directly.  S_E stays in fp32 MFMA accumulators
// across chunks and is published to LDS (rounded) once per chunk; z_E and P
// are accumulated by MFMA against a ones operand.  Segment records are fp32
// [S_E^T | z_E | P].
#include "chunk.h"

namespace la {

// ---------------------------------------------------------------------------------------
// seg_state: per (segment, head) the aggregates (S_E, z_E, P) of the segment's keys.
// K and V chunks stream into an LDS ring of R slots with direct-to-LDS loads
// (R - 1 chunks in flight while one is reduced); E = elu is applied to the
// MFMA operands, since each wavefront reads its own key columns only.  Waits
// and barriers are explicit: a step waits for its slot's loads, synchronises
// the workgroup, then refills the slot the previous step has finished reading.
// Gv: heads per value head (head bh reads the values of head bh / Gv: the feature
// blocks of one head share its values; Gv = 1: one each).
template <typename T, int D, class FM = FeatElu>
__global__ __launch_bounds__(kBlock, 2) void seg_state_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                           float* __restrict__ rec, int N, int cps, int nseg, int BH,
                                                           int Gv) {
    using DMA = TileDma<T, D>;
    constexpr int R = kC * D * (int)sizeof(T) >= 16384 ? 2 : 4;
    constexpr int RS = R > 2 ? kC * D : 16;  // slots 2 and 3 exist only for R = 4
    __shared__ __attribute__((aligned(16))) T sk0[kC * D], sk1[kC * D], sk2[RS], sk3[RS];
    __shared__ __attribute__((aligned(16))) T sv0[kC * D], sv1[kC * D], sv2[RS], sv3[RS];
    T* const ks[4] = {sk0, sk1, sk2, sk3};
    T* const vs[4] = {sv0, sv1, sv2, sv3};

    const int seg = blockIdx.x / BH, bh = blockIdx.x % BH;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int64_t hoff = (int64_t)bh * N * D, voff = (int64_t)(bh / Gv) * N * D;
    const uint32_t hbytes = (uint32_t)N * D * sizeof(T);
    const GBuf bk(k + hoff, hbytes), bv(v + voff, hbytes);
    const int tok_begin = seg * cps * kC;
    const int tok_end = min(N, tok_begin + cps * kC);
    const int nch = (tok_end - tok_begin + kC - 1) / kC;
    const int nsteps = (nch + R - 1) / R * R;
    // Chunks past the segment are aimed at row N: zeros, no memory traffic.
    auto chunk_tok = [&](int c) { return c < nch ? tok_begin + c * kC : N; };

    StateAcc<D> st;
    VecAcc<D> vz, vp;
    zero_state<D>(st);
    zero_vec<D>(vz);
    zero_vec<D>(vp);

#pragma unroll
    for (int u = 0; u < R; ++u) {
        DMA::issue(bk, chunk_tok(u), ks[u], w, lane);
        DMA::issue(bv, chunk_tok(u), vs[u], w, lane);
    }
    for (int c0 = 0; c0 < nsteps; c0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int c = c0 + u;
            // Every step from the second on refills one slot (past the segment
            // with zero chunks that move no bytes), so exactly the refills of
            // steps c-R+2 .. c-1 -- (R - 2) x 2 x PER_WAVE loads -- are younger
            // than chunk c's (more at step 0, where the wait is conservative).
            wait_vmcnt<(R - 2) * 2 * DMA::PER_WAVE>();
            raw_barrier();
            const int ur = (u + R - 1) % R;  // the slot step c - 1 read
            if (c >= 1) {
                DMA::issue(bk, chunk_tok(c - 1 + R), ks[ur], w, lane);
                DMA::issue(bv, chunk_tok(c - 1 + R), vs[ur], w, lane);
            }
            state_update<T, D, true, true, true, FM>(st, vz, vp, Tile<T, kC, D>{ks[u]}, Tile<T, kC, D>{vs[u]},
                                                     nullptr, nullptr, lane, w);
        }
    }
    wait_vmcnt<0>();  // no direct-to-LDS load may outlive the workgroup
    float* r = rec + ((int64_t)bh * nseg + seg) * Rec<D>::kSize;
    store_state<D>(r, st, lane, w);
    store_vec<D>(r + Rec<D>::kZ, vz, lane, w);
    store_vec<D>(r + Rec<D>::kP, vp, lane, w);
}

// ---------------------------------------------------------------------------------------
// total: per head, the sum of the segment records in segment order.  Records
// are loaded in batches ahead of the running sum.
template <int D>
__global__ __launch_bounds__(kBlock) void total_kernel(const float* __restrict__ rec, float* __restrict__ total,
                                                       int nseg) {
    constexpr int R4 = Rec<D>::kSize / 4;
    constexpr int NBLK = (R4 + kBlock - 1) / kBlock;
    constexpr int BATCH = 16;
    const int e4 = (blockIdx.x % NBLK) * kBlock + threadIdx.x;
    const int bh = blockIdx.x / NBLK;
    if (e4 >= R4) return;
    const f32x4* r = reinterpret_cast<const f32x4*>(rec) + (int64_t)bh * nseg * R4 + e4;
    f32x4 run = zero4();
    for (int i0 = 0; i0 < nseg; i0 += BATCH) {
        f32x4 x[BATCH];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) x[b] = i0 + b < nseg ? r[(int64_t)(i0 + b) * R4] : zero4();
#pragma unroll
        for (int b = 0; b < BATCH; ++b) run += x[b];
    }
    reinterpret_cast<f32x4*>(total)[(int64_t)bh * R4 + e4] = run;
}

// ---------------------------------------------------------------------------------------
// scan: per head, the segment records become, in place, exclusive running sums
// in segment order (dir > 0: record s holds the sum of records 0 .. s-1, the
// state before segment s) or from the last segment down (dir < 0: record s
// holds the sum of records nseg-1 .. s+1, the state after it).  The additions
// run in that order, one at a time, so each record is bitwise the sum a
// consumer would form itself.  Each thread carries one 16-byte column of the
// records through the head's segments.
template <int D>
__global__ __launch_bounds__(kBlock) void scan_kernel(float* __restrict__ rec, int nseg, int dir,
                                                      const float* __restrict__ init) {
    constexpr int R4 = Rec<D>::kSize / 4;
    constexpr int NBLK = (R4 + kBlock - 1) / kBlock;
    constexpr int BATCH = 8;
    const int e4 = (blockIdx.x % NBLK) * kBlock + threadIdx.x;
    const int bh = blockIdx.x / NBLK;
    if (e4 >= R4) return;
    f32x4* r = reinterpret_cast<f32x4*>(rec) + (int64_t)bh * nseg * R4 + e4;
    // init (nullable): one record per head the running sum starts from.
    f32x4 run = init != nullptr ? reinterpret_cast<const f32x4*>(init)[(int64_t)bh * R4 + e4] : zero4();
    for (int i0 = 0; i0 < nseg; i0 += BATCH) {
        f32x4 x[BATCH];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const int sg = dir > 0 ? i0 + b : nseg - 1 - (i0 + b);
            x[b] = i0 + b < nseg ? r[(int64_t)sg * R4] : zero4();
        }
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            if (i0 + b < nseg) {
                const int sg = dir > 0 ? i0 + b : nseg - 1 - (i0 + b);
                r[(int64_t)sg * R4] = run;
                run += x[b];
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// causal_fwd: per (segment, head), walk the segment's chunks from the state
// carried in by the segments before it.  The last segment of a head also
// writes the final state S = 1 P^T + S_E, z = N 1 + z_E when asked to.
//
// Eight wavefronts in two roles meet at one barrier per chunk.  While the
// output waves (0-3) compute chunk c's outputs from the state S(c) and the
// chunk's staged E(K), V, the state waves (4-7) stage chunk c+1 into the other
// buffers and form S(c+1) = S(c) + E(K_c)^T V_c, z_E and P from the same tiles.
// The two halves of the per-chunk work run side by side, and each role keeps
// only its own registers (more resident waves per SIMD).
//
// Per chunk and output wavefront (16 tokens t), all products on MFMA:
//   q_sum_t                    = ones . phi(Q_t)
//   A_ts = q_sum_t + phi(Q_t).E(K_s), s <= t, 32 keys per block, masked by lane bits
//   num^T[b][t] = sum_s V[s][b] A_ts + sum_a S_E^T[b][a] phi(Q_t)[a]     (tiles 0 .. D/16-1)
//   den_t - n q_sum_t = sum_s A_ts + sum_a z_E[a] phi(Q_t)[a]           (one more tile: an
//                      all-ones value column in the first product, z_E rows in the second)
// Chunk loops are unrolled by two so that each chunk's LDS buffer is a
// compile-time choice (its offsets fold into the instructions).
//
// kFused: the segment records are formed in the same launch.  Workgroups are then
// numbered segment-major, first segments first, and each one first forms its own
// segment's record (S_E, z_E, P) exactly as seg_state does (same tiles, same chunk
// order, so bitwise the same record), publishes it with agent-coherent stores and
// a per-launch flag, and waits (bounded) for the flags of the earlier segments of
// its head, whose workgroups were dispatched before it.  The carried state then
// sums their records as in the two-launch form.  A wait that gives up (a missing
// producer) makes the segment's outputs NaN and is counted in `giveups`.
// Whether a chunk held in registers has an inf or NaN element (exponent bits all ones).
template <typename T, int D>
__device__ __forceinline__ bool chunk_nonfinite(const ChunkRegs<T, D>& c) {
    bool bad = false;
#pragma unroll
    for (int i = 0; i < ChunkRegs<T, D>::NV; ++i) {
        const uint32_t w[4] = {c.r[i].x, c.r[i].y, c.r[i].z, c.r[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (sizeof(T) == 2)
                bad = bad || (w[j] & 0x7f80u) == 0x7f80u || (w[j] & 0x7f800000u) == 0x7f800000u;
            else
                bad = bad || (w[j] & 0x7f800000u) == 0x7f800000u;
        }
    }
    return bad;
}

template <typename T, int D>
struct CausalFwdCfg {
    // resident waves per SIMD the register allocation must allow (two workgroups per CU where
    // d <= 64 in bf16 and at d = 32 in fp32; fp32 tiles at d = 64 leave room for one)
    static constexpr int kWavesPerSimd = (D <= 64 && sizeof(T) == 2) || D <= 32 ? 4 : 2;
    // registers the state waves give to segment records in flight
    static constexpr int kRecordRegs = D <= 64 ? 48 : 128;
};

template <typename T, int D, class FM = FeatElu, bool kFused = false>
__global__ __launch_bounds__(2 * kBlock, (CausalFwdCfg<T, D>::kWavesPerSimd)) void causal_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ o,
    float* __restrict__ den_out, float* __restrict__ rec, float* __restrict__ S_out, float* __restrict__ z_out,
    const float* __restrict__ init, const float* __restrict__ init_n, int N, int cps, int nseg, int BH,
    int prefixed, int G, int Gv, unsigned long long* __restrict__ flags, unsigned* __restrict__ giveups,
    unsigned long long epoch, int wait_limit) {
    using M = Mma<T>;
    using F = typename M::frag;
    constexpr int KS = M::KSTEP;
    constexpr int DT = D / 16;
    // One block of LDS, so that the fused form can lay a whole fp32 record over
    // the tiles before the sweep starts.
    struct Lds {
        T e[2][kC * D], v[2][kC * D], st[2][D * D], zb[2][D];
        float p[2][D];
    };
    static_assert(sizeof(T) * (4 * kC * D + 2 * D * D) >= sizeof(float) * Rec<D>::kSize,
                  "a record fits over the tiles");
    __shared__ __attribute__((aligned(16))) Lds sm;
    T(&sm_e)[2][kC * D] = sm.e;
    T(&sm_v)[2][kC * D] = sm.v;
    T(&sm_st)[2][D * D] = sm.st;
    T(&s_zb)[2][D] = sm.zb;
    float(&s_p)[2][D] = sm.p;

    // Later segments sum more records: they are dispatched first, since a CU's
    // older workgroup issues ahead of its younger one (fused: first segments
    // first, so that every record waited on has a producer dispatched earlier).
    const int seg = kFused ? (int)(blockIdx.x / BH) : nseg - 1 - (int)(blockIdx.x / BH), bh = blockIdx.x % BH;
    // Query head bh reads the keys, values, records and start state of key/value
    // head kv (G query heads share one: grouped heads; G = 1: one each), and the
    // values of head kv / Gv (feature blocks of one head share its values).
    const int kv = bh / G;
    const int wv = wave_id(), lane = threadIdx.x & 63, g = lane >> 4;
    const int w = wv & 3;                     // wave index inside its role
    const int rtid = (int)threadIdx.x & (kBlock - 1);  // thread index inside its role
    const int64_t hoff = (int64_t)bh * N * D, kvoff = (int64_t)kv * N * D, voff = (int64_t)(kv / Gv) * N * D;
    const uint32_t hbytes = (uint32_t)N * D * sizeof(T);
    const int tok_begin = seg * cps * kC;
    const int tok_end = min(N, tok_begin + cps * kC);
    // fused: the head's records (this launch writes them; read agent-coherent)
    const GBuf brec(rec + (int64_t)kv * nseg * Rec<D>::kSize, (uint32_t)(nseg * Rec<D>::kSize * 4));
    bool ok = true;  // fused: every earlier segment's record arrived

    if constexpr (!kFused) {
        // This form waits for nothing: its wait counts (when the workspace keeps them) are zero.
        if (giveups != nullptr && threadIdx.x == 0) giveups[(int64_t)bh * nseg + seg] = 0u;
    } else {
        // ---- the segment's own record, as seg_state forms it ------------------------------
        // The state waves stage E(K) and form the record; the output waves, idle until the
        // sweep, stage V.  Each role keeps the next two chunks of its tensor in flight (two
        // register sets, chunk c in set c mod 2): the phase streams from HBM.  (At d = 128
        // the registers are the sweep's: there the state waves stream both, one chunk ahead.)
        auto next2 = [&](int c0) { return c0 + 2 * kC < tok_end ? c0 + 2 * kC : N; };  // past the segment: zeros
        if (D > 64 && wv >= 4) {
            const GBuf bk(k + kvoff, hbytes), bv(v + voff, hbytes);
            ChunkRegs<T, D> ck, cv;
            ck.load(bk, tok_begin, rtid);
            cv.load(bv, tok_begin, rtid);
            StateAcc<D> st;
            VecAcc<D> vz, vp;
            zero_state<D>(st);
            zero_vec<D>(vz);
            zero_vec<D>(vp);
            for (int c0 = tok_begin, b = 0; c0 < tok_end; c0 += kC, b ^= 1) {
                stage_elu<T, D, FM>(ck, Tile<T, kC, D>{sm_e[b]}, rtid);
                stage_raw<T, D>(cv, Tile<T, kC, D>{sm_v[b]}, rtid);
                ck.load(bk, c0 + kC < tok_end ? c0 + kC : N, rtid);
                cv.load(bv, c0 + kC < tok_end ? c0 + kC : N, rtid);
                __syncthreads();
                state_update<T, D, true, true>(st, vz, vp, Tile<T, kC, D>{sm_e[b]}, Tile<T, kC, D>{sm_v[b]}, nullptr,
                                               nullptr, lane, w);
            }
            store_record_coherent<D>(brec, (int64_t)seg * Rec<D>::kSize, st, vz, &vp, lane, w);
            wait_all_memory();
        } else if (D > 64) {
            for (int c0 = tok_begin; c0 < tok_end; c0 += kC) __syncthreads();
        } else if (wv >= 4) {
            const GBuf bk(k + kvoff, hbytes);
            ChunkRegs<T, D> ck0, ck1;
            ck0.load(bk, tok_begin, rtid);
            ck1.load(bk, tok_begin + kC < tok_end ? tok_begin + kC : N, rtid);
            StateAcc<D> st;
            VecAcc<D> vz, vp;
            zero_state<D>(st);
            zero_vec<D>(vz);
            zero_vec<D>(vp);
            auto chunk = [&](auto bsel, ChunkRegs<T, D>& ck, int c0) {
                constexpr int B = decltype(bsel)::value;
                stage_elu<T, D, FM>(ck, Tile<T, kC, D>{sm_e[B]}, rtid);
                ck.load(bk, next2(c0), rtid);
                __syncthreads();
                state_update<T, D, true, true>(st, vz, vp, Tile<T, kC, D>{sm_e[B]}, Tile<T, kC, D>{sm_v[B]}, nullptr,
                                               nullptr, lane, w);
            };
            for (int c0 = tok_begin; c0 < tok_end; c0 += 2 * kC) {
                chunk(std::integral_constant<int, 0>{}, ck0, c0);
                if (c0 + kC >= tok_end) break;
                chunk(std::integral_constant<int, 1>{}, ck1, c0 + kC);
            }
            store_record_coherent<D>(brec, (int64_t)seg * Rec<D>::kSize, st, vz, &vp, lane, w);
            wait_all_memory();
        } else {
            const GBuf bv(v + voff, hbytes);
            ChunkRegs<T, D> cv0, cv1;
            cv0.load(bv, tok_begin, rtid);
            cv1.load(bv, tok_begin + kC < tok_end ? tok_begin + kC : N, rtid);
            auto chunk = [&](auto bsel, ChunkRegs<T, D>& cv, int c0) {
                constexpr int B = decltype(bsel)::value;
                stage_raw<T, D>(cv, Tile<T, kC, D>{sm_v[B]}, rtid);
                cv.load(bv, next2(c0), rtid);
                __syncthreads();
            };
            for (int c0 = tok_begin; c0 < tok_end; c0 += 2 * kC) {
                chunk(std::integral_constant<int, 0>{}, cv0, c0);
                if (c0 + kC >= tok_end) break;
                chunk(std::integral_constant<int, 1>{}, cv1, c0 + kC);
            }
        }
        __syncthreads();  // every state wave's record stores are complete
    }

    // fused: post this segment's flag, wait for the earlier segments' (bounded), and
    // sum init + their records (every thread of the workgroup at once) into LDS over
    // the idle tiles, bitwise what carried_state forms.  The records are awaited batch
    // by batch, so that the first batches are read and summed while the last segments'
    // records (their producers finish last) are still on their way.  Called by both
    // roles, so that each keeps its own first-chunk loads in flight meanwhile; true if
    // every record arrived.
    __shared__ int s_ok;
    // The last segment of a running-sum plan has no record after it to tell whether its
    // values hold an inf or NaN; there the state waves flag each staged chunk of V (one
    // flag per state wave) and the output waves take the non-finite path only for chunks
    // that have one.
    __shared__ int s_vf[2][4];
    const bool vchk = prefixed != 0 && seg + 1 >= nseg;
    float* const xs = reinterpret_cast<float*>(&sm);
    auto fused_records = [&]() -> bool {
        unsigned long long* hf = flags + (int64_t)bh * nseg;
        if (threadIdx.x == 0) {
            post_flag(&hf[seg], epoch);
            s_ok = 1;
        }
        auto ready = [&](int j0, int j1) {
            if (threadIdx.x == 0) {
                bool all = s_ok != 0;
                for (int j = j0; j < j1; ++j) all = all && await_flag(&hf[j], epoch, wait_limit);
                s_ok = all ? 1 : 0;
            }
            __syncthreads();
        };
        sum_records_to<D, 2 * kBlock>(RecCoherent{brec}, 0, Rec<D>::kSize, seg,
                                      init != nullptr ? init + (int64_t)kv * Rec<D>::kSize : nullptr, xs,
                                      (int)threadIdx.x, ready);
        // The host reads these counts back (la_wait_failures): a give-up leaves NaN rows
        // that must not pass for a result of the data.
        if (threadIdx.x == 0) giveups[(int64_t)bh * nseg + seg] = s_ok != 0 ? 0u : 1u;
        __syncthreads();
        return s_ok != 0;
    };

    if (wv >= 4) {
        // ---- state waves -------------------------------------------------------------
        const GBuf bk(k + kvoff, hbytes), bv(v + voff, hbytes);
        // The first chunk's loads are in flight while the starting state arrives:
        // the records of the segments before this one, summed in order.
        ChunkRegs<T, D> ck, cv;
        ck.load(bk, tok_begin, rtid);
        cv.load(bv, tok_begin, rtid);
        StateAcc<D> st;
        VecAcc<D> vz, vp;
        if constexpr (kFused) {
            ok = fused_records();
            if (2 * seg >= nseg) __builtin_amdgcn_s_setprio(1);  // as the output waves below
            load_state<D>(xs, st, lane, w);
            load_vec<D>(xs + Rec<D>::kZ, vz, lane, w);
            load_vec<D>(xs + Rec<D>::kP, vp, lane, w);
            __syncthreads();  // the sum is read before any wave stages tiles over it
            if (!ok) {  // a record never arrived: the segment's outputs become NaN
                using ST = StateTiles<D>;
                const float nan = __builtin_nanf("");
#pragma unroll
                for (int ia = 0; ia < ST::NAT; ++ia)
#pragma unroll
                    for (int ib = 0; ib < ST::NBT; ++ib) st[ia][ib] = splat4(nan);
#pragma unroll
                for (int x = 0; x < ST::NVT; ++x) vz[x] = splat4(nan);
            }
        } else {
            carried_state<D, CausalFwdCfg<T, D>::kRecordRegs>(rec + (int64_t)kv * nseg * Rec<D>::kSize, Rec<D>::kSize,
                                                             seg, prefixed != 0, st, vz, vp, lane, w,
                                                             init != nullptr ? init + (int64_t)kv * Rec<D>::kSize
                                                                             : nullptr);
        }
        publish_state<T, D>(st, Tile<T, D, D>{sm_st[0]}, lane, w);
        store_vec_as<T, D>(s_zb[0], vz, lane, w);
        store_vec<D>(s_p[0], vp, lane, w);
        stage_elu<T, D, FM>(ck, Tile<T, kC, D>{sm_e[0]}, rtid);
        stage_raw<T, D>(cv, Tile<T, kC, D>{sm_v[0]}, rtid);
        if (vchk) {
            const bool nf = __builtin_amdgcn_ballot_w64(chunk_nonfinite(cv)) != 0;
            if (lane == 0) s_vf[0][w] = nf ? 1 : 0;
        }
        // Loads past the segment are aimed at row N: out of the buffer's range, they
        // return zeros without touching memory, and the loop stays branch free.
        ck.load(bk, tok_begin + kC < tok_end ? tok_begin + kC : N, rtid);
        cv.load(bv, tok_begin + kC < tok_end ? tok_begin + kC : N, rtid);
        __syncthreads();

        auto chunk = [&](auto bsel, int c0) {
            constexpr int B = decltype(bsel)::value;
            // Stage the next chunk into the other buffer (idle after the last chunk),
            // then S_E += E(K)^T V, z_E += colsum E(K), P += colsum V, published
            // for the next chunk.
            stage_elu<T, D, FM>(ck, Tile<T, kC, D>{sm_e[B ^ 1]}, rtid);
            stage_raw<T, D>(cv, Tile<T, kC, D>{sm_v[B ^ 1]}, rtid);
            if (vchk) {
                const bool nf = __builtin_amdgcn_ballot_w64(chunk_nonfinite(cv)) != 0;
                if (lane == 0) s_vf[B ^ 1][w] = nf ? 1 : 0;
            }
            ck.load(bk, c0 + 2 * kC < tok_end ? c0 + 2 * kC : N, rtid);
            cv.load(bv, c0 + 2 * kC < tok_end ? c0 + 2 * kC : N, rtid);
            state_update<T, D, true, true>(st, vz, vp, Tile<T, kC, D>{sm_e[B]}, Tile<T, kC, D>{sm_v[B]}, nullptr,
                                           nullptr, lane, w);
            publish_state<T, D>(st, Tile<T, D, D>{sm_st[B ^ 1]}, lane, w);
            store_vec_as<T, D>(s_zb[B ^ 1], vz, lane, w);
            store_vec<D>(s_p[B ^ 1], vp, lane, w);
            __syncthreads();
        };
        for (int c0 = tok_begin; c0 < tok_end; c0 += 2 * kC) {
            chunk(std::integral_constant<int, 0>{}, c0);
            if (c0 + kC >= tok_end) break;
            chunk(std::integral_constant<int, 1>{}, c0 + kC);
        }

        if (seg == nseg - 1 && bh % G == 0) {  // one query head of the group writes its state
            // P of the whole head was published into s_p[nch & 1] before the last barrier.
            using ST = StateTiles<D>;
            const int nch = (tok_end - tok_begin + kC - 1) / kC;
            if (S_out != nullptr) {
                const float* sp = s_p[nch & 1];
                float* s = S_out + (int64_t)kv * D * D;
#pragma unroll
                for (int ia = 0; ia < ST::NAT; ++ia)
#pragma unroll
                    for (int ib = 0; ib < ST::NBT; ++ib) {
                        const int b = (ST::bt0(w) + ib) * 16 + (lane & 15);
                        const float pb = sp[b];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            s[(int64_t)((ST::at0(w) + ia) * 16 + 4 * g + e) * D + b] =
                                FM::kSplit ? pb + st[ia][ib][e] : st[ia][ib][e];
                    }
            }
            if (z_out != nullptr && ST::owns_vec(w) && (lane & 15) == 0) {
#pragma unroll
                for (int x = 0; x < ST::NVT; ++x)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        z_out[(int64_t)kv * D + (ST::vt0(w) + x) * 16 + 4 * g + e] =
                            FM::kSplit ? (init_n != nullptr ? init_n[kv] + (float)N : (float)N) + vz[x][e]
                                       : vz[x][e];
            }
        }
        return;
    }

    // ---- output waves ------------------------------------------------------------------
    // Whether the segment's values hold an inf or NaN.  Masked in-chunk weights are
    // exact zeros, but 0 * inf = NaN: the block of 32 keys holding the diagonal then
    // takes its value operands with non-finite entries replaced by 0, and the rows
    // t >= s that such a value V_s[b] reaches get O_t[b] = NaN back explicitly, so no
    // row reads a later token (the recurrent form of "Why It Matters").  The segment's
    // own record holds P = the sum of its values, non-finite exactly then; with
    // running-sum records the next one (which includes this segment) stands in, and
    // the last segment of such a plan always takes the path.
    bool vbad;
    {
        const int own = prefixed ? seg + 1 : seg;
        bool bad = own >= nseg;
        if (!bad) {
            const int64_t p = (int64_t)own * Rec<D>::kSize + Rec<D>::kP;
#pragma unroll
            for (int i = 0; i < (D + kWave - 1) / kWave; ++i)
                if (i * kWave + lane < D)
                    bad = bad || !finite_f(kFused ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                                        brec.r, (uint32_t)((p + i * kWave + lane) * 4), 0,
                                                        GBuf::kCoherent))
                                                  : rec[(int64_t)kv * nseg * Rec<D>::kSize + p + i * kWave + lane]);
        }
        vbad = __builtin_amdgcn_ballot_w64(bad) != 0;
    }
    const GBuf bq(q + hoff, hbytes), bo(o + hoff, hbytes);
    const GBuf bden(den_out != nullptr ? den_out + (int64_t)bh * N : nullptr, den_out != nullptr ? (uint32_t)N * 4 : 0u);
    // Tokens before the chunk (the count of the rank-1 part of z), from the start state's count.
    float n = init_n != nullptr ? init_n[kv] + (float)tok_begin : (float)tok_begin;
    // Wavefront w takes token tile tt = (w + ci) mod 4 of chunk ci: the causal
    // mask leaves tt + 1 key tiles, and the rotation spreads that work evenly
    // over the SIMDs.
    RowFrag<T, D> qr;
    qr.load(bq, tok_begin + 16 * w, lane);
    if constexpr (kFused) {
        fused_records();
        __syncthreads();  // (the state waves read the sum)
        // The second half of the segments (dispatched last, so usually the younger of
        // the two workgroups on a CU, the one the SIMDs serve second) wait for the most
        // records and start their sweeps last: they take the higher wave priority for it.
        if (2 * seg >= nseg) __builtin_amdgcn_s_setprio(1);
    }
    // Key s = 16 j + 4 g + e of tile j is visible to token t = 16 tt + (lane & 15)
    // iff j < tt, or j == tt and bit lane of diag[e] is set.
    uint64_t diag[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) diag[e] = __ballot(4 * g + e <= (lane & 15));
    const float zero = opaque_zero();
    const F one = M::ones();
    __syncthreads();

    auto chunk = [&](auto bsel, int c0, int ci) {
        constexpr int B = decltype(bsel)::value;
        const Tile<T, kC, D> tE{sm_e[B]}, tV{sm_v[B]};
        const Tile<T, D, D> tSt{sm_st[B]};
        const bool more = c0 + kC < tok_end;
        const int tt = (w + ci) & 3;
        const bool cbad = vbad && (!vchk || (s_vf[B][0] | s_vf[B][1] | s_vf[B][2] | s_vf[B][3]) != 0);
        const int tl = 16 * tt + (lane & 15);  // this lane's token (accumulator column)

        F qf[D / KS];
        qr.template phi_ops<FM>(qf);
        qr.load(bq, more ? c0 + kC + 16 * ((w + ci + 1) & 3) : N, lane);
        // q_sum_t, the weight of the rank-1 parts (unsplit features have none).
        float qs_t = 0.f;
        if constexpr (FM::kSplit) {
            f32x4 acc_q = zero4();
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += KS) acc_q = M::mma(one, qf[k0 / KS], acc_q);
            qs_t = acc_q[0];
        }

        f32x4 acc[DT + 1];
#pragma unroll
        for (int m = 0; m <= DT; ++m) acc[m] = zero4();
        // In-chunk part, 32 keys (two tiles) per block; blocks past the diagonal are skipped.
#pragma unroll
        for (int kb = 0; kb < kC / 32; ++kb) {
            if (2 * kb <= tt) {
                f32x4 a[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int j = 2 * kb + h;
                    a[h] = splat4(qs_t);
#pragma unroll
                    for (int k0 = 0; k0 < D; k0 += KS) a[h] = M::mma(M::ld(tE, 16 * j, k0, lane), qf[k0 / KS], a[h]);
                    // all ones when j < tt (resp. j <= tt), from sign shifts: scalar only
                    const uint64_t lt = ~(uint64_t)((int64_t)(tt - j - 1) >> 63);
                    const uint64_t le = ~(uint64_t)((int64_t)(tt - j) >> 63);
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[h][e] = lane_bit(lt | (le & diag[e])) ? a[h][e] : zero;
                }
                auto av = [&](auto san) {
#pragma unroll
                    for (int kk = 0; kk < 32; kk += KS) {
                        const F yf = M::acc_op(a, kk);
#pragma unroll
                        for (int m = 0; m < DT; ++m) {
                            F vf = M::ld_tr_acc(tV, 32 * kb + kk, 16 * m, lane);
                            if constexpr (decltype(san)::value) vf = finite_or_zero(vf);
                            acc[m] = M::mma(vf, yf, acc[m]);
                        }
                        acc[DT] = M::mma(one, yf, acc[DT]);
                    }
                };
                if (cbad && 2 * kb + 1 >= tt)  // the block holding the diagonal tile
                    av(std::true_type{});
                else
                    av(std::false_type{});
            }
        }
        // State part: S_E^T phi(Q_t) and z_E . phi(Q_t).
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += KS) {
            const F yf = qf[k0 / KS];
#pragma unroll
            for (int m = 0; m < DT; ++m) acc[m] = M::mma(M::ld(tSt, 16 * m, k0, lane), yf, acc[m]);
            acc[DT] = M::mma(M::vec_op(s_zb[B], k0, lane), yf, acc[DT]);
        }
        const float den = acc[DT][0] + n * qs_t;
        const float inv = rcp_f(den);
        const int tok = c0 + tl;  // rows past the head are dropped by the buffer range
#pragma unroll
        for (int m = 0; m < DT; ++m) {
            const int b0 = 16 * m + 4 * g;
            const f32x4 p4 = lds4(&s_p[B][b0]);
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (acc[m][e] + qs_t * p4[e]) * inv;
            if (cbad) {  // the non-finite values of keys s <= t that the diagonal block dropped
                for (int s = 32 * (tt >> 1); s <= tl; ++s) {
                    const f32x4 vv = lds4(&tV.at(s, b0));
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] += vv[e] - vv[e];  // 0, or NaN
                }
            }
            gstore4<T>(bo, (uint32_t)(tok * D + b0), x);
        }
        if (den_out != nullptr && g == 0) bden.st4f((uint32_t)tok * 4, den);
        n += (float)min(kC, N - c0);
        __syncthreads();
    };
    for (int c0 = tok_begin, ci = 0; c0 < tok_end; c0 += 2 * kC, ci += 2) {
        chunk(std::integral_constant<int, 0>{}, c0, ci);
        if (c0 + kC >= tok_end) break;
        chunk(std::integral_constant<int, 1>{}, c0 + kC, ci + 1);
    }
}

// ---------------------------------------------------------------------------------------
// noncausal_fwd: every row reads the head's total state; each wavefront works
// on its own token tiles with phi(Q) in registers (no barrier in the loop).
template <typename T, int D, class FM = FeatElu>
__global__ __launch_bounds__(kBlock) void noncausal_fwd_kernel(const T* __restrict__ q, T* __restrict__ o,
                                                               float* __restrict__ den_out,
                                                               const float* __restrict__ total, int ntotal, int N,
                                                               int cps, int nseg, int BH) {
    using M = Mma<T>;
    constexpr int KS = M::KSTEP;
    constexpr int DT = D / 16;
    __shared__ __attribute__((aligned(16))) T sm_st[D * D];
    __shared__ __attribute__((aligned(16))) float s_z[D], s_p[D];
    const Tile<T, D, D> tSt{sm_st};

    const int seg = blockIdx.x / BH, bh = blockIdx.x % BH;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 4;
    const int64_t hoff = (int64_t)bh * N * D;
    const uint32_t hbytes = (uint32_t)N * D * sizeof(T);
    const GBuf bq(q + hoff, hbytes), bo(o + hoff, hbytes);
    const int tok_begin = seg * cps * kC;
    const int tok_end = min(N, tok_begin + cps * kC);
    // The head's state: the sum of its ntotal records in order (ntotal = nseg:
    // the segment records themselves; ntotal = 1: a precomputed total).
    {
        StateAcc<D> st;
        VecAcc<D> vz, vp;
        zero_state<D>(st);
        zero_vec<D>(vz);
        zero_vec<D>(vp);
        add_records<D>(total + (int64_t)bh * ntotal * Rec<D>::kSize, Rec<D>::kSize, ntotal, st, vz, vp, lane, w);
        publish_state<T, D>(st, tSt, lane, w);
        store_vec<D>(s_z, vz, lane, w);
        store_vec<D>(s_p, vp, lane, w);
    }
    const float n = (float)N;
    const int t0 = 16 * w;
    const int tl = t0 + (lane & 15);
    RowFrag<T, D> qr;
    qr.load(bq, tok_begin + t0, lane);
    __syncthreads();

    for (int c0 = tok_begin; c0 < tok_end; c0 += kC) {
        typename M::frag qf[D / KS];
        const float zdot = sum_over_groups(qr.template phi_ops<FM>(qf, s_z, lane));
        qr.load(bq, c0 + kC < tok_end ? c0 + kC + t0 : N, lane);
        const typename M::frag one = M::ones();
        f32x4 acc_q = zero4();
        f32x4 acc[DT];
#pragma unroll
        for (int m = 0; m < DT; ++m) acc[m] = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += KS) {
            const typename M::frag yf = qf[k0 / KS];
            if constexpr (FM::kSplit) acc_q = M::mma(one, yf, acc_q);
#pragma unroll
            for (int m = 0; m < DT; ++m) acc[m] = M::mma(M::ld(tSt, 16 * m, k0, lane), yf, acc[m]);
        }
        const float qs_t = FM::kSplit ? acc_q[0] : 0.f;  // weight of the rank-1 parts (none when unsplit)
        const float den = n * qs_t + zdot;
        const float inv = rcp_f(den);
        const int tok = c0 + tl;
        if (den_out != nullptr && g == 0 && tok < tok_end) den_out[(int64_t)bh * N + tok] = den;
#pragma unroll
        for (int m = 0; m < DT; ++m) {
            const int b0 = 16 * m + 4 * g;
            const f32x4 p4 = lds4(&s_p[b0]);
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (acc[m][e] + qs_t * p4[e]) * inv;
            gstore4<T>(bo, (uint32_t)(tok * D + b0), x);
        }
    }
}

// ---------------------------------------------------------------------------------------
// state_split: a start state (S0, z0) given as plain sums, rewritten in the split
// form the kernels carry: S0 = 1 P0^T + S0_E, z0 = n0 1 + z0_E with P0 and n0 the
// means over the feature index a, so that S0_E and z0_E hold only the deviations
// (as small as a prefix's own S_E, z_E; the rank-1 parts stay in fp32).  Out: the
// record [S0_E^T | z0_E | P0] and n0 per head.  Either input may be null (zero).
// split = 0 (features carried unsplit): P0 = 0, n0 = 0, the record is S0, z0 itself.
// init_n may be null (no count wanted).
// The state is staged through LDS (rows padded by one float) so that both its reads
// and the transposed record's writes are coalesced; column b's mean is summed by
// thread b in feature order (fixed order: bitwise reproducible).
template <int D>
__global__ __launch_bounds__(kBlock) void state_split_kernel(const float* __restrict__ S0, const float* __restrict__ z0,
                                                             float* __restrict__ init, float* __restrict__ init_n,
                                                             int split) {
    __shared__ float s_S[D][D + 1];
    __shared__ float s_p[D];
    __shared__ float s_n;
    const int bh = blockIdx.x, tid = threadIdx.x;
    float* r = init + (int64_t)bh * Rec<D>::kSize;
    const float* Sh = S0 != nullptr ? S0 + (int64_t)bh * D * D : nullptr;
    const float* zh = z0 != nullptr ? z0 + (int64_t)bh * D : nullptr;
    constexpr int D4 = D / 4;
    for (int i = tid; i < D * D4; i += kBlock) {  // row i / D4, columns 4 (i % D4) ..
        const int aa = i / D4, c = 4 * (i % D4);
        const f32x4 x = Sh != nullptr ? *reinterpret_cast<const f32x4*>(Sh + aa * D + c) : zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e) s_S[aa][c + e] = x[e];
    }
    if (tid == kBlock - 1) {  // n0: the mean of z0 over the features
        float n0 = 0.f;
        if (zh != nullptr && split) {
            for (int a = 0; a < D; ++a) n0 += zh[a];
            n0 *= 1.f / (float)D;
        }
        s_n = n0;
        if (init_n != nullptr) init_n[bh] = n0;
    }
    __syncthreads();
    if (tid < D) {  // P0[b]: the mean of column b
        float p = 0.f;
        if (Sh != nullptr && split) {
            for (int a = 0; a < D; ++a) p += s_S[a][tid];
            p *= 1.f / (float)D;
        }
        s_p[tid] = p;
        r[Rec<D>::kP + tid] = p;
    }
    __syncthreads();
    // Record [S0_E^T | z0_E | P0]: element (b, a) of the transposed block is S0[a][b] - P0[b].
    for (int i = tid; i < D * D4; i += kBlock) {  // row i / D4 of the block, columns 4 (i % D4) ..
        const int bb = i / D4, a0 = 4 * (i % D4);
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = s_S[a0 + e][bb] - s_p[bb];
        *reinterpret_cast<f32x4*>(r + Rec<D>::kSt + bb * D + a0) = y;
    }
    if (tid < D) r[Rec<D>::kZ + tid] = zh != nullptr ? zh[tid] - s_n : 0.f;  // feature tid of z0_E
}

// dst[i] = src[i], or 0 when src is null.
__global__ __launch_bounds__(kBlock) void fill_zero_kernel(float* __restrict__ p, const float* __restrict__ src,
                                                           size_t n) {
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (size_t)gridDim.x * kBlock)
        p[i] = src != nullptr ? src[i] : 0.f;
}

// ---------------------------------------------------------------------------------------
// Host launchers.
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

hipError_t launch_state_split(int d, const float* S0, const float* z0, float* init, float* init_n, int64_t BH,
                              hipStream_t s, int feat) {
    LA_DISPATCH_D(d, hipLaunchKernelGGL((state_split_kernel<D>), dim3((unsigned)BH), dim3(kBlock), 0, s, S0, z0, init,
                                        init_n, feat == kFeatGiven ? 0 : 1));
    return hipGetLastError();
}

hipError_t launch_copy_or_zero(float* p, const float* src, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, p, src, n);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s) { return launch_copy_or_zero(p, nullptr, n, s); }

// ---------------------------------------------------------------------------------------
// Pieces of the fp32 causal forward at d = 128, which runs on feature blocks (its fp32
// tiles at d = 128 do not fit a CU's LDS): phi_blocks writes phi(x) = elu(x) + 1 of
// x [heads][N][KF db] in block layout [heads][KF][N][db]; copy_cols moves a block of
// `cols` columns between row-major fp32 matrices of different widths.
__global__ __launch_bounds__(kBlock) void phi_blocks_kernel(const float* __restrict__ x, float* __restrict__ out,
                                                            int64_t heads, int64_t N, int KF, int db) {
    const int64_t q4 = db / 4;                          // 16-byte groups per block row
    const int64_t total = heads * N * KF * q4;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBlock) {
        const int64_t c4 = i % q4, r = i / q4;           // r = (head, row, block): input order
        const int64_t j = r % KF, hn = r / KF, n = hn % N, h = hn / N;
        const f32x4 a = *reinterpret_cast<const f32x4*>(x + (hn * KF + j) * db + 4 * c4);
        f32x4 b;
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = phi_f(a[e]);
        *reinterpret_cast<f32x4*>(out + ((h * KF + j) * N + n) * db + 4 * c4) = b;
    }
}

__global__ __launch_bounds__(kBlock) void copy_cols_kernel(float* __restrict__ dst, int64_t dst_ld,
                                                           const float* __restrict__ src, int64_t src_ld,
                                                           int64_t rows, int cols) {
    const int64_t q4 = cols / 4, total = rows * q4;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBlock) {
        const int64_t r = i / q4, c4 = i % q4;
        *reinterpret_cast<f32x4*>(dst + r * dst_ld + 4 * c4) = *reinterpret_cast<const f32x4*>(src + r * src_ld + 4 * c4);
    }
}

// The gradient back through phi_blocks for two sets of feature gradients (the value halves'):
// dx [heads][N][KF db] = (dF0 + dF1 in block layout) * phi'(x), phi'(x) = exp(min(x, 0)).
__global__ __launch_bounds__(kBlock) void phi_blocks_grad_kernel(const float* __restrict__ x,
                                                                 const float* __restrict__ dF0,
                                                                 const float* __restrict__ dF1, float* __restrict__ dx,
                                                                 int64_t heads, int64_t N, int KF, int db) {
    const int64_t q4 = db / 4;
    const int64_t total = heads * N * KF * q4;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBlock) {
        const int64_t c4 = i % q4, r = i / q4;
        const int64_t j = r % KF, hn = r / KF, n = hn % N, h = hn / N;
        const int64_t bo = ((h * KF + j) * N + n) * db + 4 * c4, xo = (hn * KF + j) * db + 4 * c4;
        const f32x4 a = *reinterpret_cast<const f32x4*>(x + xo);
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(dF0 + bo), g1 = *reinterpret_cast<const f32x4*>(dF1 + bo);
        f32x4 r4;
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] = (g0[e] + g1[e]) * dphi_f(a[e]);
        *reinterpret_cast<f32x4*>(dx + xo) = r4;
    }
}

hipError_t launch_phi_blocks_grad(const float* x, const float* dF0, const float* dF1, float* dx, int64_t heads,
                                  int64_t N, int KF, int db, hipStream_t s) {
    if (db % 4 != 0) return hipErrorInvalidValue;
    const int64_t total = heads * N * KF * (db / 4);
    if (total == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((total + kBlock - 1) / kBlock, 8192);
    hipLaunchKernelGGL(phi_blocks_grad_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, x, dF0, dF1, dx, heads, N,
                       KF, db);
    return hipGetLastError();
}

hipError_t launch_phi_blocks(const float* x, float* out, int64_t heads, int64_t N, int KF, int db, hipStream_t s) {
    if (db % 4 != 0) return hipErrorInvalidValue;
    const int64_t total = heads * N * KF * (db / 4);
    if (total == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((total + kBlock - 1) / kBlock, 8192);
    hipLaunchKernelGGL(phi_blocks_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, x, out, heads, N, KF, db);
    return hipGetLastError();
}

hipError_t launch_copy_cols(float* dst, int64_t dst_ld, const float* src, int64_t src_ld, int64_t rows, int cols,
                            hipStream_t s) {
    if (cols % 4 != 0) return hipErrorInvalidValue;
    const int64_t total = rows * (cols / 4);
    if (total == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((total + kBlock - 1) / kBlock, 8192);
    hipLaunchKernelGGL(copy_cols_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, dst, dst_ld, src, src_ld, rows,
                       cols);
    return hipGetLastError();
}

template <class FM>
static hipError_t launch_seg_state_fm(int dt, int d, const void* k, const void* v, float* rec, int64_t BH, int64_t N,
                                      SegPlan p, hipStream_t s, int Gv) {
    const dim3 grid((unsigned)(p.nseg * BH));
    if (dt == kBF16) {
        LA_DISPATCH_D(d, hipLaunchKernelGGL((seg_state_kernel<bf16, D, FM>), grid, dim3(kBlock), 0, s, (const bf16*)k,
                                            (const bf16*)v, rec, (int)N, p.cps, p.nseg, (int)BH, Gv));
    } else {
        LA_DISPATCH_D(d, hipLaunchKernelGGL((seg_state_kernel<float, D, FM>), grid, dim3(kBlock), 0, s, (const float*)k,
                                            (const float*)v, rec, (int)N, p.cps, p.nseg, (int)BH, Gv));
    }
    return hipGetLastError();
}

hipError_t launch_seg_state(int dt, int d, const void* k, const void* v, float* rec, int64_t BH, int64_t N,
                            SegPlan p, hipStream_t s, int feat, int Gv) {
    return feat == kFeatGiven ? launch_seg_state_fm<FeatGiven>(dt, d, k, v, rec, BH, N, p, s, Gv)
                              : launch_seg_state_fm<FeatElu>(dt, d, k, v, rec, BH, N, p, s, Gv);
}

hipError_t launch_total(int d, const float* rec, float* total, int64_t BH, int nseg, hipStream_t s) {
    const int r4 = (int)(rec_floats(d) / 4);
    const dim3 grid((unsigned)(((r4 + kBlock - 1) / kBlock) * BH));
    LA_DISPATCH_D(d, hipLaunchKernelGGL((total_kernel<D>), grid, dim3(kBlock), 0, s, rec, total, nseg));
    return hipGetLastError();
}

hipError_t launch_scan(int d, float* rec, int64_t BH, int nseg, int dir, hipStream_t s, const float* init) {
    const int r4 = (int)(rec_floats(d) / 4);
    const dim3 grid((unsigned)(((r4 + kBlock - 1) / kBlock) * BH));
    LA_DISPATCH_D(d, hipLaunchKernelGGL((scan_kernel<D>), grid, dim3(kBlock), 0, s, rec, nseg, dir, init));
    return hipGetLastError();
}

template <class FM, bool kFused>
static hipError_t launch_causal_fwd_fm(int dt, int d, const void* q, const void* k, const void* v, void* o,
                                       float* den_out, float* rec, float* S_out, float* z_out, int64_t BH,
                                       int64_t N, SegPlan p, hipStream_t s, const float* init, const float* init_n,
                                       int G, int Gv, unsigned long long* flags, unsigned* giveups,
                                       unsigned long long epoch, int wait_limit) {
    const dim3 grid((unsigned)(p.nseg * BH));
#define LA_CFWD(TT, DD)                                                                                          \
    hipLaunchKernelGGL((causal_fwd_kernel<TT, DD, FM, kFused>), grid, dim3(2 * kBlock), 0, s, (const TT*)q,       \
                       (const TT*)k, (const TT*)v, (TT*)o, den_out, rec, S_out, z_out, init, init_n, (int)N, p.cps, \
                       p.nseg, (int)BH, (int)p.scan, G, Gv, flags, giveups, epoch, wait_limit)
    if (dt == kBF16) {
        switch (d) {
            case 32: LA_CFWD(bf16, 32); break;
            case 64: LA_CFWD(bf16, 64); break;
            case 128: LA_CFWD(bf16, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (d) {
            case 32: LA_CFWD(float, 32); break;
            case 64: LA_CFWD(float, 64); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef LA_CFWD
    return hipGetLastError();
}

hipError_t launch_causal_fwd(int dt, int d, const void* q, const void* k, const void* v, void* o, float* den_out,
                             const float* rec, float* S_out, float* z_out, int64_t BH, int64_t N, SegPlan p,
                             hipStream_t s, const float* init, const float* init_n, int feat, int G, int Gv,
                             unsigned* giveups) {
    float* r = const_cast<float*>(rec);  // only read by this form
    return feat == kFeatGiven
               ? launch_causal_fwd_fm<FeatGiven, false>(dt, d, q, k, v, o, den_out, r, S_out, z_out, BH, N, p, s, init,
                                                        init_n, G, Gv, nullptr, giveups, 0, 0)
               : launch_causal_fwd_fm<FeatElu, false>(dt, d, q, k, v, o, den_out, r, S_out, z_out, BH, N, p, s, init,
                                                      init_n, G, Gv, nullptr, giveups, 0, 0);
}

hipError_t launch_causal_fwd_fused(int dt, int d, const void* q, const void* k, const void* v, void* o,
                                   float* den_out, float* rec, float* S_out, float* z_out, int64_t BH, int64_t N,
                                   SegPlan p, hipStream_t s, const float* init, const float* init_n, int feat,
                                   unsigned long long* flags, unsigned* giveups, unsigned long long epoch,
                                   int wait_limit, int Gv) {
    if (p.scan) return hipErrorInvalidValue;  // the records are summed directly
    return feat == kFeatGiven
               ? launch_causal_fwd_fm<FeatGiven, true>(dt, d, q, k, v, o, den_out, rec, S_out, z_out, BH, N, p, s, init,
                                                       init_n, 1, Gv, flags, giveups, epoch, wait_limit)
               : launch_causal_fwd_fm<FeatElu, true>(dt, d, q, k, v, o, den_out, rec, S_out, z_out, BH, N, p, s, init,
                                                     init_n, 1, Gv, flags, giveups, epoch, wait_limit);
}

template <class FM>
static hipError_t launch_noncausal_fwd_fm(int dt, int d, const void* q, void* o, float* den_out, const float* total,
                                          int ntotal, int64_t BH, int64_t N, SegPlan p, hipStream_t s) {
    const dim3 grid((unsigned)(p.nseg * BH));
    if (dt == kBF16) {
        LA_DISPATCH_D(d, hipLaunchKernelGGL((noncausal_fwd_kernel<bf16, D, FM>), grid, dim3(kBlock), 0, s,
                                            (const bf16*)q, (bf16*)o, den_out, total, ntotal, (int)N, p.cps, p.nseg,
                                            (int)BH));
    } else {
        LA_DISPATCH_D(d, hipLaunchKernelGGL((noncausal_fwd_kernel<float, D, FM>), grid, dim3(kBlock), 0, s,
                                            (const float*)q, (float*)o, den_out, total, ntotal, (int)N, p.cps, p.nseg,
                                            (int)BH));
    }
    return hipGetLastError();
}

hipError_t launch_noncausal_fwd(int dt, int d, const void* q, void* o, const float* total, int ntotal, int64_t BH,
                                int64_t N, SegPlan p, hipStream_t s, int feat, float* den_out) {
    return feat == kFeatGiven ? launch_noncausal_fwd_fm<FeatGiven>(dt, d, q, o, den_out, total, ntotal, BH, N, p, s)
                              : launch_noncausal_fwd_fm<FeatElu>(dt, d, q, o, den_out, total, ntotal, BH, N, p, s);
}

}  // namespace la
