// launch.h -- host-side launchers of the gfx950 kernels (internal to the library).
//
// Every launcher enqueues on `stream` and returns the launch status; shapes and
// pointers have been validated by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace la {

constexpr int kChunk = 64;       // tokens per chunk (one MFMA-tiled block of the scan)
constexpr int kBlock = 256;      // threads per workgroup (4 wavefronts)

// Minimum wavefronts per SIMD the register allocator must allow for the large
// per-chunk kernels (2 = two resident workgroups per CU).
#ifndef LA_HEAVY_WAVES_PER_SIMD
#define LA_HEAVY_WAVES_PER_SIMD 2
#endif

enum DType { kF32 = 0, kBF16 = 1 };
// Feature map of the sequence kernels: elu + 1 applied to the inputs, or inputs that
// already are the features.
enum FeatureMap { kFeatElu = 0, kFeatGiven = 1 };

// Sequence segmentation: each (segment, head) pair is one workgroup; a segment
// is `cps` consecutive chunks.  A segment starts from the sum of the fp32 state
// aggregates of the segments before it (after it, for the backward's suffix state).
struct SegPlan {
    int cps;    // chunks per segment
    int nseg;   // segments per head
    bool scan;  // records are turned into running sums by a scan pass (long heads);
                // otherwise each consumer sums the records it needs itself
};
// Segments per head up to which consumers sum the segment records themselves
// (each workgroup re-reads its predecessors' records: quadratic in the segment
// count, cheaper than a scan pass only while that count is small).
constexpr int kDirectRecordMaxSegments = 12;
// causal: the plan of the causal calls (d = 128 heads and a few more at d = 64 may take one
// round of fewer segments where the default would need the running-sum pass).
SegPlan plan_segments(int64_t BH, int64_t N, int64_t d, bool causal = true);

// Number of floats in one segment-state record for head dimension d:
// S_E^T [d][d], z_E [d], P [d].
inline int64_t rec_floats(int64_t d) { return d * d + 2 * d; }

// Forward pieces.  Segment records are per-segment aggregates laid out
// [BH][nseg][rec_floats(d)]; workgroups are numbered segment-major.
// Gv: heads per value head (head bh reads the values of head bh / Gv).
hipError_t launch_seg_state(int dt, int d, const void* k, const void* v, float* rec, int64_t BH,
                            int64_t N, SegPlan p, hipStream_t s, int feat = kFeatElu, int Gv = 1);
// Per-head sum of the segment records (segment order).
hipError_t launch_total(int d, const float* rec, float* total, int64_t BH, int nseg, hipStream_t s);
// In place: record s becomes the sum of the records before it (dir > 0) or after it (dir < 0),
// starting from init[bh] (one record per head) when init is non-null.
hipError_t launch_scan(int d, float* rec, int64_t BH, int nseg, int dir, hipStream_t s,
                       const float* init = nullptr);
// Causal outputs; the last segment of each head writes S_out / z_out when non-null.
// init / init_n (nullable): per head, a start-state record and its token count n0
// (from launch_state_split); the carried state of every segment starts from them.
// G: query heads per key/value head (BH counts query heads; k, v, rec, init, S_out
// and z_out are indexed by key/value head bh / G).  Gv: key/value heads per value head
// (v is indexed by (bh / G) / Gv).  giveups (nullable, BH * nseg counts): set to zero,
// so that a wait-count query after this launch reports none.
hipError_t launch_causal_fwd(int dt, int d, const void* q, const void* k, const void* v, void* o,
                             float* den_out, const float* rec, float* S_out, float* z_out, int64_t BH,
                             int64_t N, SegPlan p, hipStream_t s, const float* init = nullptr,
                             const float* init_n = nullptr, int feat = kFeatElu, int G = 1, int Gv = 1,
                             unsigned* giveups = nullptr);
// The same outputs in one launch (plans with !p.scan, one query head per key/value
// head): each workgroup forms its segment's record into rec itself (bitwise what
// launch_seg_state writes), publishes it with a flag, and waits for the earlier
// segments' (flags BH * nseg words, epoch and wait_limit as for the fused backward;
// giveups BH * nseg counts, 1 where a wait gave up and the segment's rows are NaN).
hipError_t launch_causal_fwd_fused(int dt, int d, const void* q, const void* k, const void* v, void* o,
                                   float* den_out, float* rec, float* S_out, float* z_out, int64_t BH, int64_t N,
                                   SegPlan p, hipStream_t s, const float* init, const float* init_n, int feat,
                                   unsigned long long* flags, unsigned* giveups, unsigned long long epoch,
                                   int wait_limit, int Gv = 1);
// A start state (S0 [BH][d][d], z0 [BH][d], either nullable = zero) in the carried split
// form: one record [S0_E^T | z0_E | P0] per head in init, and n0 per head in init_n.
hipError_t launch_state_split(int d, const float* S0, const float* z0, float* init, float* init_n, int64_t BH,
                              hipStream_t s, int feat = kFeatElu);
// Non-causal outputs from each head's state: the in-order sum of `ntotal`
// records per head at `total` (the segment records, or one precomputed total).
// den_out (nullable): phi(Q_i)^T z per row, [BH][N].
hipError_t launch_noncausal_fwd(int dt, int d, const void* q, void* o, const float* total, int ntotal,
                                int64_t BH, int64_t N, SegPlan p, hipStream_t s, int feat = kFeatElu,
                                float* den_out = nullptr);

// Backward pieces.  bwd_prefix starts each segment from the sum of the forward
// records before it and writes the segment's suffix-state aggregate to rrec;
// bwd_suffix starts each segment from the sum of the rrec records after it.
// init / init_n, rinit (nullable): the forward's start state (split record and count per
// head) and a record of upstream final-state gradients; dS0, dz0 (nullable) receive the
// start state's gradient.
hipError_t launch_bwd_prefix(int dt, int d, const void* q, const void* k, const void* v,
                             const void* dout, void* dq, float* rowstat, float* rrec,
                             const float* rec, int64_t BH, int64_t N, SegPlan p, hipStream_t s,
                             const float* init = nullptr, const float* init_n = nullptr, int feat = kFeatElu,
                             int mode = 0, int Gv = 1, const float* den_in = nullptr);
// mode (given features only): 0 the sweep; 1 statistics (den_in [BH / Gv][N] given, each row's
// (den, G . num of this head) to rowstat, no dq, no records); 2 from (den, g) in rowstat.
// Gv: heads per value head (v and dout of head bh / Gv).
// The backward's per-segment (R, r) records from q, dout and the saved per-row
// statistics, for head dimensions whose prefix sweep does not form them (d > 64).
hipError_t launch_rseg(int dt, int d, const void* q, const void* dout, const float* rowstat, float* rrec, int64_t BH,
                       int64_t N, SegPlan p, hipStream_t s, int feat = kFeatElu, int Gv = 1);
constexpr bool prefix_forms_records(int d) { return d <= 64; }
// Default bound on the polls of one wait between workgroups (each poll sleeps
// about 128 cycles after a coherent load: tens of milliseconds at most).
constexpr int kDefaultWaitLimit = 1 << 16;
// Both backward sweeps in one launch (plans without the record scan); flags holds
// BH * nseg words, epoch is a value no earlier launch on this workspace used,
// wait_limit bounds the polls of each wait for a later segment's record; every
// workgroup writes the number of its waits that gave up to giveups[BH * nseg].
hipError_t launch_bwd_fused(int dt, int d, const void* q, const void* k, const void* v, const void* dout, void* dq,
                            void* dk, void* dv, float* rowstat, float* rrec, const float* rec, unsigned long long* flags,
                            unsigned* giveups, unsigned long long epoch, int wait_limit, int64_t BH, int64_t N,
                            SegPlan p, hipStream_t s,
                            const float* init = nullptr, const float* init_n = nullptr, const float* rinit = nullptr,
                            float* dS0 = nullptr, float* dz0 = nullptr, int feat = kFeatElu);
hipError_t launch_bwd_suffix(int dt, int d, const void* q, const void* k, const void* v,
                             const void* dout, void* dk, void* dv, const float* rowstat,
                             const float* rrec, int64_t BH, int64_t N, SegPlan p, hipStream_t s,
                             const float* rinit = nullptr, float* dS0 = nullptr, float* dz0 = nullptr,
                             int feat = kFeatElu, int Gv = 1);

// Non-causal backward.  ncbwd_q: dQ of every row from the head's key state (the
// in-order sum of `ntotal` records per head at `total`) and each segment's
// (R, r) record; ncbwd_kv: dK, dV of every key row from the in-order sum of
// `ntotal` (R, r) records per head at `rtotal`.
hipError_t launch_ncbwd_q(int dt, int d, const void* q, const void* dout, void* dq, const float* total, int ntotal,
                          float* rrec, int64_t BH, int64_t N, SegPlan p, hipStream_t s, int feat = kFeatElu,
                          int mode = 0, int Gv = 1, const float* den_in = nullptr, float* rowstat = nullptr);
// mode (given features only): 0 the pass; 1 statistics (den_in [BH / Gv][N] given, each row's
// (den, G . num of this head) to rowstat [BH][N] float2, no dq, no record); 2 the pass with (den, g)
// read from rowstat.  Gv: heads per value head (dout of head bh / Gv).
hipError_t launch_ncbwd_kv(int dt, int d, const void* k, const void* v, void* dk, void* dv, const float* rtotal,
                           int ntotal, int64_t BH, int64_t N, SegPlan p, hipStream_t s, int feat = kFeatElu,
                           int Gv = 1);  // v of head bh / Gv

// Zero-fill n floats with a kernel (no memset node, so the call can sit in a captured graph).
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s);
// Copy n floats from src (zero-fill when src is null) with the same kernel.
hipError_t launch_copy_or_zero(float* p, const float* src, size_t n, hipStream_t s);
// fp32 pieces of the causal forward at d = 128 on feature blocks: phi(x) = elu(x) + 1 of
// x [heads][N][KF db] into block layout [heads][KF][N][db] (db a multiple of 4); and a
// block of `cols` columns (a multiple of 4; 16-byte aligned rows) copied between
// row-major matrices: dst[r][c] = src[r][c], r < rows, c < cols, rows dst_ld and src_ld
// floats apart.
hipError_t launch_phi_blocks(const float* x, float* out, int64_t heads, int64_t N, int KF, int db, hipStream_t s);
hipError_t launch_copy_cols(float* dst, int64_t dst_ld, const float* src, int64_t src_ld, int64_t rows, int cols,
                            hipStream_t s);
// And back: dx [heads][N][KF db] = (dF0 + dF1) * phi'(x) with dF0, dF1 in block layout.
hipError_t launch_phi_blocks_grad(const float* x, const float* dF0, const float* dF1, float* dx, int64_t heads,
                                  int64_t N, int KF, int db, hipStream_t s);

// Decode.
hipError_t launch_decode(int dt, int d, float* S, float* z, const void* q, const void* k,
                         const void* v, void* o, int64_t BH, hipStream_t s);
// T decode steps per key/value head in one pass over its state, read by G query heads;
// k, v are [BHkv][T][d], q, o are [BHkv][G][T][d].  KF feature blocks: KF states per
// key/value head ([BHkv][KF][d][d]), k [BHkv][KF][T][d], q, o [BHkv][G][KF][T][d], v as
// before; den_out (nullable) takes the denominators in the layout of q's rows.
hipError_t launch_decode_steps(int dt, int d, float* S, float* z, const void* q, const void* k,
                               const void* v, void* o, int64_t BHkv, int64_t T, int64_t G, hipStream_t s,
                               int feat = kFeatElu, int KF = 1, float* den_out = nullptr);
// FAVOR+ random features of `rows` rows of x [rows][d]: out[r][i] = exp(omega_i . x_r - |x_r|^2 / 2)
// for the d rows of omega [d][d] fp32 (m = d features; the constant 1/sqrt(m) is left out).
hipError_t launch_favor_features(int dt, int d, const void* x, const float* omega, void* out, int64_t rows,
                                 hipStream_t s, int64_t N = 0, int KF = 1);
// dx = Omega^T (dF * F) - x sum(dF * F) per row (the gradient through the features F of x,
// m = d, omega [d][d]).  KF blocks: omega [KF d][d], F and dF [heads][KF][N][d] for x [heads][N][d]
// (rows = heads x N), dx summed over the blocks.
hipError_t launch_favor_features_bwd(int dt, int d, const void* x, const float* omega, const void* F, const void* dF,
                                     void* dx, int64_t rows, hipStream_t s, int64_t N = 0, int KF = 1);
// KF feature blocks of rows x [rows][d] (rows = heads x N; omega [KF d][d]) into
// out [heads][KF][N][d]; N = 0: one head of all rows.
// o = sum_j den_j o_j / sum_j den_j over the KF feature blocks of each head (ob
// [heads][KF][N][d], db [heads][KF][N]); den_out (nullable) gets sum_j den_j.
// (db null: o = sum_j o_j.)
hipError_t launch_combine_blocks(int dt, int d, const void* ob, const float* db, void* o, float* den_out,
                                 int64_t rows, int64_t N, int KF, hipStream_t s);
// Backward row statistics over KF feature blocks: rowstat [heads][KF][N] float2 (den, G . num_j)
// becomes (den, g) in every block, g = -(sum_j G . num_j) / den.
hipError_t launch_combine_stats(float* rowstat, int64_t rows, int64_t N, int KF, hipStream_t s);
// The same (den, g) from the forward's output o and the upstream gradient dout ([heads][N][d],
// rows = heads x N) and den [heads][N]: g = -G . O with G = dO / den rounded to dt.
hipError_t launch_stats_from_output(int dt, int d, const void* dout, const void* o, const float* den, float* rowstat,
                                    int64_t rows, int64_t N, int KF, hipStream_t s);

}  // namespace la
