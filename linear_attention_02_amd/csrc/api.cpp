// api.cpp -- the C ABI (include/linattn.h): argument validation, workspace
// layout and kernel sequencing.  No device memory is allocated here; every
// launch goes on the caller's stream.
#include "linattn.h"

#include <hip/hip_runtime.h>

#include <unistd.h>

#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "launch.h"

namespace la {

SegPlan plan_segments(int64_t BH, int64_t N, int64_t d, bool causal) {
    const int64_t nchunk = (N + kChunk - 1) / kChunk;
    // Aim for about 512 workgroups (2 per CU): the heavy kernels keep 2-3
    // workgroups resident per CU, and starting a segment costs one record read
    // per segment before it, so fewer, longer segments are cheaper.  Segments
    // grow to 64 chunks where that keeps a head within the segment count whose
    // records are summed directly (one launch each way, no running-sum pass).
    // Past that, at d = 128 (whose sweeps hold one workgroup per CU), one round
    // of workgroups that keeps at least 3/4 of the 256 CUs busy with at most that
    // many segments per head is taken (the fused forward at B1 H32 N131072: 1.34
    // against 1.52 ms for a running-sum plan); otherwise segments of 32 chunks,
    // past which shorter segments balance the rounds better.  Shorter causal heads
    // whose plan would need the running-sum pass take that one round too (the
    // non-causal passes sum their records in a pass of their own and keep the
    // larger count of workgroups).
    constexpr int64_t kCUs = 256;
    int64_t cps = (BH * nchunk + 2 * kCUs - 1) / (2 * kCUs);
    if (cps < 1) cps = 1;
    // One round of workgroups (the heavy kernels hold one per CU at d = 128, two below), at most
    // kDirectRecordMaxSegments segments per head, when that fills at least 3/4 of the
    // workgroup slots (segments per head; 0 when it does not).
    const int64_t slots = d >= 128 ? kCUs : 2 * kCUs;
    int64_t one_round = 0;
    if (BH <= slots) {
        one_round = slots / BH < kDirectRecordMaxSegments ? slots / BH : kDirectRecordMaxSegments;
        if (4 * BH * one_round < 3 * slots) one_round = 0;
    }
    if (cps > 32) {
        const int64_t longest = cps < 64 ? cps : 64;
        if ((nchunk + longest - 1) / longest <= kDirectRecordMaxSegments)
            cps = longest;
        else if (d >= 128 && one_round >= 1)
            cps = (nchunk + one_round - 1) / one_round;
        else
            cps = 32;
    } else if (causal && one_round >= 1 && (nchunk + cps - 1) / cps > kDirectRecordMaxSegments) {
        // A d = 128 plan that would need the running-sum pass (B1 H32 N8192: 16 segments of 8
        // chunks in two rounds, 224 us) takes the one round instead (8 segments of 16 chunks).
        cps = (nchunk + one_round - 1) / one_round;
    }
    SegPlan p;
    p.cps = (int)cps;
    p.nseg = (int)((nchunk + cps - 1) / cps);
    if (p.nseg < 1) p.nseg = 1;
    p.scan = p.nseg > kDirectRecordMaxSegments;
    return p;
}

}  // namespace la

namespace {

thread_local std::string g_last_error;

la_status fail(la_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
la_status fail(la_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

la_status hip_fail(hipError_t e, const char* what) {
    return fail(LA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- optional per-kernel timing (benchmarks) ---------------------------------------------
// While enabled on a thread, every kernel launched by a call on that thread is
// bracketed by two HIP events on its stream.  Events come from a per-thread
// pool that is created once and reused; nothing is allocated on the device.
struct KernelTiming {
    bool on = false;
    std::vector<hipEvent_t> pool;  // 2 events per record
    std::vector<const char*> names;
    size_t used = 0;               // records in use
};
thread_local KernelTiming g_timing;

struct Timed {
    hipStream_t s;
    hipEvent_t stop = nullptr;
    Timed(const char* name, hipStream_t stream) : s(stream) {
        KernelTiming& T = g_timing;
        if (!T.on) return;
        if (2 * (T.used + 1) > T.pool.size()) {
            hipEvent_t a = nullptr, b = nullptr;
            if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return;
            T.pool.push_back(a);
            T.pool.push_back(b);
        }
        if (T.names.size() < T.used + 1) T.names.resize(T.used + 1);
        T.names[T.used] = name;
        (void)hipEventRecord(T.pool[2 * T.used], s);  // timing only: a failed record leaves no entry time
        stop = T.pool[2 * T.used + 1];
        ++T.used;
    }
    ~Timed() {
        if (stop != nullptr) (void)hipEventRecord(stop, s);
    }
};

template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& f) {
    Timed t(name, s);
    return f();
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    const char* name;
    const void* p;
    size_t bytes;
};

bool overlap(const Range& a, const Range& b) {
    if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

size_t elem_size(la_dtype dt) { return dt == LA_BF16 ? 2 : 4; }

// Shape checks common to the sequence calls.  Sets *empty when there is no work.
la_status check_shape(int64_t B, int64_t H, int64_t N, int64_t d, int chunk, la_dtype dt, bool* empty) {
    if (dt != LA_F32 && dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "dtype %d is not LA_F32 or LA_BF16", (int)dt);
    if (d != 32 && d != 64 && d != 128) return fail(LA_ERR_UNSUPPORTED, "d = %lld; built for 32, 64 and 128", (long long)d);
    if (chunk != 0 && chunk != la::kChunk)
        return fail(LA_ERR_UNSUPPORTED, "chunk = %d; only 0 (default) and %d are supported", chunk, la::kChunk);
    if (B < 0 || H < 0 || N < 0) return fail(LA_ERR_INVALID_ARGUMENT, "negative size (B=%lld H=%lld N=%lld)",
                                             (long long)B, (long long)H, (long long)N);
    if (N > (int64_t)1 << 30) return fail(LA_ERR_UNSUPPORTED, "N = %lld exceeds 2^30 tokens per head", (long long)N);
    // Kernels address one head through a buffer resource with a 31-bit byte range.
    if (N * d * (int64_t)elem_size(dt) + 64 * d * (int64_t)elem_size(dt) > ((int64_t)1 << 31) - 1)
        return fail(LA_ERR_UNSUPPORTED, "one head of N = %lld tokens at d = %lld exceeds 2^31 bytes", (long long)N, (long long)d);
    if (B > 0 && H > ((int64_t)1 << 31) / B) return fail(LA_ERR_UNSUPPORTED, "B*H exceeds 2^31 heads");
    *empty = (B == 0 || H == 0 || N == 0);
    return LA_OK;
}

// Workspace layout of the sequence calls.
struct Layout {
    la::SegPlan plan;
    int64_t heads = 0;
    size_t rec = 0, total = 0, rrec = 0, rtotal = 0, rowstat = 0, flags = 0, giveups = 0, init = 0, init_n = 0,
           rinit = 0;  // byte offsets
    bool fused = false;  // backward: both sweeps in one launch
    size_t bytes = 0;
};

Layout layout(la_op op, int64_t B, int64_t H, int64_t N, int64_t d) {
    Layout L;
    const int64_t BH = B * H;
    L.plan = la::plan_segments(BH, N, d, op == LA_OP_FWD_CAUSAL || op == LA_OP_BWD_CAUSAL);
    L.heads = BH;
    const size_t recb = (size_t)BH * L.plan.nseg * la::rec_floats(d) * sizeof(float);
    size_t off = 0;
    L.rec = off;
    off += align_up(recb);
    const size_t totb = (size_t)BH * la::rec_floats(d) * sizeof(float);
    if (op == LA_OP_FWD_NONCAUSAL) {
        L.total = off;
        off += align_up(totb);
    } else if (op == LA_OP_BWD_NONCAUSAL) {
        L.total = off;
        off += align_up(totb);
        L.rrec = off;
        off += align_up(recb);
        L.rtotal = off;
        off += align_up(totb);
    } else if (op == LA_OP_FWD_CAUSAL) {
        L.init = off;  // a start state in split form, when one is given
        off += align_up(totb);
        L.init_n = off;
        off += align_up((size_t)BH * sizeof(float));
        if (!L.plan.scan) {  // the fused forward's per-segment flags and wait counts
            L.flags = off;
            off += align_up((size_t)BH * L.plan.nseg * sizeof(unsigned long long));
            L.giveups = off;
            off += align_up((size_t)BH * L.plan.nseg * sizeof(unsigned));
        }
    } else if (op == LA_OP_BWD_CAUSAL) {
        L.rrec = off;
        off += align_up(recb);
        L.rowstat = off;
        off += align_up((size_t)BH * N * 2 * sizeof(float));
        L.fused = !L.plan.scan && la::prefix_forms_records((int)d);
        if (L.fused) {  // the fused backward's per-segment flags, and each workgroup's count of waits given up
            L.flags = off;
            off += align_up((size_t)BH * L.plan.nseg * sizeof(unsigned long long));
            L.giveups = off;
            off += align_up((size_t)BH * L.plan.nseg * sizeof(unsigned));
        }
        // a start state in split form, its counts, and the record of final-state gradients
        L.init = off;
        off += align_up(totb);
        L.init_n = off;
        off += align_up((size_t)BH * sizeof(float));
        L.rinit = off;
        off += align_up(totb);
    }
    L.bytes = off;
    return L;
}

// A value for the fused backward's flag words that no earlier launch of this
// process used and, being seeded from the clock and the process id, that flag
// words another process left in a reused buffer do not hold (never zero, so a
// zero-filled buffer never matches either).
// Polls a workgroup spends waiting for another's record before it gives up
// (its outputs are then NaN); lowered only by tests of that path.
std::atomic<int> g_wait_limit{la::kDefaultWaitLimit};

unsigned long long next_epoch() {
    static std::atomic<unsigned long long> counter{[] {
        unsigned long long x = (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
        x ^= (unsigned long long)getpid() << 40;
        x *= 0x9E3779B97F4A7C15ull;  // spread the bits (golden-ratio multiplier)
        return x ^ (x >> 29);
    }()};
    unsigned long long e;
    do e = counter.fetch_add(1, std::memory_order_relaxed); while (e == 0);
    return e;
}

// The saved forward state: every segment record, then (filled by the non-causal
// forward only) one total per head.  The records of the non-causal plan: the causal
// plan never has more segments, so its records fit in front of the totals too.
size_t saved_records_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
    const la::SegPlan p = la::plan_segments(B * H, N, d, false);
    return align_up((size_t)(B * H) * p.nseg * la::rec_floats(d) * sizeof(float));
}

size_t saved_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
    return saved_records_bytes(B, H, N, d) + (size_t)(B * H) * la::rec_floats(d) * sizeof(float);
}

struct BlockLayout {
    size_t inner = 0, ob = 0, db = 0, bytes = 0;
};
BlockLayout block_layout(bool causal, int64_t B, int64_t H, int64_t N, int64_t d, int64_t KF, la_dtype dt) {
    BlockLayout L;
    if (B == 0 || H == 0 || N == 0) return L;
    L.inner = layout(causal ? LA_OP_FWD_CAUSAL : LA_OP_FWD_NONCAUSAL, B, H * KF, N, d).bytes;
    if (KF == 1) {
        L.bytes = L.inner;
        return L;
    }
    L.ob = align_up(L.inner);
    L.db = L.ob + align_up((size_t)B * H * KF * N * d * elem_size(dt));
    L.bytes = L.db + align_up((size_t)B * H * KF * N * sizeof(float));
    return L;
}


// fp32 at d = 128, the causal forward: its fp32 tiles at d = 128 do not fit a CU's
// LDS, so it runs on feature blocks.  phi(q), phi(k) go to two blocks of 64 features
// each ([BH][2][N][64]), and each half of the value columns runs as the causal forward
// on those blocks (la_forward_causal_features_blocks with m = 128, d = 64: the blocks
// share one normalization); outputs and states are put back together.  Workspace:
// the features, one value half and its output, the start and final state's halves,
// and one block workspace per value half (so that the wait counts of both remain).
struct F128Layout {
    size_t fq = 0, fk = 0, vh = 0, oh = 0, s0h = 0, sh = 0, blk[2] = {0, 0}, blk_bytes = 0, bytes = 0;
};
F128Layout f128_layout(int64_t B, int64_t H, int64_t N) {
    F128Layout L;
    if (B == 0 || H == 0 || N == 0) return L;
    const int64_t BH = B * H;
    const size_t feat = align_up((size_t)BH * N * 128 * sizeof(float)), half = align_up((size_t)BH * N * 64 * sizeof(float));
    const size_t st = align_up((size_t)BH * 128 * 64 * sizeof(float));
    L.fk = feat;
    L.vh = 2 * feat;
    L.oh = L.vh + half;
    L.s0h = L.oh + half;
    L.sh = L.s0h + st;
    L.blk_bytes = align_up(block_layout(true, B, H, N, 64, 2, LA_F32).bytes);
    L.blk[0] = L.sh + st;
    L.blk[1] = L.blk[0] + L.blk_bytes;
    L.bytes = L.blk[1] + L.blk_bytes;
    return L;
}

// fp32 at d = 128, the causal and non-causal backward, on the same feature blocks: per
// value half, the forward on the blocks (its output half and the head's den) and the
// blocks' backward with g from that output half (the halves' g add up to the row's g,
// and dphi(Q), dphi(K) are linear in G and g, so the halves' feature gradients add up);
// dq, dk = the sum over the halves times phi'.  Workspace: features and their two
// gradients each, one value half with its output, upstream gradient and dv, den, and
// the blocks' forward and backward workspaces.
struct B128Layout {
    size_t fq = 0, fk = 0, dfq[2] = {0, 0}, dfk[2] = {0, 0}, vh = 0, oh = 0, doh = 0, dvh = 0, den = 0;
    size_t fwd = 0, fwd_bytes = 0, bwd = 0, bwd_bytes = 0, bytes = 0;
};
B128Layout b128_layout(bool causal, int64_t B, int64_t H, int64_t N) {
    B128Layout L;
    if (B == 0 || H == 0 || N == 0) return L;
    const int64_t BH = B * H;
    const size_t feat = align_up((size_t)BH * N * 128 * sizeof(float)), half = align_up((size_t)BH * N * 64 * sizeof(float));
    L.fk = feat;
    L.dfq[0] = 2 * feat;
    L.dfq[1] = 3 * feat;
    L.dfk[0] = 4 * feat;
    L.dfk[1] = 5 * feat;
    L.vh = 6 * feat;
    L.oh = L.vh + half;
    L.doh = L.oh + half;
    L.dvh = L.doh + half;
    L.den = L.dvh + half;
    L.fwd = L.den + align_up((size_t)BH * N * sizeof(float));
    L.fwd_bytes = align_up(block_layout(causal, B, H, N, 64, 2, LA_F32).bytes);
    L.bwd = L.fwd + L.fwd_bytes;
    // the blocks' backward: its block heads' workspace and dv, and (non-causal) two row statistics per block row
    L.bwd_bytes = align_up(layout(causal ? LA_OP_BWD_CAUSAL : LA_OP_BWD_NONCAUSAL, B, 2 * H, N, 64).bytes) +
                  align_up((size_t)BH * N * 128 * sizeof(float)) +
                  (causal ? 0 : align_up((size_t)BH * 2 * N * 2 * sizeof(float)));
    L.bytes = L.bwd + L.bwd_bytes;
    return L;
}

la_status check_workspace(const Layout& L, const void* ws, size_t ws_bytes) {
    if (L.bytes == 0) return LA_OK;
    if ((int64_t)L.plan.nseg * L.heads > ((int64_t)1 << 24))
        return fail(LA_ERR_UNSUPPORTED, "%lld workgroups exceed the 2^24 grid limit",
                    (long long)L.plan.nseg * L.heads);
    if (ws == nullptr) return fail(LA_ERR_WORKSPACE, "workspace is NULL; %zu bytes are needed", L.bytes);
    if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "workspace must be %zu-byte aligned", kAlign);
    if (ws_bytes < L.bytes) return fail(LA_ERR_WORKSPACE, "workspace has %zu bytes; %zu are needed", ws_bytes, L.bytes);
    return LA_OK;
}

la_status check_ptrs(const Range* in, int nin, const Range* out, int nout) {
    for (int i = 0; i < nin + nout; ++i) {
        const Range& r = i < nin ? in[i] : out[i - nin];
        if (r.p != nullptr && !aligned16(r.p)) return fail(LA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", r.name);
    }
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(out[i], in[j]))
                return fail(LA_ERR_INVALID_ARGUMENT, "output %s overlaps input %s", out[i].name, in[j].name);
        for (int j = i + 1; j < nout; ++j)
            if (overlap(out[i], out[j]))
                return fail(LA_ERR_INVALID_ARGUMENT, "outputs %s and %s overlap", out[i].name, out[j].name);
    }
    return LA_OK;
}

}  // namespace

extern "C" {

const char* la_status_string(la_status s) {
    switch (s) {
        case LA_OK: return "LA_OK";
        case LA_ERR_INVALID_ARGUMENT: return "LA_ERR_INVALID_ARGUMENT";
        case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
        case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE";
        case LA_ERR_HIP: return "LA_ERR_HIP";
    }
    return "LA_ERR_UNKNOWN";
}

const char* la_last_error_message(void) { return g_last_error.c_str(); }

const char* la_version(void) { return "linattn 0.1.0 (gfx950)"; }

la_status la_profile_enable(int on) {
    g_timing.on = on != 0;
    g_timing.used = 0;
    return LA_OK;
}

la_status la_debug_set_wait_limit(int polls) {
    if (polls < 0) return fail(LA_ERR_INVALID_ARGUMENT, "polls must be >= 0 (got %d)", polls);
    g_wait_limit.store(polls, std::memory_order_relaxed);
    return LA_OK;
}

int la_debug_wait_limit(void) { return g_wait_limit.load(std::memory_order_relaxed); }

int la_profile_count(void) { return (int)g_timing.used; }

la_status la_profile_entry(int i, const char** name, float* ms) {
    if (i < 0 || (size_t)i >= g_timing.used || name == nullptr || ms == nullptr)
        return fail(LA_ERR_INVALID_ARGUMENT, "profile entry %d out of range (have %zu)", i, g_timing.used);
    hipEvent_t a = g_timing.pool[2 * i], b = g_timing.pool[2 * i + 1];
    hipError_t e = hipEventSynchronize(b);
    if (e != hipSuccess) return hip_fail(e, "profile event sync");
    if ((e = hipEventElapsedTime(ms, a, b)) != hipSuccess) return hip_fail(e, "profile elapsed time");
    *name = g_timing.names[i];
    return LA_OK;
}

la_status la_workspace_size(la_op op, int64_t B, int64_t H, int64_t N, int64_t d, int chunk, la_dtype dt,
                            size_t* bytes_out) {
    if (bytes_out == nullptr) return fail(LA_ERR_INVALID_ARGUMENT, "bytes_out is NULL");
    if (op != LA_OP_FWD_NONCAUSAL && op != LA_OP_FWD_CAUSAL && op != LA_OP_BWD_CAUSAL && op != LA_OP_BWD_NONCAUSAL)
        return fail(LA_ERR_INVALID_ARGUMENT, "unknown op %d", (int)op);
    bool empty = false;
    la_status st = check_shape(B, H, N, d, chunk, dt, &empty);
    if (st != LA_OK) return st;
    if (op == LA_OP_FWD_CAUSAL && dt == LA_F32 && d == 128)
        *bytes_out = empty ? 0 : f128_layout(B, H, N).bytes;
    else if ((op == LA_OP_BWD_CAUSAL || op == LA_OP_BWD_NONCAUSAL) && dt == LA_F32 && d == 128)
        *bytes_out = empty ? 0 : b128_layout(op == LA_OP_BWD_CAUSAL, B, H, N).bytes;
    else
        *bytes_out = empty ? 0 : layout(op, B, H, N, d).bytes;
    return LA_OK;
}

la_status la_saved_state_size(int64_t B, int64_t H, int64_t N, int64_t d, int chunk, la_dtype dt,
                              size_t* bytes_out) {
    if (bytes_out == nullptr) return fail(LA_ERR_INVALID_ARGUMENT, "bytes_out is NULL");
    bool empty = false;
    la_status st = check_shape(B, H, N, d, chunk, dt, &empty);
    if (st != LA_OK) return st;
    *bytes_out = empty ? 0 : saved_bytes(B, H, N, d);
    return LA_OK;
}

}  // extern "C"

namespace {

// Gv: heads per value head (v has B H / Gv heads; head h reads value head h / Gv).
// den_out (nullable): [B][H][N] fp32 denominators.
la_status forward_noncausal(const void* q, const void* k, const void* v, void* o, void* saved_state,
                            size_t saved_state_bytes, int64_t B, int64_t H, int64_t N, int64_t d, la_dtype dt,
                            void* workspace, size_t workspace_bytes, void* stream, int feat, int64_t Gv = 1,
                            float* den_out = nullptr) {
    bool empty = false;
    la_status st = check_shape(B, H, N, d, 0, dt, &empty);
    if (st != LA_OK) return st;
    // Empty tensors (no tokens) may come as NULL pointers.
    if (N > 0 && (!q || !k || !v || !o)) return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v and o must be non-NULL");
    const size_t tb = (size_t)B * H * N * d * elem_size(dt);
    const size_t sb = saved_state ? saved_bytes(B, H, N, d) : 0;
    if (saved_state && saved_state_bytes < sb)
        return fail(LA_ERR_INVALID_ARGUMENT, "saved_state has %zu bytes; %zu are needed", saved_state_bytes, sb);
    const Range in[] = {{"q", q, tb}, {"k", k, tb}, {"v", v, tb / Gv}};
    const Range out[] = {{"o", o, tb}, {"saved_state", saved_state, sb},
                         {"den_out", den_out, (size_t)B * H * N * sizeof(float)}};
    if ((st = check_ptrs(in, 3, out, 3)) != LA_OK) return st;
    if (empty) return LA_OK;
    const Layout L = layout(LA_OP_FWD_NONCAUSAL, B, H, N, d);
    if ((st = check_workspace(L, workspace, workspace_bytes)) != LA_OK) return st;
    const Range wsr[] = {{"workspace", workspace, L.bytes}};
    if ((st = check_ptrs(in, 3, wsr, 1)) != LA_OK) return st;
    for (const Range& r : out)
        if (overlap(wsr[0], r)) return fail(LA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);

    char* ws = static_cast<char*>(workspace);
    // The segment records and the totals go straight into the saved state when one is asked for.
    float* rec = saved_state ? static_cast<float*>(saved_state) : reinterpret_cast<float*>(ws + L.rec);
    float* total = saved_state ? reinterpret_cast<float*>(static_cast<char*>(saved_state) + saved_records_bytes(B, H, N, d))
                               : reinterpret_cast<float*>(ws + L.total);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t BH = B * H;
    const int idt = dt == LA_BF16 ? la::kBF16 : la::kF32;
    hipError_t e;
    if ((e = timed("seg_state", s, [&] {
             return la::launch_seg_state(idt, (int)d, k, v, rec, BH, N, L.plan, s, feat, (int)Gv);
         })) != hipSuccess)
        return hip_fail(e, "seg_state launch");
    // One total per head, read by every readout workgroup (and by the backward, from the saved state).
    if ((e = timed("total", s, [&] { return la::launch_total((int)d, rec, total, BH, L.plan.nseg, s); })) != hipSuccess)
        return hip_fail(e, "total launch");
    if ((e = timed("noncausal_fwd", s, [&] {
             return la::launch_noncausal_fwd(idt, (int)d, q, o, total, 1, BH, N, L.plan, s, feat, den_out);
         })) != hipSuccess)
        return hip_fail(e, "noncausal_fwd launch");
    return LA_OK;
}

// Hkv: key/value heads (H a multiple of it); k, v, the start state and the final state
// are per key/value head, q, o and den per query head.  Gv: key/value heads per value
// head (v has B Hkv / Gv heads).
la_status forward_causal_f128(const void* q, const void* k, const void* v, void* o, const float* S0, const float* z0,
                              float* den_out, float* S_out, float* z_out, int64_t B, int64_t H, int64_t N,
                              void* workspace, size_t workspace_bytes, hipStream_t s);

la_status forward_causal(const void* q, const void* k, const void* v, void* o, const float* S0, const float* z0,
                         float* den_out, float* S_out, float* z_out, void* saved_state, size_t saved_state_bytes,
                         int64_t B, int64_t H, int64_t N, int64_t d, int chunk, la_dtype dt, void* workspace,
                         size_t workspace_bytes, void* stream, int feat, int64_t Hkv, int64_t Gv = 1) {
    bool empty = false;
    la_status st = check_shape(B, H, N, d, chunk, dt, &empty);
    if (st != LA_OK) return st;
    if (Hkv < 0 || (Hkv == 0) != (H == 0) || (Hkv > 0 && H % Hkv != 0))
        return fail(LA_ERR_INVALID_ARGUMENT, "H = %lld query heads must be a multiple of Hkv = %lld", (long long)H,
                    (long long)Hkv);
    if (Hkv != H && saved_state)
        return fail(LA_ERR_INVALID_ARGUMENT, "saved_state is for la_backward_causal, which has no grouped heads");
    // fp32 at d = 128 runs on feature blocks (forward_causal_f128): the default map on plain heads.
    const bool f128 = dt == LA_F32 && d == 128;
    if (f128 && (Hkv != H || Gv != 1 || feat != la::kFeatElu))
        return fail(LA_ERR_UNSUPPORTED, "fp32 at d = 128: only the causal forward of phi = elu + 1 on plain heads is built");
    // Empty tensors (no tokens) may come as NULL pointers.
    if (N > 0 && (!q || !k || !v || !o)) return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v and o must be non-NULL");
    const bool from_state = S0 != nullptr || z0 != nullptr;
    if (from_state && saved_state)
        return fail(LA_ERR_INVALID_ARGUMENT,
                    "saved_state is for la_backward_causal, which starts from a zero state: not with S0 / z0");
    const size_t tb = (size_t)B * H * N * d * elem_size(dt), kb = (size_t)B * Hkv * N * d * elem_size(dt);
    const size_t Sb = (size_t)B * Hkv * d * d * sizeof(float), zb = (size_t)B * Hkv * d * sizeof(float);
    const Range in[] = {{"q", q, tb}, {"k", k, kb}, {"v", v, kb / Gv}};
    const size_t sb = saved_state ? saved_bytes(B, H, N, d) : 0;
    if (saved_state && saved_state_bytes < sb)
        return fail(LA_ERR_INVALID_ARGUMENT, "saved_state has %zu bytes; %zu are needed", saved_state_bytes, sb);
    const Range out[] = {{"o", o, tb},
                         {"den_out", den_out, (size_t)B * H * N * sizeof(float)},
                         {"S_out", S_out, Sb},
                         {"z_out", z_out, zb},
                         {"saved_state", saved_state, sb}};
    if ((st = check_ptrs(in, 3, out, 5)) != LA_OK) return st;
    // The start state may be the very buffer the final state goes to (continuing in
    // place: it is read before anything is written), but no other output.
    const Range init_in[] = {{"S0", S0, Sb}, {"z0", z0, zb}};
    for (const Range& r : init_in) {
        if (r.p != nullptr && !aligned16(r.p)) return fail(LA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", r.name);
        for (const Range& x : out)
            if (overlap(r, x) && !(r.p == x.p && r.bytes == x.bytes && (x.p == S_out || x.p == z_out)))
                return fail(LA_ERR_INVALID_ARGUMENT, "%s overlaps output %s", r.name, x.name);
    }
    if (overlap(init_in[0], init_in[1])) return fail(LA_ERR_INVALID_ARGUMENT, "S0 and z0 overlap");
    if (B == 0 || H == 0) return LA_OK;
    const int64_t BH = B * H, BHkv = B * Hkv;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (N == 0) {  // empty sequence: the final state is the start state
        if (S_out && S_out != S0) {
            e = timed("fill_zero", s, [&] { return la::launch_copy_or_zero(S_out, S0, (size_t)BHkv * d * d, s); });
            if (e != hipSuccess) return hip_fail(e, "S_out");
        }
        if (z_out && z_out != z0) {
            e = timed("fill_zero", s, [&] { return la::launch_copy_or_zero(z_out, z0, (size_t)BHkv * d, s); });
            if (e != hipSuccess) return hip_fail(e, "z_out");
        }
        return LA_OK;
    }
    // (fp32 at d = 128 leaves a saved state unused: its backward recomputes the forward on the feature blocks.)
    if (f128) return forward_causal_f128(q, k, v, o, S0, z0, den_out, S_out, z_out, B, H, N, workspace, workspace_bytes, s);
    const Layout L = layout(LA_OP_FWD_CAUSAL, B, H, N, d);
    if ((st = check_workspace(L, workspace, workspace_bytes)) != LA_OK) return st;
    const Range wsr[] = {{"workspace", workspace, L.bytes}};
    if ((st = check_ptrs(in, 3, wsr, 1)) != LA_OK) return st;
    for (const Range& r : out)
        if (overlap(wsr[0], r)) return fail(LA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);

    char* ws = static_cast<char*>(workspace);
    // The segment records go straight into the saved state when one is asked for.
    float* rec = saved_state ? static_cast<float*>(saved_state) : reinterpret_cast<float*>(ws + L.rec);
    float* init = from_state ? reinterpret_cast<float*>(ws + L.init) : nullptr;
    float* init_n = from_state ? reinterpret_cast<float*>(ws + L.init_n) : nullptr;
    const int idt = dt == LA_BF16 ? la::kBF16 : la::kF32;
    // The key state once per key/value head (the plan is the query heads'; its records fit).
    if (from_state &&
        (e = timed("state_split", s, [&] { return la::launch_state_split((int)d, S0, z0, init, init_n, BHkv, s, feat); })) !=
            hipSuccess)
        return hip_fail(e, "state_split launch");
    unsigned* giveups = L.plan.scan ? nullptr : reinterpret_cast<unsigned*>(ws + L.giveups);
    if (!L.plan.scan && Hkv == H) {
        // one launch: every workgroup forms its own segment's record, then waits for the earlier ones
        unsigned long long* flags = reinterpret_cast<unsigned long long*>(ws + L.flags);
        const unsigned long long epoch = next_epoch();
        if ((e = timed("causal_fwd_fused", s, [&] {
                 return la::launch_causal_fwd_fused(idt, (int)d, q, k, v, o, den_out, rec, S_out, z_out, BH, N,
                                                    L.plan, s, init, init_n, feat, flags, giveups, epoch,
                                                    g_wait_limit.load(std::memory_order_relaxed), (int)Gv);
             })) != hipSuccess)
            return hip_fail(e, "causal_fwd_fused launch");
        return LA_OK;
    }
    if ((e = timed("seg_state", s, [&] {
             return la::launch_seg_state(idt, (int)d, k, v, rec, BHkv, N, L.plan, s, feat, (int)Gv);
         })) != hipSuccess)
        return hip_fail(e, "seg_state launch");
    if (L.plan.scan &&
        (e = timed("scan", s, [&] { return la::launch_scan((int)d, rec, BHkv, L.plan.nseg, 1, s, init); })) != hipSuccess)
        return hip_fail(e, "scan launch");
    if ((e = timed("causal_fwd", s, [&] {
             return la::launch_causal_fwd(idt, (int)d, q, k, v, o, den_out, rec, S_out, z_out, BH, N, L.plan, s, init,
                                          init_n, feat, (int)(H / Hkv), (int)Gv, giveups);
         })) != hipSuccess)
        return hip_fail(e, "causal_fwd launch");
    return LA_OK;
}

}  // namespace

namespace la {

// The causal forward on a workspace the caller supplies (for the entry point whose
// workspace is a static device array); the same checks and launches as la_forward_causal.
la_status forward_causal_on(const void* q, const void* k, const void* v, void* o, const float* S0, const float* z0,
                            float* den_out, float* S_out, float* z_out, int64_t B, int64_t H, int64_t N, int64_t d,
                            int chunk, la_dtype dt, void* workspace, size_t workspace_bytes, void* stream) {
    return forward_causal(q, k, v, o, S0, z0, den_out, S_out, z_out, nullptr, 0, B, H, N, d, chunk, dt, workspace,
                          workspace_bytes, stream, la::kFeatElu, H);
}

la_status fail_status(la_status s, const char* msg) { return fail(s, "%s", msg); }

}  // namespace la

extern "C" {

la_status la_forward_noncausal(const void* q, const void* k, const void* v, void* o, void* saved_state,
                               size_t saved_state_bytes, int64_t B, int64_t H, int64_t N, int64_t d, la_dtype dt,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return forward_noncausal(q, k, v, o, saved_state, saved_state_bytes, B, H, N, d, dt, workspace, workspace_bytes,
                             stream, la::kFeatElu);
}

la_status la_forward_noncausal_features(const void* fq, const void* fk, const void* v, void* o, int64_t B, int64_t H,
                                        int64_t N, int64_t d, la_dtype dt, void* workspace, size_t workspace_bytes,
                                        void* stream) {
    return forward_noncausal(fq, fk, v, o, nullptr, 0, B, H, N, d, dt, workspace, workspace_bytes, stream,
                             la::kFeatGiven);
}

la_status la_forward_causal(const void* q, const void* k, const void* v, void* o, const float* S0, const float* z0,
                            float* den_out, float* S_out, float* z_out, void* saved_state, size_t saved_state_bytes,
                            int64_t B, int64_t H, int64_t N, int64_t d, int chunk, la_dtype dt, void* workspace,
                            size_t workspace_bytes, void* stream) {
    return forward_causal(q, k, v, o, S0, z0, den_out, S_out, z_out, saved_state, saved_state_bytes, B, H, N, d, chunk,
                          dt, workspace, workspace_bytes, stream, la::kFeatElu, H);
}

la_status la_forward_causal_grouped(const void* q, const void* k, const void* v, void* o, const float* S0,
                                    const float* z0, float* den_out, float* S_out, float* z_out, int64_t B, int64_t H,
                                    int64_t Hkv, int64_t N, int64_t d, int chunk, la_dtype dt, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    return forward_causal(q, k, v, o, S0, z0, den_out, S_out, z_out, nullptr, 0, B, H, N, d, chunk, dt, workspace,
                          workspace_bytes, stream, la::kFeatElu, Hkv);
}

la_status la_forward_causal_features(const void* fq, const void* fk, const void* v, void* o, const float* S0,
                                     const float* z0, float* den_out, float* S_out, float* z_out, int64_t B, int64_t H,
                                     int64_t N, int64_t d, la_dtype dt, void* workspace, size_t workspace_bytes,
                                     void* stream) {
    return forward_causal(fq, fk, v, o, S0, z0, den_out, S_out, z_out, nullptr, 0, B, H, N, d, 0, dt, workspace,
                          workspace_bytes, stream, la::kFeatGiven, H);
}

la_status la_favor_features(const void* x, const float* omega, void* out, int64_t rows, int64_t d, la_dtype dt,
                            void* stream) {
    if (dt != LA_F32 && dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "dtype %d is not LA_F32 or LA_BF16", (int)dt);
    if (d != 32 && d != 64 && d != 128) return fail(LA_ERR_UNSUPPORTED, "d = %lld; built for 32, 64 and 128", (long long)d);
    if (rows < 0) return fail(LA_ERR_INVALID_ARGUMENT, "negative row count %lld", (long long)rows);
    if (rows > ((int64_t)1 << 40)) return fail(LA_ERR_UNSUPPORTED, "rows = %lld exceeds 2^40", (long long)rows);
    if (!omega) return fail(LA_ERR_INVALID_ARGUMENT, "omega must be non-NULL");
    if (rows > 0 && (!x || !out)) return fail(LA_ERR_INVALID_ARGUMENT, "x and out must be non-NULL");
    const size_t xb = (size_t)rows * d * elem_size(dt);
    const Range in[] = {{"x", x, xb}, {"omega", omega, (size_t)d * d * sizeof(float)}};
    const Range out_r[] = {{"out", out, xb}};
    la_status st = check_ptrs(in, 2, out_r, 1);
    if (st != LA_OK) return st;
    if (rows == 0) return LA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed("favor_features", s, [&] {
        return la::launch_favor_features(dt == LA_BF16 ? la::kBF16 : la::kF32, (int)d, x, omega, out, rows, s);
    });
    if (e != hipSuccess) return hip_fail(e, "favor_features launch");
    return LA_OK;
}

// ---- more random features than d: KF = m / d feature blocks -----------------------------
}  // extern "C"

namespace {

la_status check_blocks(int64_t d, int64_t m) {
    if (m < d || d <= 0 || m % d != 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "m = %lld features must be a positive multiple of d = %lld", (long long)m,
                    (long long)d);
    if (m / d > 64) return fail(LA_ERR_UNSUPPORTED, "m / d = %lld feature blocks; at most 64", (long long)(m / d));
    return LA_OK;
}

// Workspace of a call on KF feature blocks: the m = d call's workspace for B x (H KF)
// heads, then every block's outputs o_j [B][H][KF][N][d] and den_j [B][H][KF][N].
la_status forward_blocks(bool causal, const void* fq, const void* fk, const void* v, void* o, const float* S0,
                         const float* z0, float* den_out, float* S_out, float* z_out, int64_t B, int64_t H, int64_t N,
                         int64_t d, int64_t m, la_dtype dt, void* workspace, size_t workspace_bytes, void* stream) {
    la_status st = check_blocks(d, m);
    if (st != LA_OK) return st;
    bool empty = false;
    if ((st = check_shape(B, H, N, d, 0, dt, &empty)) != LA_OK) return st;
    const int64_t KF = m / d;
    if (KF == 1) {
        return causal ? forward_causal(fq, fk, v, o, S0, z0, den_out, S_out, z_out, nullptr, 0, B, H, N, d, 0, dt,
                                       workspace, workspace_bytes, stream, la::kFeatGiven, H)
                      : forward_noncausal(fq, fk, v, o, nullptr, 0, B, H, N, d, dt, workspace, workspace_bytes, stream,
                                          la::kFeatGiven, 1, den_out);
    }
    if (causal && dt == LA_F32 && d == 128)
        return fail(LA_ERR_UNSUPPORTED, "fp32 causal forward is built for d = 32 and 64");
    if (N > 0 && (!fq || !fk || !v || !o)) return fail(LA_ERR_INVALID_ARGUMENT, "fq, fk, v and o must be non-NULL");
    const size_t tb = (size_t)B * H * N * d * elem_size(dt), fb = tb * KF;
    const size_t Sb = (size_t)B * H * m * d * sizeof(float), zb = (size_t)B * H * m * sizeof(float);
    const Range in[] = {{"fq", fq, fb}, {"fk", fk, fb}, {"v", v, tb}};
    const Range out[] = {{"o", o, tb}, {"den_out", den_out, (size_t)B * H * N * sizeof(float)}};
    if ((st = check_ptrs(in, 3, out, 2)) != LA_OK) return st;
    const Range states[] = {{"S0", S0, Sb}, {"z0", z0, zb}, {"S_out", S_out, Sb}, {"z_out", z_out, zb}};
    for (const Range& r : states)
        for (const Range& x : out)
            if (overlap(r, x)) return fail(LA_ERR_INVALID_ARGUMENT, "%s overlaps output %s", r.name, x.name);
    if (B == 0 || H == 0) return LA_OK;
    const BlockLayout BL = block_layout(causal, B, H, N, d, KF, dt);
    char* ws = static_cast<char*>(workspace);
    if (BL.bytes > 0) {
        if (ws == nullptr) return fail(LA_ERR_WORKSPACE, "workspace is NULL; %zu bytes are needed", BL.bytes);
        if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
            return fail(LA_ERR_INVALID_ARGUMENT, "workspace must be %zu-byte aligned", kAlign);
        if (workspace_bytes < BL.bytes)
            return fail(LA_ERR_WORKSPACE, "workspace has %zu bytes; %zu are needed", workspace_bytes, BL.bytes);
        const Range wsr = {"workspace", ws, BL.bytes};
        for (const Range& r : in)
            if (overlap(wsr, r)) return fail(LA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
        for (const Range& r : out)
            if (overlap(wsr, r)) return fail(LA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
        for (const Range& r : states)
            if (overlap(wsr, r)) return fail(LA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
    }
    // Every block as a head of its own, reading its head's values (Gv = KF) ...
    void* ob = BL.bytes > 0 ? ws + BL.ob : nullptr;
    float* db = BL.bytes > 0 ? reinterpret_cast<float*>(ws + BL.db) : nullptr;
    st = causal ? forward_causal(fq, fk, v, ob, S0, z0, db, S_out, z_out, nullptr, 0, B, H * KF, N, d, 0, dt, ws,
                                 BL.inner, stream, la::kFeatGiven, H * KF, KF)
                : forward_noncausal(fq, fk, v, ob, nullptr, 0, B, H * KF, N, d, dt, ws, BL.inner, stream,
                                    la::kFeatGiven, KF, db);
    if (st != LA_OK || N == 0) return st;
    // ... then num = sum_j num_j and den = sum_j den_j.
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed("combine_blocks", s, [&] {
        return la::launch_combine_blocks(dt == LA_BF16 ? la::kBF16 : la::kF32, (int)d, ob, db, o, den_out, B * H * N,
                                         N, (int)KF, s);
    });
    if (e != hipSuccess) return hip_fail(e, "combine_blocks launch");
    return LA_OK;
}

la_status forward_causal_f128(const void* q, const void* k, const void* v, void* o, const float* S0, const float* z0,
                              float* den_out, float* S_out, float* z_out, int64_t B, int64_t H, int64_t N,
                              void* workspace, size_t workspace_bytes, hipStream_t s) {
    const F128Layout L = f128_layout(B, H, N);
    char* ws = static_cast<char*>(workspace);
    if (ws == nullptr) return fail(LA_ERR_WORKSPACE, "workspace is NULL; %zu bytes are needed", L.bytes);
    if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "workspace must be %zu-byte aligned", kAlign);
    if (workspace_bytes < L.bytes)
        return fail(LA_ERR_WORKSPACE, "workspace has %zu bytes; %zu are needed", workspace_bytes, L.bytes);
    const int64_t BH = B * H;
    const size_t tb = (size_t)BH * N * 128 * sizeof(float), Sb = (size_t)BH * 128 * 128 * sizeof(float);
    const size_t zb = (size_t)BH * 128 * sizeof(float);
    const Range wsr = {"workspace", ws, L.bytes};
    const Range others[] = {{"q", q, tb},          {"k", k, tb},   {"v", v, tb},   {"o", o, tb},
                            {"den_out", den_out, (size_t)BH * N * sizeof(float)}, {"S0", S0, Sb}, {"z0", z0, zb},
                            {"S_out", S_out, Sb}, {"z_out", z_out, zb}};
    for (const Range& r : others)
        if (overlap(wsr, r)) return fail(LA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
    float* fq = reinterpret_cast<float*>(ws + L.fq);
    float* fk = reinterpret_cast<float*>(ws + L.fk);
    float* vh = reinterpret_cast<float*>(ws + L.vh);
    float* oh = reinterpret_cast<float*>(ws + L.oh);
    float* s0h = reinterpret_cast<float*>(ws + L.s0h);
    float* sh = reinterpret_cast<float*>(ws + L.sh);
    hipError_t e;
    if ((e = timed("phi_blocks", s, [&] { return la::launch_phi_blocks(static_cast<const float*>(q), fq, BH, N, 2, 64, s); })) !=
            hipSuccess ||
        (e = timed("phi_blocks", s, [&] { return la::launch_phi_blocks(static_cast<const float*>(k), fk, BH, N, 2, 64, s); })) !=
            hipSuccess)
        return hip_fail(e, "phi_blocks launch");
    for (int h = 0; h < 2; ++h) {
        // The start state is read and the final state written half by half: in place (S_out = S0,
        // z_out = z0) each half is copied out before its columns are overwritten, and z is written last.
        const float* vsrc = static_cast<const float*>(v) + 64 * h;
        if ((e = timed("copy_cols", s, [&] { return la::launch_copy_cols(vh, 64, vsrc, 128, BH * N, 64, s); })) !=
            hipSuccess)
            return hip_fail(e, "copy_cols launch");
        if (S0 != nullptr &&
            (e = timed("copy_cols", s, [&] { return la::launch_copy_cols(s0h, 64, S0 + 64 * h, 128, BH * 128, 64, s); })) !=
                hipSuccess)
            return hip_fail(e, "copy_cols launch");
        const bool last = h == 1;
        const la_status st = forward_blocks(true, fq, fk, vh, oh, S0 != nullptr ? s0h : nullptr, z0,
                                            last ? den_out : nullptr, S_out != nullptr ? sh : nullptr,
                                            last ? z_out : nullptr, B, H, N, 64, 128, LA_F32, ws + L.blk[h],
                                            L.blk_bytes, s);
        if (st != LA_OK) return st;
        float* odst = static_cast<float*>(o) + 64 * h;
        if ((e = timed("copy_cols", s, [&] { return la::launch_copy_cols(odst, 128, oh, 64, BH * N, 64, s); })) !=
            hipSuccess)
            return hip_fail(e, "copy_cols launch");
        if (S_out != nullptr &&
            (e = timed("copy_cols", s, [&] { return la::launch_copy_cols(S_out + 64 * h, 128, sh, 64, BH * 128, 64, s); })) !=
                hipSuccess)
            return hip_fail(e, "copy_cols launch");
    }
    return LA_OK;
}

}  // namespace

extern "C" {

la_status la_features_workspace_size(int causal, int64_t B, int64_t H, int64_t N, int64_t d, int64_t m, la_dtype dt,
                                     size_t* bytes_out) {
    if (bytes_out == nullptr) return fail(LA_ERR_INVALID_ARGUMENT, "bytes_out is NULL");
    la_status st = check_blocks(d, m);
    if (st != LA_OK) return st;
    bool empty = false;
    if ((st = check_shape(B, H, N, d, 0, dt, &empty)) != LA_OK) return st;
    if (causal == 4) {  // non-causal backward: the block heads' workspace, their dv, the row statistics
        const int64_t KF = m / d;
        if (empty) { *bytes_out = 0; return LA_OK; }
        const size_t wb = layout(LA_OP_BWD_NONCAUSAL, B, H * KF, N, d).bytes;
        *bytes_out = KF == 1 ? wb
                             : align_up(wb) + align_up((size_t)B * H * KF * N * d * elem_size(dt)) +
                                   align_up((size_t)B * H * KF * N * 2 * sizeof(float));
        return LA_OK;
    }
    if (causal == 3) {  // causal backward: the block heads' backward workspace, then their dv
        const int64_t KF = m / d;
        if (empty) { *bytes_out = 0; return LA_OK; }
        const size_t wb = layout(LA_OP_BWD_CAUSAL, B, H * KF, N, d).bytes;
        *bytes_out = KF == 1 ? wb : align_up(wb) + align_up((size_t)B * H * KF * N * d * elem_size(dt));
        return LA_OK;
    }
    if (causal == 2) {  // multi-token decode: N = T tokens per call, H query heads
        const int64_t KF = m / d;
        *bytes_out = (empty || KF == 1) ? 0
                                        : align_up((size_t)B * H * KF * N * d * elem_size(dt)) +
                                              align_up((size_t)B * H * KF * N * sizeof(float));
        return LA_OK;
    }
    *bytes_out = empty ? 0 : block_layout(causal != 0, B, H, N, d, m / d, dt).bytes;
    return LA_OK;
}

la_status la_favor_features_backward(const void* x, const float* omega, const void* F, const void* dF, void* dx,
                                     int64_t rows, int64_t d, la_dtype dt, void* stream) {
    if (dt != LA_F32 && dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "dtype %d is not LA_F32 or LA_BF16", (int)dt);
    if (d != 32 && d != 64 && d != 128) return fail(LA_ERR_UNSUPPORTED, "d = %lld; built for 32, 64 and 128", (long long)d);
    if (rows < 0) return fail(LA_ERR_INVALID_ARGUMENT, "negative row count %lld", (long long)rows);
    if (rows > ((int64_t)1 << 40)) return fail(LA_ERR_UNSUPPORTED, "rows = %lld exceeds 2^40", (long long)rows);
    if (!omega) return fail(LA_ERR_INVALID_ARGUMENT, "omega must be non-NULL");
    if (rows > 0 && (!x || !F || !dF || !dx)) return fail(LA_ERR_INVALID_ARGUMENT, "x, F, dF and dx must be non-NULL");
    const size_t xb = (size_t)rows * d * elem_size(dt);
    const Range in[] = {{"x", x, xb}, {"omega", omega, (size_t)d * d * sizeof(float)}, {"F", F, xb}, {"dF", dF, xb}};
    const Range out_r[] = {{"dx", dx, xb}};
    la_status st = check_ptrs(in, 4, out_r, 1);
    if (st != LA_OK) return st;
    if (rows == 0) return LA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed("favor_features_bwd", s, [&] {
        return la::launch_favor_features_bwd(dt == LA_BF16 ? la::kBF16 : la::kF32, (int)d, x, omega, F, dF, dx, rows, s);
    });
    if (e != hipSuccess) return hip_fail(e, "favor_features_bwd launch");
    return LA_OK;
}

la_status la_favor_features_blocks_backward(const void* x, const float* omega, const void* F, const void* dF,
                                            void* dx, int64_t heads, int64_t N, int64_t d, int64_t m, la_dtype dt,
                                            void* stream) {
    la_status st = check_blocks(d, m);
    if (st != LA_OK) return st;
    if (dt != LA_F32 && dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "dtype %d is not LA_F32 or LA_BF16", (int)dt);
    if (d != 32 && d != 64 && d != 128) return fail(LA_ERR_UNSUPPORTED, "d = %lld; built for 32, 64 and 128", (long long)d);
    if (heads < 0 || N < 0) return fail(LA_ERR_INVALID_ARGUMENT, "negative heads %lld or N %lld", (long long)heads,
                                        (long long)N);
    const int64_t rows = heads * N;
    if (rows > ((int64_t)1 << 40)) return fail(LA_ERR_UNSUPPORTED, "rows = %lld exceeds 2^40", (long long)rows);
    if (!omega) return fail(LA_ERR_INVALID_ARGUMENT, "omega must be non-NULL");
    if (rows > 0 && (!x || !F || !dF || !dx)) return fail(LA_ERR_INVALID_ARGUMENT, "x, F, dF and dx must be non-NULL");
    const size_t xb = (size_t)rows * d * elem_size(dt), fb = xb * (size_t)(m / d);
    const Range in[] = {{"x", x, xb}, {"omega", omega, (size_t)m * d * sizeof(float)}, {"F", F, fb}, {"dF", dF, fb}};
    const Range out_r[] = {{"dx", dx, xb}};
    if ((st = check_ptrs(in, 4, out_r, 1)) != LA_OK) return st;
    if (rows == 0) return LA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed("favor_features_bwd", s, [&] {
        return la::launch_favor_features_bwd(dt == LA_BF16 ? la::kBF16 : la::kF32, (int)d, x, omega, F, dF, dx, rows, s,
                                             N, (int)(m / d));
    });
    if (e != hipSuccess) return hip_fail(e, "favor_features_bwd launch");
    return LA_OK;
}

la_status la_favor_features_blocks(const void* x, const float* omega, void* out, int64_t heads, int64_t N, int64_t d,
                                   int64_t m, la_dtype dt, void* stream) {
    la_status st = check_blocks(d, m);
    if (st != LA_OK) return st;
    if (dt != LA_F32 && dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "dtype %d is not LA_F32 or LA_BF16", (int)dt);
    if (d != 32 && d != 64 && d != 128) return fail(LA_ERR_UNSUPPORTED, "d = %lld; built for 32, 64 and 128", (long long)d);
    if (heads < 0 || N < 0) return fail(LA_ERR_INVALID_ARGUMENT, "negative heads %lld or N %lld", (long long)heads,
                                        (long long)N);
    const int64_t rows = heads * N;
    if (rows > ((int64_t)1 << 40)) return fail(LA_ERR_UNSUPPORTED, "rows = %lld exceeds 2^40", (long long)rows);
    if (!omega) return fail(LA_ERR_INVALID_ARGUMENT, "omega must be non-NULL");
    if (rows > 0 && (!x || !out)) return fail(LA_ERR_INVALID_ARGUMENT, "x and out must be non-NULL");
    const size_t xb = (size_t)rows * d * elem_size(dt);
    const Range in[] = {{"x", x, xb}, {"omega", omega, (size_t)m * d * sizeof(float)}};
    const Range out_r[] = {{"out", out, xb * (size_t)(m / d)}};
    if ((st = check_ptrs(in, 2, out_r, 1)) != LA_OK) return st;
    if (rows == 0) return LA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed("favor_features", s, [&] {
        return la::launch_favor_features(dt == LA_BF16 ? la::kBF16 : la::kF32, (int)d, x, omega, out, rows, s, N,
                                         (int)(m / d));
    });
    if (e != hipSuccess) return hip_fail(e, "favor_features launch");
    return LA_OK;
}

la_status la_forward_causal_features_blocks(const void* fq, const void* fk, const void* v, void* o, const float* S0,
                                            const float* z0, float* den_out, float* S_out, float* z_out, int64_t B,
                                            int64_t H, int64_t N, int64_t d, int64_t m, la_dtype dt, void* workspace,
                                            size_t workspace_bytes, void* stream) {
    return forward_blocks(true, fq, fk, v, o, S0, z0, den_out, S_out, z_out, B, H, N, d, m, dt, workspace,
                          workspace_bytes, stream);
}

la_status la_forward_noncausal_features_blocks(const void* fq, const void* fk, const void* v, void* o, float* den_out,
                                               int64_t B, int64_t H, int64_t N, int64_t d, int64_t m, la_dtype dt,
                                               void* workspace, size_t workspace_bytes, void* stream) {
    return forward_blocks(false, fq, fk, v, o, nullptr, nullptr, den_out, nullptr, nullptr, B, H, N, d, m, dt,
                          workspace, workspace_bytes, stream);
}



static la_status backward_f128(bool causal, const void* q, const void* k, const void* v, const void* dout, void* dq,
                               void* dk, void* dv, int64_t B, int64_t H, int64_t N, void* workspace,
                               size_t workspace_bytes, hipStream_t s);

static la_status backward_causal(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                                 void* dv, const void* saved_state, size_t saved_state_bytes, const float* S0,
                                 const float* z0, const float* dSN, const float* dzN, float* dS0, float* dz0,
                                 int64_t B, int64_t H, int64_t N, int64_t d, int chunk, la_dtype dt, void* workspace,
                                 size_t workspace_bytes, void* stream, int feat = la::kFeatElu) {
    bool empty = false;
    la_status st = check_shape(B, H, N, d, chunk, dt, &empty);
    if (st != LA_OK) return st;
    // fp32 at d = 128 runs on feature blocks (backward_causal_f128): the default map from a zero state.
    const bool f128 = dt == LA_F32 && d == 128;
    if (f128 && (feat != la::kFeatElu || S0 || z0 || dSN || dzN || dS0 || dz0))
        return fail(LA_ERR_UNSUPPORTED, "fp32 at d = 128: only the causal backward of phi = elu + 1 from a zero state is built");
    if (N > 0 && (!q || !k || !v || !dout || !dq || !dk || !dv))
        return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v, dout, dq, dk and dv must be non-NULL");
    const size_t tb = (size_t)B * H * N * d * elem_size(dt);
    const size_t sb = saved_state ? saved_bytes(B, H, N, d) : 0;
    if (saved_state && saved_state_bytes < sb)
        return fail(LA_ERR_INVALID_ARGUMENT, "saved_state has %zu bytes; %zu are needed", saved_state_bytes, sb);
    const size_t Sb = (size_t)B * H * d * d * sizeof(float), zb = (size_t)B * H * d * sizeof(float);
    const Range in[] = {{"q", q, tb},           {"k", k, tb},     {"v", v, tb},     {"dout", dout, tb},
                        {"saved_state", saved_state, sb}, {"S0", S0, Sb}, {"z0", z0, zb}, {"dS_out", dSN, Sb},
                        {"dz_out", dzN, zb}};
    const Range out[] = {{"dq", dq, tb}, {"dk", dk, tb}, {"dv", dv, tb}, {"dS0", dS0, Sb}, {"dz0", dz0, zb}};
    if ((st = check_ptrs(in, 9, out, 5)) != LA_OK) return st;
    if (B == 0 || H == 0) return LA_OK;
    const int64_t BH = B * H;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (N == 0) {  // no tokens: the start state's gradient is the final state's
        if (dS0 && (e = timed("fill_zero", s, [&] { return la::launch_copy_or_zero(dS0, dSN, (size_t)BH * d * d, s); })) != hipSuccess)
            return hip_fail(e, "dS0");
        if (dz0 && (e = timed("fill_zero", s, [&] { return la::launch_copy_or_zero(dz0, dzN, (size_t)BH * d, s); })) != hipSuccess)
            return hip_fail(e, "dz0");
        return LA_OK;
    }
    // (fp32 at d = 128 does not read a saved state: it recomputes the forward on the feature blocks.)
    if (f128) return backward_f128(true, q, k, v, dout, dq, dk, dv, B, H, N, workspace, workspace_bytes, s);
    const Layout L = layout(LA_OP_BWD_CAUSAL, B, H, N, d);
    if ((st = check_workspace(L, workspace, workspace_bytes)) != LA_OK) return st;
    const Range wsr[] = {{"workspace", workspace, L.bytes}};
    if ((st = check_ptrs(in, 9, wsr, 1)) != LA_OK) return st;
    for (const Range& r : out)
        if (overlap(wsr[0], r)) return fail(LA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);

    char* ws = static_cast<char*>(workspace);
    float* rec = saved_state ? const_cast<float*>(static_cast<const float*>(saved_state))
                             : reinterpret_cast<float*>(ws + L.rec);
    float* rrec = reinterpret_cast<float*>(ws + L.rrec);
    float* rowstat = reinterpret_cast<float*>(ws + L.rowstat);
    const bool from_state = S0 != nullptr || z0 != nullptr;
    const bool state_grad = dSN != nullptr || dzN != nullptr;
    float* init = from_state ? reinterpret_cast<float*>(ws + L.init) : nullptr;
    float* init_n = from_state ? reinterpret_cast<float*>(ws + L.init_n) : nullptr;
    float* rinit = state_grad ? reinterpret_cast<float*>(ws + L.rinit) : nullptr;
    const int idt = dt == LA_BF16 ? la::kBF16 : la::kF32;
    if (from_state &&
        (e = timed("state_split", s, [&] { return la::launch_state_split((int)d, S0, z0, init, init_n, BH, s); })) !=
            hipSuccess)
        return hip_fail(e, "state_split launch");
    // The final-state gradients as an unsplit record: the suffix sums carry no split.
    if (state_grad && (e = timed("state_split", s, [&] {
                           return la::launch_state_split((int)d, dSN, dzN, rinit, nullptr, BH, s, la::kFeatGiven);
                       })) != hipSuccess)
        return hip_fail(e, "state_split launch");
    if (saved_state == nullptr) {
        if ((e = timed("seg_state", s, [&] { return la::launch_seg_state(idt, (int)d, k, v, rec, BH, N, L.plan, s, feat); })) != hipSuccess)
            return hip_fail(e, "seg_state launch");
        if (L.plan.scan &&
            (e = timed("scan", s, [&] { return la::launch_scan((int)d, rec, BH, L.plan.nseg, 1, s, init); })) != hipSuccess)
            return hip_fail(e, "scan launch");
    }
    if (L.fused) {
        unsigned long long* flags = reinterpret_cast<unsigned long long*>(ws + L.flags);
        unsigned* giveups = reinterpret_cast<unsigned*>(ws + L.giveups);
        const unsigned long long epoch = next_epoch();
        if ((e = timed("bwd_fused", s, [&] {
                 return la::launch_bwd_fused(idt, (int)d, q, k, v, dout, dq, dk, dv, rowstat, rrec, rec, flags, giveups,
                                             epoch,
                                             g_wait_limit.load(std::memory_order_relaxed), BH, N, L.plan, s, init,
                                             init_n, rinit, dS0, dz0, feat);
             })) != hipSuccess)
            return hip_fail(e, "bwd_fused launch");
        return LA_OK;
    }
    if ((e = timed("bwd_prefix", s, [&] { return la::launch_bwd_prefix(idt, (int)d, q, k, v, dout, dq, rowstat, rrec, rec, BH, N, L.plan, s, init, init_n, feat); })) !=
        hipSuccess)
        return hip_fail(e, "bwd_prefix launch");
    if (!la::prefix_forms_records((int)d) &&
        (e = timed("rseg", s, [&] { return la::launch_rseg(idt, (int)d, q, dout, rowstat, rrec, BH, N, L.plan, s, feat); })) !=
            hipSuccess)
        return hip_fail(e, "rseg launch");
    if (L.plan.scan && (e = timed("rscan", s, [&] { return la::launch_scan((int)d, rrec, BH, L.plan.nseg, -1, s, rinit); })) != hipSuccess)
        return hip_fail(e, "rscan launch");
    if ((e = timed("bwd_suffix", s, [&] { return la::launch_bwd_suffix(idt, (int)d, q, k, v, dout, dk, dv, rowstat, rrec, BH, N, L.plan, s, rinit, dS0, dz0, feat); })) !=
        hipSuccess)
        return hip_fail(e, "bwd_suffix launch");
    return LA_OK;
}

la_status la_backward_causal(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                             void* dv, const void* saved_state, size_t saved_state_bytes, int64_t B, int64_t H,
                             int64_t N, int64_t d, int chunk, la_dtype dt, void* workspace, size_t workspace_bytes,
                             void* stream) {
    return backward_causal(q, k, v, dout, dq, dk, dv, saved_state, saved_state_bytes, nullptr, nullptr, nullptr,
                           nullptr, nullptr, nullptr, B, H, N, d, chunk, dt, workspace, workspace_bytes, stream);
}

la_status la_backward_causal_state(const void* q, const void* k, const void* v, const void* dout, const float* S0,
                                   const float* z0, const float* dS_out, const float* dz_out, void* dq, void* dk,
                                   void* dv, float* dS0, float* dz0, int64_t B, int64_t H, int64_t N, int64_t d,
                                   int chunk, la_dtype dt, void* workspace, size_t workspace_bytes, void* stream) {
    return backward_causal(q, k, v, dout, dq, dk, dv, nullptr, 0, S0, z0, dS_out, dz_out, dS0, dz0, B, H, N, d, chunk,
                           dt, workspace, workspace_bytes, stream);
}

la_status la_wait_failures(la_op op, const void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t N,
                           int64_t d, la_dtype dt, void* stream, int64_t* failures_out) {
    if (failures_out == nullptr) return fail(LA_ERR_INVALID_ARGUMENT, "failures_out is NULL");
    if (op != LA_OP_FWD_CAUSAL && op != LA_OP_BWD_CAUSAL)
        return fail(LA_ERR_INVALID_ARGUMENT, "op %d has no waits between workgroups", (int)op);
    bool empty = false;
    la_status st = check_shape(B, H, N, d, 0, dt, &empty);
    if (st != LA_OK) return st;
    *failures_out = 0;
    if (empty) return LA_OK;
    if (op == LA_OP_BWD_CAUSAL && dt == LA_F32 && d == 128) return LA_OK;  // feature-block passes: no waits
    if (op == LA_OP_FWD_CAUSAL && dt == LA_F32 && d == 128) {  // the two value halves' launches on feature blocks
        const F128Layout F = f128_layout(B, H, N);
        const Layout Li = layout(LA_OP_FWD_CAUSAL, B, 2 * H, N, 64);
        if (Li.plan.scan) return LA_OK;
        if (workspace == nullptr || workspace_bytes < F.bytes)
            return fail(LA_ERR_WORKSPACE, "workspace has %zu bytes; %zu are needed", workspace_bytes, F.bytes);
        hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "stream synchronize");
        std::vector<unsigned> slots((size_t)Li.heads * Li.plan.nseg);
        int64_t n = 0;
        for (int h = 0; h < 2; ++h) {
            e = hipMemcpy(slots.data(), static_cast<const char*>(workspace) + F.blk[h] + Li.giveups,
                          slots.size() * sizeof(unsigned), hipMemcpyDeviceToHost);
            if (e != hipSuccess) return hip_fail(e, "copy of the wait counts");
            for (unsigned c : slots) n += c;
        }
        *failures_out = n;
        return LA_OK;
    }
    const Layout L = layout(op, B, H, N, d);
    if (op == LA_OP_BWD_CAUSAL ? !L.fused : L.plan.scan) return LA_OK;  // launches that wait for nothing
    if ((st = check_workspace(L, workspace, workspace_bytes)) != LA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    std::vector<unsigned> slots((size_t)L.heads * L.plan.nseg);
    e = hipMemcpy(slots.data(), static_cast<const char*>(workspace) + L.giveups, slots.size() * sizeof(unsigned),
                  hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "copy of the wait counts");
    int64_t n = 0;
    for (unsigned c : slots) n += c;
    *failures_out = n;
    return LA_OK;
}

static la_status backward_noncausal(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                                    void* dv, const void* saved_state, size_t saved_state_bytes, int64_t B, int64_t H,
                                    int64_t N, int64_t d, la_dtype dt, void* workspace, size_t workspace_bytes,
                                    void* stream, int feat) {
    bool empty = false;
    la_status st = check_shape(B, H, N, d, 0, dt, &empty);
    if (st != LA_OK) return st;
    // fp32 at d = 128 runs on feature blocks (backward_f128), for phi = elu + 1.
    const bool f128 = dt == LA_F32 && d == 128;
    if (f128 && feat != la::kFeatElu)
        return fail(LA_ERR_UNSUPPORTED, "fp32 at d = 128: only the non-causal backward of phi = elu + 1 is built");
    if (N > 0 && (!q || !k || !v || !dout || !dq || !dk || !dv))
        return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v, dout, dq, dk and dv must be non-NULL");
    const size_t tb = (size_t)B * H * N * d * elem_size(dt);
    const size_t sb = saved_state ? saved_bytes(B, H, N, d) : 0;
    if (saved_state && saved_state_bytes < sb)
        return fail(LA_ERR_INVALID_ARGUMENT, "saved_state has %zu bytes; %zu are needed", saved_state_bytes, sb);
    const Range in[] = {{"q", q, tb}, {"k", k, tb}, {"v", v, tb}, {"dout", dout, tb}, {"saved_state", saved_state, sb}};
    const Range out[] = {{"dq", dq, tb}, {"dk", dk, tb}, {"dv", dv, tb}};
    if ((st = check_ptrs(in, 5, out, 3)) != LA_OK) return st;
    if (empty) return LA_OK;
    // (fp32 at d = 128 does not read a saved state: it recomputes the forward on the feature blocks.)
    if (f128)
        return backward_f128(false, q, k, v, dout, dq, dk, dv, B, H, N, workspace, workspace_bytes,
                             static_cast<hipStream_t>(stream));
    const Layout L = layout(LA_OP_BWD_NONCAUSAL, B, H, N, d);
    if ((st = check_workspace(L, workspace, workspace_bytes)) != LA_OK) return st;
    const Range wsr[] = {{"workspace", workspace, L.bytes}};
    if ((st = check_ptrs(in, 5, wsr, 1)) != LA_OK) return st;
    for (const Range& r : out)
        if (overlap(wsr[0], r)) return fail(LA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);

    char* ws = static_cast<char*>(workspace);
    // With a saved state the forward's totals are read from it; otherwise they are rebuilt here.
    float* total = saved_state ? reinterpret_cast<float*>(const_cast<char*>(static_cast<const char*>(saved_state)) +
                                                          saved_records_bytes(B, H, N, d))
                               : reinterpret_cast<float*>(ws + L.total);
    float* rec = reinterpret_cast<float*>(ws + L.rec);
    float* rrec = reinterpret_cast<float*>(ws + L.rrec);
    float* rtotal = reinterpret_cast<float*>(ws + L.rtotal);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t BH = B * H;
    const int idt = dt == LA_BF16 ? la::kBF16 : la::kF32;
    hipError_t e;
    if (saved_state == nullptr) {
        if ((e = timed("seg_state", s, [&] { return la::launch_seg_state(idt, (int)d, k, v, rec, BH, N, L.plan, s, feat); })) != hipSuccess)
            return hip_fail(e, "seg_state launch");
        if ((e = timed("total", s, [&] { return la::launch_total((int)d, rec, total, BH, L.plan.nseg, s); })) != hipSuccess)
            return hip_fail(e, "total launch");
    }
    if ((e = timed("ncbwd_q", s, [&] {
             return la::launch_ncbwd_q(idt, (int)d, q, dout, dq, total, 1, rrec, BH, N, L.plan, s, feat);
         })) != hipSuccess)
        return hip_fail(e, "ncbwd_q launch");
    if ((e = timed("total", s, [&] { return la::launch_total((int)d, rrec, rtotal, BH, L.plan.nseg, s); })) != hipSuccess)
        return hip_fail(e, "total launch");
    if ((e = timed("ncbwd_kv", s, [&] {
             return la::launch_ncbwd_kv(idt, (int)d, k, v, dk, dv, rtotal, 1, BH, N, L.plan, s, feat);
         })) != hipSuccess)
        return hip_fail(e, "ncbwd_kv launch");
    return LA_OK;
}

la_status la_backward_noncausal(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                                void* dv, const void* saved_state, size_t saved_state_bytes, int64_t B, int64_t H,
                                int64_t N, int64_t d, la_dtype dt, void* workspace, size_t workspace_bytes,
                                void* stream) {
    return backward_noncausal(q, k, v, dout, dq, dk, dv, saved_state, saved_state_bytes, B, H, N, d, dt, workspace,
                              workspace_bytes, stream, la::kFeatElu);
}

la_status la_backward_causal_features(const void* fq, const void* fk, const void* v, const void* dout, void* dfq,
                                      void* dfk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, la_dtype dt,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    return backward_causal(fq, fk, v, dout, dfq, dfk, dv, nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, B, H, N, d, 0, dt, workspace, workspace_bytes, stream, la::kFeatGiven);
}

la_status la_backward_noncausal_features(const void* fq, const void* fk, const void* v, const void* dout, void* dfq,
                                         void* dfk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, la_dtype dt,
                                         void* workspace, size_t workspace_bytes, void* stream) {
    return backward_noncausal(fq, fk, v, dout, dfq, dfk, dv, nullptr, 0, B, H, N, d, dt, workspace, workspace_bytes,
                              stream, la::kFeatGiven);
}

la_status la_backward_causal_features_blocks(const void* fq, const void* fk, const void* v, const void* dout,
                                             const float* den, const void* o, void* dfq, void* dfk, void* dv, int64_t B, int64_t H,
                                             int64_t N, int64_t d, int64_t m, la_dtype dt, void* workspace,
                                             size_t workspace_bytes, void* stream) {
    la_status st = check_blocks(d, m);
    if (st != LA_OK) return st;
    const int64_t KF = m / d;
    if (KF == 1)
        return backward_causal(fq, fk, v, dout, dfq, dfk, dv, nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr,
                               nullptr, B, H, N, d, 0, dt, workspace, workspace_bytes, stream, la::kFeatGiven);
    bool empty = false;
    if ((st = check_shape(B, H * KF, N, d, 0, dt, &empty)) != LA_OK) return st;
    if (dt == LA_F32 && d == 128) return fail(LA_ERR_UNSUPPORTED, "fp32 causal backward is built for d = 32 and 64");
    if (N > 0 && (!fq || !fk || !v || !dout || !den || !dfq || !dfk || !dv))
        return fail(LA_ERR_INVALID_ARGUMENT, "fq, fk, v, dout, den, dfq, dfk and dv must be non-NULL");
    const size_t tb = (size_t)B * H * N * d * elem_size(dt), fb = tb * KF;
    const Range in[] = {{"fq", fq, fb}, {"fk", fk, fb}, {"v", v, tb}, {"dout", dout, tb},
                        {"den", den, (size_t)B * H * N * sizeof(float)}, {"o", o, o ? tb : 0}};
    const Range out[] = {{"dfq", dfq, fb}, {"dfk", dfk, fb}, {"dv", dv, tb}};
    if ((st = check_ptrs(in, 6, out, 3)) != LA_OK) return st;
    if (empty) return LA_OK;
    const int64_t BHb = B * H * KF;  // block heads
    const Layout L = layout(LA_OP_BWD_CAUSAL, B, H * KF, N, d);
    const size_t dvb_off = align_up(L.bytes), need = dvb_off + align_up(fb);
    if (workspace == nullptr) return fail(LA_ERR_WORKSPACE, "workspace is NULL; %zu bytes are needed", need);
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "workspace must be %zu-byte aligned", kAlign);
    if (workspace_bytes < need)
        return fail(LA_ERR_WORKSPACE, "workspace has %zu bytes; %zu are needed", workspace_bytes, need);
    const Range wsr[] = {{"workspace", workspace, need}};
    if ((st = check_ptrs(in, 6, wsr, 1)) != LA_OK) return st;
    for (const Range& r : out)
        if (overlap(wsr[0], r)) return fail(LA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
    if ((int64_t)L.plan.nseg * BHb > ((int64_t)1 << 24))
        return fail(LA_ERR_UNSUPPORTED, "%lld workgroups exceed the 2^24 grid limit", (long long)L.plan.nseg * BHb);

    char* ws = static_cast<char*>(workspace);
    float* rec = reinterpret_cast<float*>(ws + L.rec);
    float* rrec = reinterpret_cast<float*>(ws + L.rrec);
    float* rowstat = reinterpret_cast<float*>(ws + L.rowstat);
    void* dvb = ws + dvb_off;
    const int idt = dt == LA_BF16 ? la::kBF16 : la::kF32;
    const int G = (int)KF;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    // Every block as a head of its own over its head's values and upstream gradient: the key
    // aggregates, then the rows' G . num of each block with the head's den and G ...
    if ((e = timed("seg_state", s, [&] {
             return la::launch_seg_state(idt, (int)d, fk, v, rec, BHb, N, L.plan, s, la::kFeatGiven, G);
         })) != hipSuccess)
        return hip_fail(e, "seg_state launch");
    if (L.plan.scan &&
        (e = timed("scan", s, [&] { return la::launch_scan((int)d, rec, BHb, L.plan.nseg, 1, s, nullptr); })) != hipSuccess)
        return hip_fail(e, "scan launch");
    // (With the forward's output, g = -G . O of every row comes from one elementwise pass instead.)
    if (o != nullptr) {
        if ((e = timed("stats_from_output", s, [&] {
                 return la::launch_stats_from_output(idt, (int)d, dout, o, den, rowstat, B * H * N, N, G, s);
             })) != hipSuccess)
            return hip_fail(e, "stats_from_output launch");
    } else {
        if ((e = timed("bwd_prefix", s, [&] {
                 return la::launch_bwd_prefix(idt, (int)d, fq, fk, v, dout, dfq, rowstat, rrec, rec, BHb, N, L.plan, s,
                                              nullptr, nullptr, la::kFeatGiven, 1, G, den);
             })) != hipSuccess)
            return hip_fail(e, "bwd_prefix launch");
        // ... the head's g = -(sum_j G . num_j) / den for every block ...
        if ((e = timed("combine_stats", s, [&] { return la::launch_combine_stats(rowstat, B * H * N, N, G, s); })) !=
            hipSuccess)
            return hip_fail(e, "combine_stats launch");
    }
    // ... then each block's sweeps with the head's (den, g): dfq, dfk and its share of dv.
    if ((e = timed("bwd_prefix", s, [&] {
             return la::launch_bwd_prefix(idt, (int)d, fq, fk, v, dout, dfq, rowstat, rrec, rec, BHb, N, L.plan, s,
                                          nullptr, nullptr, la::kFeatGiven, 2, G, nullptr);
         })) != hipSuccess)
        return hip_fail(e, "bwd_prefix launch");
    if (!la::prefix_forms_records((int)d) && (e = timed("rseg", s, [&] {
                                                  return la::launch_rseg(idt, (int)d, fq, dout, rowstat, rrec, BHb, N,
                                                                         L.plan, s, la::kFeatGiven, G);
                                              })) != hipSuccess)
        return hip_fail(e, "rseg launch");
    if (L.plan.scan &&
        (e = timed("rscan", s, [&] { return la::launch_scan((int)d, rrec, BHb, L.plan.nseg, -1, s, nullptr); })) != hipSuccess)
        return hip_fail(e, "rscan launch");
    if ((e = timed("bwd_suffix", s, [&] {
             return la::launch_bwd_suffix(idt, (int)d, fq, fk, v, dout, dfk, dvb, rowstat, rrec, BHb, N, L.plan, s,
                                          nullptr, nullptr, nullptr, la::kFeatGiven, G);
         })) != hipSuccess)
        return hip_fail(e, "bwd_suffix launch");
    if ((e = timed("combine_blocks", s, [&] {
             return la::launch_combine_blocks(idt, (int)d, dvb, nullptr, dv, nullptr, B * H * N, N, G, s);
         })) != hipSuccess)
        return hip_fail(e, "combine_blocks launch");
    return LA_OK;
}

la_status la_backward_noncausal_features_blocks(const void* fq, const void* fk, const void* v, const void* dout,
                                                const float* den, const void* o, void* dfq, void* dfk, void* dv, int64_t B,
                                                int64_t H, int64_t N, int64_t d, int64_t m, la_dtype dt,
                                                void* workspace, size_t workspace_bytes, void* stream) {
    la_status st = check_blocks(d, m);
    if (st != LA_OK) return st;
    const int64_t KF = m / d;
    if (KF == 1)
        return backward_noncausal(fq, fk, v, dout, dfq, dfk, dv, nullptr, 0, B, H, N, d, dt, workspace,
                                  workspace_bytes, stream, la::kFeatGiven);
    bool empty = false;
    if ((st = check_shape(B, H * KF, N, d, 0, dt, &empty)) != LA_OK) return st;
    if (dt == LA_F32 && d == 128) return fail(LA_ERR_UNSUPPORTED, "fp32 non-causal backward is built for d = 32 and 64");
    if (N > 0 && (!fq || !fk || !v || !dout || !den || !dfq || !dfk || !dv))
        return fail(LA_ERR_INVALID_ARGUMENT, "fq, fk, v, dout, den, dfq, dfk and dv must be non-NULL");
    const size_t tb = (size_t)B * H * N * d * elem_size(dt), fb = tb * KF;
    const Range in[] = {{"fq", fq, fb}, {"fk", fk, fb}, {"v", v, tb}, {"dout", dout, tb},
                        {"den", den, (size_t)B * H * N * sizeof(float)}, {"o", o, o ? tb : 0}};
    const Range out[] = {{"dfq", dfq, fb}, {"dfk", dfk, fb}, {"dv", dv, tb}};
    if ((st = check_ptrs(in, 6, out, 3)) != LA_OK) return st;
    if (empty) return LA_OK;
    const int64_t BHb = B * H * KF;  // block heads
    const Layout L = layout(LA_OP_BWD_NONCAUSAL, B, H * KF, N, d);
    const size_t dvb_off = align_up(L.bytes), rs_off = dvb_off + align_up(fb);
    const size_t need = rs_off + align_up((size_t)BHb * N * 2 * sizeof(float));
    if (workspace == nullptr) return fail(LA_ERR_WORKSPACE, "workspace is NULL; %zu bytes are needed", need);
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "workspace must be %zu-byte aligned", kAlign);
    if (workspace_bytes < need)
        return fail(LA_ERR_WORKSPACE, "workspace has %zu bytes; %zu are needed", workspace_bytes, need);
    const Range wsr[] = {{"workspace", workspace, need}};
    if ((st = check_ptrs(in, 6, wsr, 1)) != LA_OK) return st;
    for (const Range& r : out)
        if (overlap(wsr[0], r)) return fail(LA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
    if ((int64_t)L.plan.nseg * BHb > ((int64_t)1 << 24))
        return fail(LA_ERR_UNSUPPORTED, "%lld workgroups exceed the 2^24 grid limit", (long long)L.plan.nseg * BHb);

    char* ws = static_cast<char*>(workspace);
    float* total = reinterpret_cast<float*>(ws + L.total);
    float* rec = reinterpret_cast<float*>(ws + L.rec);
    float* rrec = reinterpret_cast<float*>(ws + L.rrec);
    float* rtotal = reinterpret_cast<float*>(ws + L.rtotal);
    void* dvb = ws + dvb_off;
    float* rowstat = reinterpret_cast<float*>(ws + rs_off);
    const int idt = dt == LA_BF16 ? la::kBF16 : la::kF32;
    const int G = (int)KF;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    // Every block as a head of its own over its head's values and upstream gradient: its key
    // state, then the rows' G . num of each block with the head's den and G ...
    if ((e = timed("seg_state", s, [&] {
             return la::launch_seg_state(idt, (int)d, fk, v, rec, BHb, N, L.plan, s, la::kFeatGiven, G);
         })) != hipSuccess)
        return hip_fail(e, "seg_state launch");
    if ((e = timed("total", s, [&] { return la::launch_total((int)d, rec, total, BHb, L.plan.nseg, s); })) != hipSuccess)
        return hip_fail(e, "total launch");
    // (With the forward's output, g = -G . O of every row comes from one elementwise pass instead.)
    if (o != nullptr) {
        if ((e = timed("stats_from_output", s, [&] {
                 return la::launch_stats_from_output(idt, (int)d, dout, o, den, rowstat, B * H * N, N, G, s);
             })) != hipSuccess)
            return hip_fail(e, "stats_from_output launch");
    } else {
        if ((e = timed("ncbwd_q", s, [&] {
                 return la::launch_ncbwd_q(idt, (int)d, fq, dout, dfq, total, 1, rrec, BHb, N, L.plan, s,
                                           la::kFeatGiven, 1, G, den, rowstat);
             })) != hipSuccess)
            return hip_fail(e, "ncbwd_q launch");
        // ... the head's g = -(sum_j G . num_j) / den for every block ...
        if ((e = timed("combine_stats", s, [&] { return la::launch_combine_stats(rowstat, B * H * N, N, G, s); })) !=
            hipSuccess)
            return hip_fail(e, "combine_stats launch");
    }
    // ... then each block's passes with the head's (den, g): dfq_j and (R_j, r_j), dfk_j and its share of dv.
    if ((e = timed("ncbwd_q", s, [&] {
             return la::launch_ncbwd_q(idt, (int)d, fq, dout, dfq, total, 1, rrec, BHb, N, L.plan, s, la::kFeatGiven,
                                       2, G, nullptr, rowstat);
         })) != hipSuccess)
        return hip_fail(e, "ncbwd_q launch");
    if ((e = timed("total", s, [&] { return la::launch_total((int)d, rrec, rtotal, BHb, L.plan.nseg, s); })) != hipSuccess)
        return hip_fail(e, "total launch");
    if ((e = timed("ncbwd_kv", s, [&] {
             return la::launch_ncbwd_kv(idt, (int)d, fk, v, dfk, dvb, rtotal, 1, BHb, N, L.plan, s, la::kFeatGiven, G);
         })) != hipSuccess)
        return hip_fail(e, "ncbwd_kv launch");
    if ((e = timed("combine_blocks", s, [&] {
             return la::launch_combine_blocks(idt, (int)d, dvb, nullptr, dv, nullptr, B * H * N, N, G, s);
         })) != hipSuccess)
        return hip_fail(e, "combine_blocks launch");
    return LA_OK;
}

la_status la_decode_step(float* S, float* z, const void* q, const void* k, const void* v, void* o, int64_t B,
                         int64_t H, int64_t d, la_dtype dt, void* stream) {
    if (dt != LA_F32 && dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "dtype %d is not LA_F32 or LA_BF16", (int)dt);
    if (d != 32 && d != 64 && d != 128) return fail(LA_ERR_UNSUPPORTED, "d = %lld; built for 32, 64 and 128", (long long)d);
    if (B < 0 || H < 0) return fail(LA_ERR_INVALID_ARGUMENT, "negative size (B=%lld H=%lld)", (long long)B, (long long)H);
    if (B > 0 && H > ((int64_t)1 << 24) / B) return fail(LA_ERR_UNSUPPORTED, "B*H exceeds 2^24 heads");
    if (!S || !z || !q || !k || !v || !o) return fail(LA_ERR_INVALID_ARGUMENT, "S, z, q, k, v and o must be non-NULL");
    const int64_t BH = B * H;
    const size_t vb = (size_t)BH * d * elem_size(dt);
    const Range in[] = {{"q", q, vb}, {"k", k, vb}, {"v", v, vb}};
    const Range out[] = {{"S", S, (size_t)BH * d * d * sizeof(float)},
                         {"z", z, (size_t)BH * d * sizeof(float)},
                         {"o", o, vb}};
    la_status st = check_ptrs(in, 3, out, 3);
    if (st != LA_OK) return st;
    if (BH == 0) return LA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed("decode", s, [&] {
        return la::launch_decode(dt == LA_BF16 ? la::kBF16 : la::kF32, (int)d, S, z, q, k, v, o, BH, s);
    });
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return LA_OK;
}

// KF > 1: features in KF blocks (q [B][H][KF][T][d], k [B][Hkv][KF][T][d], states
// [B][Hkv][KF d][d]); the blocks' outputs and denominators go to the workspace and are
// combined into o.
static la_status decode_steps(float* S, float* z, const void* q, const void* k, const void* v, void* o, int64_t B,
                              int64_t H, int64_t Hkv, int64_t T, int64_t d, la_dtype dt, void* stream, int feat,
                              int64_t KF = 1, void* workspace = nullptr, size_t workspace_bytes = 0) {
    if (dt != LA_F32 && dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "dtype %d is not LA_F32 or LA_BF16", (int)dt);
    if (d != 32 && d != 64 && d != 128) return fail(LA_ERR_UNSUPPORTED, "d = %lld; built for 32, 64 and 128", (long long)d);
    if (B < 0 || H < 0 || Hkv < 0 || T < 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "negative size (B=%lld H=%lld Hkv=%lld T=%lld)", (long long)B, (long long)H,
                    (long long)Hkv, (long long)T);
    if ((Hkv == 0) != (H == 0) || (Hkv > 0 && H % Hkv != 0))
        return fail(LA_ERR_INVALID_ARGUMENT, "H = %lld query heads must be a multiple of Hkv = %lld", (long long)H,
                    (long long)Hkv);
    if (B > 0 && H > ((int64_t)1 << 24) / B) return fail(LA_ERR_UNSUPPORTED, "B*H exceeds 2^24 heads");
    if (T > ((int64_t)1 << 24)) return fail(LA_ERR_UNSUPPORTED, "T = %lld exceeds 2^24 tokens per call", (long long)T);
    if (!S || !z) return fail(LA_ERR_INVALID_ARGUMENT, "S and z must be non-NULL");
    // Empty token tensors (T = 0) may come as NULL pointers.
    if (T > 0 && (!q || !k || !v || !o)) return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v and o must be non-NULL");
    const int64_t BHkv = B * Hkv;
    const size_t qb = (size_t)B * H * T * d * elem_size(dt), kb = (size_t)BHkv * T * d * elem_size(dt);
    const Range in[] = {{"q", q, qb * KF}, {"k", k, kb * KF}, {"v", v, kb}};
    const Range out[] = {{"S", S, (size_t)BHkv * KF * d * d * sizeof(float)},
                         {"z", z, (size_t)BHkv * KF * d * sizeof(float)},
                         {"o", o, qb}};
    la_status st = check_ptrs(in, 3, out, 3);
    if (st != LA_OK) return st;
    if (BHkv == 0 || T == 0) return LA_OK;
    const int idt = dt == LA_BF16 ? la::kBF16 : la::kF32;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ob = o;
    float* db = nullptr;
    if (KF > 1) {  // the blocks' outputs and denominators, then their combination
        const size_t obb = align_up(qb * KF), need = obb + align_up((size_t)B * H * KF * T * sizeof(float));
        if (workspace == nullptr) return fail(LA_ERR_WORKSPACE, "workspace is NULL; %zu bytes are needed", need);
        if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
            return fail(LA_ERR_INVALID_ARGUMENT, "workspace must be %zu-byte aligned", kAlign);
        if (workspace_bytes < need)
            return fail(LA_ERR_WORKSPACE, "workspace has %zu bytes; %zu are needed", workspace_bytes, need);
        const Range wsr = {"workspace", workspace, need};
        for (const Range& r : in)
            if (overlap(wsr, r)) return fail(LA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
        for (const Range& r : out)
            if (overlap(wsr, r)) return fail(LA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
        ob = workspace;
        db = reinterpret_cast<float*>(static_cast<char*>(workspace) + obb);
    }
    hipError_t e = timed("decode_steps", s, [&] {
        return la::launch_decode_steps(idt, (int)d, S, z, q, k, v, ob, BHkv, T, H / Hkv, s, feat, (int)KF, db);
    });
    if (e != hipSuccess) return hip_fail(e, "decode_steps launch");
    if (KF > 1) {
        e = timed("combine_blocks", s, [&] {
            return la::launch_combine_blocks(idt, (int)d, ob, db, o, nullptr, B * H * T, T, (int)KF, s);
        });
        if (e != hipSuccess) return hip_fail(e, "combine_blocks launch");
    }
    return LA_OK;
}

la_status la_decode_steps(float* S, float* z, const void* q, const void* k, const void* v, void* o, int64_t B,
                          int64_t H, int64_t Hkv, int64_t T, int64_t d, la_dtype dt, void* stream) {
    return decode_steps(S, z, q, k, v, o, B, H, Hkv, T, d, dt, stream, la::kFeatElu);
}

la_status la_decode_steps_features(float* S, float* z, const void* fq, const void* fk, const void* v, void* o,
                                   int64_t B, int64_t H, int64_t Hkv, int64_t T, int64_t d, la_dtype dt,
                                   void* stream) {
    return decode_steps(S, z, fq, fk, v, o, B, H, Hkv, T, d, dt, stream, la::kFeatGiven);
}

la_status la_decode_steps_features_blocks(float* S, float* z, const void* fq, const void* fk, const void* v, void* o,
                                          int64_t B, int64_t H, int64_t Hkv, int64_t T, int64_t d, int64_t m,
                                          la_dtype dt, void* workspace, size_t workspace_bytes, void* stream) {
    la_status st = check_blocks(d, m);
    if (st != LA_OK) return st;
    return decode_steps(S, z, fq, fk, v, o, B, H, Hkv, T, d, dt, stream, la::kFeatGiven, m / d, workspace,
                        workspace_bytes);
}

}  // extern "C"

static la_status backward_f128(bool causal, const void* q, const void* k, const void* v, const void* dout, void* dq,
                               void* dk, void* dv, int64_t B, int64_t H, int64_t N, void* workspace,
                               size_t workspace_bytes, hipStream_t s) {
    const B128Layout L = b128_layout(causal, B, H, N);
    char* ws = static_cast<char*>(workspace);
    if (ws == nullptr) return fail(LA_ERR_WORKSPACE, "workspace is NULL; %zu bytes are needed", L.bytes);
    if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "workspace must be %zu-byte aligned", kAlign);
    if (workspace_bytes < L.bytes)
        return fail(LA_ERR_WORKSPACE, "workspace has %zu bytes; %zu are needed", workspace_bytes, L.bytes);
    const int64_t BH = B * H;
    const size_t tb = (size_t)BH * N * 128 * sizeof(float);
    const Range wsr = {"workspace", ws, L.bytes};
    const Range others[] = {{"q", q, tb},   {"k", k, tb},   {"v", v, tb},  {"dout", dout, tb},
                            {"dq", dq, tb}, {"dk", dk, tb}, {"dv", dv, tb}};
    for (const Range& r : others)
        if (overlap(wsr, r)) return fail(LA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
    float* fq = reinterpret_cast<float*>(ws + L.fq);
    float* fk = reinterpret_cast<float*>(ws + L.fk);
    float* vh = reinterpret_cast<float*>(ws + L.vh);
    float* oh = reinterpret_cast<float*>(ws + L.oh);
    float* doh = reinterpret_cast<float*>(ws + L.doh);
    float* dvh = reinterpret_cast<float*>(ws + L.dvh);
    float* den = reinterpret_cast<float*>(ws + L.den);
    const float* fq_in = static_cast<const float*>(q);
    const float* fk_in = static_cast<const float*>(k);
    hipError_t e;
    if ((e = timed("phi_blocks", s, [&] { return la::launch_phi_blocks(fq_in, fq, BH, N, 2, 64, s); })) != hipSuccess ||
        (e = timed("phi_blocks", s, [&] { return la::launch_phi_blocks(fk_in, fk, BH, N, 2, 64, s); })) != hipSuccess)
        return hip_fail(e, "phi_blocks launch");
    for (int h = 0; h < 2; ++h) {
        const float* vsrc = static_cast<const float*>(v) + 64 * h;
        const float* dosrc = static_cast<const float*>(dout) + 64 * h;
        if ((e = timed("copy_cols", s, [&] { return la::launch_copy_cols(vh, 64, vsrc, 128, BH * N, 64, s); })) !=
                hipSuccess ||
            (e = timed("copy_cols", s, [&] { return la::launch_copy_cols(doh, 64, dosrc, 128, BH * N, 64, s); })) !=
                hipSuccess)
            return hip_fail(e, "copy_cols launch");
        la_status st = forward_blocks(causal, fq, fk, vh, oh, nullptr, nullptr, den, nullptr, nullptr, B, H, N, 64,
                                      128, LA_F32, ws + L.fwd, L.fwd_bytes, s);
        if (st != LA_OK) return st;
        st = causal ? la_backward_causal_features_blocks(fq, fk, vh, doh, den, oh, ws + L.dfq[h], ws + L.dfk[h], dvh,
                                                         B, H, N, 64, 128, LA_F32, ws + L.bwd, L.bwd_bytes, s)
                    : la_backward_noncausal_features_blocks(fq, fk, vh, doh, den, oh, ws + L.dfq[h], ws + L.dfk[h],
                                                            dvh, B, H, N, 64, 128, LA_F32, ws + L.bwd, L.bwd_bytes, s);
        if (st != LA_OK) return st;
        float* dvdst = static_cast<float*>(dv) + 64 * h;
        if ((e = timed("copy_cols", s, [&] { return la::launch_copy_cols(dvdst, 128, dvh, 64, BH * N, 64, s); })) !=
            hipSuccess)
            return hip_fail(e, "copy_cols launch");
    }
    const float* dfq0 = reinterpret_cast<const float*>(ws + L.dfq[0]);
    const float* dfq1 = reinterpret_cast<const float*>(ws + L.dfq[1]);
    const float* dfk0 = reinterpret_cast<const float*>(ws + L.dfk[0]);
    const float* dfk1 = reinterpret_cast<const float*>(ws + L.dfk[1]);
    if ((e = timed("phi_blocks_grad", s, [&] {
             return la::launch_phi_blocks_grad(fq_in, dfq0, dfq1, static_cast<float*>(dq), BH, N, 2, 64, s);
         })) != hipSuccess ||
        (e = timed("phi_blocks_grad", s, [&] {
             return la::launch_phi_blocks_grad(fk_in, dfk0, dfk1, static_cast<float*>(dk), BH, N, 2, 64, s);
         })) != hipSuccess)
        return hip_fail(e, "phi_blocks_grad launch");
    return LA_OK;
}
