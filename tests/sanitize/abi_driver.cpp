// abi_driver.cpp -- the host half of the C ABI (csrc/api.cpp: argument validation,
// size arithmetic, workspace layout, kernel sequencing) under AddressSanitizer and
// UndefinedBehaviorSanitizer, with every kernel launcher replaced by a stub that only
// counts calls (tests/test_sanitize.py generates the stubs from csrc/launch.h), so no
// GPU is needed.  Pointers are fake device addresses, which host code never
// dereferences.  Each case checks the documented status, and whether anything would
// have been launched.  Exit status 0: every case as expected, no sanitizer report.
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "linattn.h"

extern int g_stub_launches;  // defined by the generated stubs

namespace {

int g_bad = 0;
void* P(uint64_t a) { return reinterpret_cast<void*>(static_cast<uintptr_t>(a)); }
float* F(uint64_t a) { return reinterpret_cast<float*>(static_cast<uintptr_t>(a)); }
constexpr uint64_t A = 0x10000000ull, GB = 1ull << 30;

// Runs call(), checks its status and that it launched something iff `launches`.
template <class F_>
void check(const char* what, la_status want, bool launches, F_ call) {
    const int before = g_stub_launches;
    const la_status got = call();
    if (got != want) {
        std::fprintf(stderr, "FAIL %s: status %d, want %d (%s)\n", what, (int)got, (int)want, la_last_error_message());
        g_bad = 1;
    }
    const bool did = g_stub_launches != before;
    if (did != launches) {
        std::fprintf(stderr, "FAIL %s: launches %d -> %d (expected %s)\n", what, before, g_stub_launches,
                     launches ? "some" : "none");
        g_bad = 1;
    }
}

size_t ws(la_op op, int64_t B, int64_t H, int64_t N, int64_t d, la_dtype dt = LA_BF16, int chunk = 0) {
    size_t n = 0;
    const la_status s = la_workspace_size(op, B, H, N, d, chunk, dt, &n);
    return s == LA_OK ? n : (size_t)-1;
}

// Sequence tensors far apart: q, k, v, o / dout, then outputs, then the workspace.
struct Seq {
    uint64_t q = A, k = A + 4 * GB, v = A + 8 * GB, o = A + 12 * GB, dout = A + 16 * GB, dq = A + 20 * GB,
             dk = A + 24 * GB, dv = A + 28 * GB, w = A + 32 * GB, st = A + 40 * GB, aux = A + 44 * GB;
};

}  // namespace

int main() {
    const Seq s;
    // ---- workspace sizes over many shapes: alignment, zero-token shapes, limits near 2^31 ----
    const int64_t Bs[] = {1, 3, 64}, Hs[] = {1, 16, 1024}, Ns[] = {0, 1, 63, 64, 65, 4096, 131072, 1 << 22};
    const int64_t ds[] = {32, 64, 128};
    const la_op ops[] = {LA_OP_FWD_NONCAUSAL, LA_OP_FWD_CAUSAL, LA_OP_BWD_CAUSAL, LA_OP_BWD_NONCAUSAL};
    for (la_op op : ops)
        for (int64_t B : Bs)
            for (int64_t H : Hs)
                for (int64_t N : Ns)
                    for (int64_t d : ds)
                        for (la_dtype dt : {LA_BF16, LA_F32}) {
                            const size_t n = ws(op, B, H, N, d, dt);
                            if (n == (size_t)-1) continue;  // a shape beyond a documented limit
                            if (n % 256 != 0 || (N == 0 && n != 0)) {
                                std::fprintf(stderr, "FAIL workspace %d %lld %lld %lld %lld: %zu\n", (int)op,
                                             (long long)B, (long long)H, (long long)N, (long long)d, n);
                                g_bad = 1;
                            }
                        }
    size_t tmp = 0;
    check("workspace: d unsupported", LA_ERR_UNSUPPORTED, false,
          [&] { return la_workspace_size(LA_OP_FWD_CAUSAL, 1, 1, 64, 48, 0, LA_BF16, &tmp); });
    check("workspace: negative", LA_ERR_INVALID_ARGUMENT, false,
          [&] { return la_workspace_size(LA_OP_FWD_CAUSAL, -1, 1, 64, 64, 0, LA_BF16, &tmp); });
    check("workspace: N beyond 2^30", LA_ERR_UNSUPPORTED, false,
          [&] { return la_workspace_size(LA_OP_FWD_CAUSAL, 1, 1, (int64_t)1 << 31, 64, 0, LA_BF16, &tmp); });
    check("workspace: head beyond 2^31 bytes", LA_ERR_UNSUPPORTED, false,
          [&] { return la_workspace_size(LA_OP_FWD_CAUSAL, 1, 1, (int64_t)1 << 24, 128, 0, LA_F32, &tmp); });
    check("workspace: B*H beyond 2^31", LA_ERR_UNSUPPORTED, false,
          [&] { return la_workspace_size(LA_OP_FWD_CAUSAL, (int64_t)1 << 20, (int64_t)1 << 12, 64, 64, 0, LA_BF16, &tmp); });
    check("workspace: NULL out", LA_ERR_INVALID_ARGUMENT, false,
          [&] { return la_workspace_size(LA_OP_FWD_CAUSAL, 1, 1, 64, 64, 0, LA_BF16, nullptr); });
    check("saved state size", LA_OK, false, [&] { return la_saved_state_size(4, 16, 4096, 64, 0, LA_BF16, &tmp); });

    // ---- causal forward ----
    const size_t wf = ws(LA_OP_FWD_CAUSAL, 4, 16, 4096, 64);
    auto fwd = [&](int64_t B, int64_t H, int64_t N, int64_t d, uint64_t q, uint64_t o, uint64_t w, size_t wb,
                   la_dtype dt = LA_BF16, const float* S0 = nullptr, float* S_out = nullptr, float* z_out = nullptr) {
        return la_forward_causal(P(q), P(s.k), P(s.v), P(o), S0, nullptr, nullptr, S_out, z_out, nullptr, 0, B, H, N,
                                 d, 0, dt, P(w), wb, nullptr);
    };
    check("fwd: valid Mid", LA_OK, true, [&] { return fwd(4, 16, 4096, 64, s.q, s.o, s.w, wf); });
    check("fwd: NULL q", LA_ERR_INVALID_ARGUMENT, false, [&] { return fwd(4, 16, 4096, 64, 0, s.o, s.w, wf); });
    check("fwd: misaligned o", LA_ERR_INVALID_ARGUMENT, false, [&] { return fwd(4, 16, 4096, 64, s.q, s.o + 2, s.w, wf); });
    check("fwd: o overlaps q", LA_ERR_INVALID_ARGUMENT, false, [&] { return fwd(4, 16, 4096, 64, s.q, s.q + 64, s.w, wf); });
    check("fwd: workspace short", LA_ERR_WORKSPACE, false, [&] { return fwd(4, 16, 4096, 64, s.q, s.o, s.w, wf - 256); });
    check("fwd: workspace overlaps v", LA_ERR_INVALID_ARGUMENT, false,
          [&] { return fwd(4, 16, 4096, 64, s.q, s.o, s.v + 256, wf); });
    check("fwd: no tokens", LA_OK, false, [&] { return fwd(4, 16, 0, 64, 0, 0, 0, 0); });
    check("fwd: fp32 d=128 (feature blocks)", LA_OK, true, [&] { return fwd(1, 1, 64, 128, s.q, s.o, s.w, GB, LA_F32); });
    check("fwd: fp32 d=128 workspace short", LA_ERR_WORKSPACE, false,
          [&] { return fwd(1, 1, 64, 128, s.q, s.o, s.w, ws(LA_OP_FWD_CAUSAL, 1, 1, 64, 128, LA_F32) - 256, LA_F32); });
    const size_t wv = ws(LA_OP_FWD_CAUSAL, 1, 32, 131072, 128);
    check("fwd: valid Very long (one round of 8 segments per head)", LA_OK, true,
          [&] { return fwd(1, 32, 131072, 128, s.q, s.o, s.w, wv); });
    const size_t wsc = ws(LA_OP_FWD_CAUSAL, 1, 4, 1 << 20, 128);
    check("fwd: valid B1 H4 N2^20 d128 (scan plan)", LA_OK, true,
          [&] { return fwd(1, 4, 1 << 20, 128, s.q, s.o, s.w, wsc); });
    const int64_t nmax = ((int64_t)1 << 31) / (128 * 2) - 64 - 1;
    check("fwd: longest head d=128", LA_OK, true,
          [&] { return fwd(1, 1, nmax, 128, s.q, s.o, s.w, ws(LA_OP_FWD_CAUSAL, 1, 1, nmax, 128)); });
    check("fwd: start state in place", LA_OK, true, [&] {
        return fwd(2, 3, 1000, 64, s.q, s.o, s.w, GB, LA_BF16, F(s.st), F(s.st), F(s.st + GB / 2));
    });

    // ---- causal backward (fused plan, scan plan, d = 128), state variant ----
    auto bwd = [&](int64_t B, int64_t H, int64_t N, int64_t d, uint64_t dq, size_t wb) {
        return la_backward_causal(P(s.q), P(s.k), P(s.v), P(s.dout), P(dq), P(s.dk), P(s.dv), nullptr, 0, B, H, N, d,
                                  0, LA_BF16, P(s.w), wb, nullptr);
    };
    check("bwd: valid Mid (fused)", LA_OK, true, [&] { return bwd(4, 16, 4096, 64, s.dq, ws(LA_OP_BWD_CAUSAL, 4, 16, 4096, 64)); });
    check("bwd: valid Long (d = 128)", LA_OK, true,
          [&] { return bwd(8, 16, 16384, 128, s.dq, ws(LA_OP_BWD_CAUSAL, 8, 16, 16384, 128)); });
    check("bwd: valid scan plan", LA_OK, true,
          [&] { return bwd(1, 2, 65536, 64, s.dq, ws(LA_OP_BWD_CAUSAL, 1, 2, 65536, 64)); });
    check("bwd: dq overlaps dk", LA_ERR_INVALID_ARGUMENT, false,
          [&] { return bwd(4, 16, 4096, 64, s.dk, ws(LA_OP_BWD_CAUSAL, 4, 16, 4096, 64)); });
    check("bwd: workspace short", LA_ERR_WORKSPACE, false, [&] { return bwd(4, 16, 4096, 64, s.dq, 1024); });
    auto bwd32 = [&](int64_t N, size_t wb) {
        return la_backward_causal(P(s.q), P(s.k), P(s.v), P(s.dout), P(s.dq), P(s.dk), P(s.dv), nullptr, 0, 2, 3, N,
                                  128, 0, LA_F32, P(s.w), wb, nullptr);
    };
    check("bwd: fp32 d=128 (feature blocks)", LA_OK, true,
          [&] { return bwd32(1000, ws(LA_OP_BWD_CAUSAL, 2, 3, 1000, 128, LA_F32)); });
    check("bwd: fp32 d=128 workspace short", LA_ERR_WORKSPACE, false,
          [&] { return bwd32(1000, ws(LA_OP_BWD_CAUSAL, 2, 3, 1000, 128, LA_F32) - 256); });
    check("bwd state: valid", LA_OK, true, [&] {
        return la_backward_causal_state(P(s.q), P(s.k), P(s.v), P(s.dout), F(s.st), F(s.st + GB / 4),
                                        F(s.st + GB / 2), F(s.st + 3 * GB / 4), P(s.dq), P(s.dk), P(s.dv), F(s.aux),
                                        F(s.aux + GB / 2), 2, 3, 1000, 64, 0, LA_BF16, P(s.w), GB, nullptr);
    });
    int64_t fails = -1;
    check("wait failures: NULL out", LA_ERR_INVALID_ARGUMENT, false,
          [&] { return la_wait_failures(LA_OP_BWD_CAUSAL, P(s.w), GB, 4, 16, 4096, 64, LA_BF16, nullptr, nullptr); });
    check("wait failures: an op without waits", LA_ERR_INVALID_ARGUMENT, false,
          [&] { return la_wait_failures(LA_OP_FWD_NONCAUSAL, P(s.w), GB, 4, 16, 4096, 64, LA_BF16, nullptr, &fails); });
    check("wait failures: separate sweeps (d = 128)", LA_OK, false, [&] {
        return la_wait_failures(LA_OP_BWD_CAUSAL, P(s.w), GB, 8, 16, 16384, 128, LA_BF16, nullptr, &fails);
    });
    if (fails != 0) { std::fprintf(stderr, "FAIL wait failures of a non-fused plan: %lld\n", (long long)fails); g_bad = 1; }

    // ---- non-causal forward and backward ----
    check("noncausal fwd: valid", LA_OK, true, [&] {
        return la_forward_noncausal(P(s.q), P(s.k), P(s.v), P(s.o), nullptr, 0, 4, 16, 4096, 64, LA_BF16, P(s.w),
                                    ws(LA_OP_FWD_NONCAUSAL, 4, 16, 4096, 64), nullptr);
    });
    check("noncausal bwd: valid", LA_OK, true, [&] {
        return la_backward_noncausal(P(s.q), P(s.k), P(s.v), P(s.dout), P(s.dq), P(s.dk), P(s.dv), nullptr, 0, 4, 16,
                                     4096, 64, LA_BF16, P(s.w), ws(LA_OP_BWD_NONCAUSAL, 4, 16, 4096, 64), nullptr);
    });
    check("noncausal bwd: fp32 d=128 (feature blocks)", LA_OK, true, [&] {
        return la_backward_noncausal(P(s.q), P(s.k), P(s.v), P(s.dout), P(s.dq), P(s.dk), P(s.dv), nullptr, 0, 2, 3,
                                     1000, 128, LA_F32, P(s.w), ws(LA_OP_BWD_NONCAUSAL, 2, 3, 1000, 128, LA_F32),
                                     nullptr);
    });
    check("noncausal bwd: fp32 d=128 workspace short", LA_ERR_WORKSPACE, false, [&] {
        return la_backward_noncausal(P(s.q), P(s.k), P(s.v), P(s.dout), P(s.dq), P(s.dk), P(s.dv), nullptr, 0, 2, 3,
                                     1000, 128, LA_F32, P(s.w), ws(LA_OP_BWD_NONCAUSAL, 2, 3, 1000, 128, LA_F32) - 256,
                                     nullptr);
    });
    check("noncausal bwd: dtype unknown", LA_ERR_UNSUPPORTED, false, [&] {
        return la_backward_noncausal(P(s.q), P(s.k), P(s.v), P(s.dout), P(s.dq), P(s.dk), P(s.dv), nullptr, 0, 4, 16,
                                     4096, 64, (la_dtype)7, P(s.w), GB, nullptr);
    });

    // ---- decode ----
    check("decode: valid", LA_OK, true, [&] {
        return la_decode_step(F(s.st), F(s.st + GB), P(s.q), P(s.k), P(s.v), P(s.o), 256, 32, 128, LA_BF16, nullptr);
    });
    check("decode: q overlaps S", LA_ERR_INVALID_ARGUMENT, false, [&] {
        return la_decode_step(F(s.st), F(s.st + GB), P(s.st + 64), P(s.k), P(s.v), P(s.o), 256, 32, 128, LA_BF16,
                              nullptr);
    });
    check("decode steps: grouped", LA_OK, true, [&] {
        return la_decode_steps(F(s.st), F(s.st + GB), P(s.q), P(s.k), P(s.v), P(s.o), 4, 32, 4, 16, 128, LA_BF16,
                               nullptr);
    });
    check("decode steps: H not a multiple of Hkv", LA_ERR_INVALID_ARGUMENT, false, [&] {
        return la_decode_steps(F(s.st), F(s.st + GB), P(s.q), P(s.k), P(s.v), P(s.o), 4, 30, 4, 16, 128, LA_BF16,
                               nullptr);
    });

    // ---- FAVOR+ features and the calls on them ----
    check("favor features: valid", LA_OK, true,
          [&] { return la_favor_features(P(s.q), F(s.st), P(s.o), 4 * 16 * 4096, 64, LA_BF16, nullptr); });
    check("favor features: NULL omega", LA_ERR_INVALID_ARGUMENT, false,
          [&] { return la_favor_features(P(s.q), nullptr, P(s.o), 4096, 64, LA_BF16, nullptr); });
    size_t wfb = 0;
    check("features workspace (m = 2d)", LA_OK, false,
          [&] { return la_features_workspace_size(1, 4, 16, 4096, 64, 128, LA_BF16, &wfb); });
    check("features blocks fwd: valid", LA_OK, true, [&] {
        return la_forward_causal_features_blocks(P(s.q), P(s.k), P(s.v), P(s.o), nullptr, nullptr, F(s.aux), nullptr,
                                                 nullptr, 4, 16, 4096, 64, 128, LA_BF16, P(s.w), wfb, nullptr);
    });
    check("features blocks fwd: m not a multiple of d", LA_ERR_INVALID_ARGUMENT, false, [&] {
        return la_forward_causal_features_blocks(P(s.q), P(s.k), P(s.v), P(s.o), nullptr, nullptr, nullptr, nullptr,
                                                 nullptr, 4, 16, 4096, 64, 100, LA_BF16, P(s.w), wfb, nullptr);
    });
    check("features blocks bwd: valid", LA_OK, true, [&] {
        size_t wb = 0;
        la_features_workspace_size(3, 4, 16, 4096, 64, 128, LA_BF16, &wb);
        return la_backward_causal_features_blocks(P(s.q), P(s.k), P(s.v), P(s.dout), F(s.aux), P(s.o), P(s.dq),
                                                  P(s.dk), P(s.dv), 4, 16, 4096, 64, 128, LA_BF16, P(s.w), wb, nullptr);
    });
    check("grouped prefill: valid", LA_OK, true, [&] {
        return la_forward_causal_grouped(P(s.q), P(s.k), P(s.v), P(s.o), nullptr, nullptr, nullptr, nullptr, nullptr,
                                         2, 32, 4, 8337, 64, 0, LA_BF16, P(s.w), GB, nullptr);
    });

    if (g_bad) return 1;
    std::printf("abi driver: all cases as documented (%d stub launches)\n", g_stub_launches);
    return 0;
}
