// noalloc.hip -- la_forward_causal_noalloc: the causal forward with its workspace in a
// static device array, for callers that cannot allocate device memory (code under
// stream capture into a HIP graph, tight serving loops, harnesses that forbid
// hipMalloc).  The array is a file-scope __device__ object of the library's code
// object: each GPU the library runs on holds its own copy, at its own address, for
// the life of the process.  Host code never passes the array's name to a kernel
// (on the host it is only a stand-in); it asks the runtime once per device for the
// device address and passes that.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "linattn.h"

namespace la {
la_status forward_causal_on(const void* q, const void* k, const void* v, void* o, const float* S0, const float* z0,
                            float* den_out, float* S_out, float* z_out, int64_t B, int64_t H, int64_t N, int64_t d,
                            int chunk, la_dtype dt, void* workspace, size_t workspace_bytes, void* stream);
la_status fail_status(la_status s, const char* msg);
}  // namespace la

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // the array's device address, per device

// The device address of `scratch` on the current device (looked up on the first call there).
la_status scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return la::fail_status(LA_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return la::fail_status(LA_ERR_UNSUPPORTED, "device index beyond 64");
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return la::fail_status(LA_ERR_HIP, "hipGetSymbolAddress of the static scratch array failed");
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return LA_OK;
}

}  // namespace

extern "C" {

la_status la_forward_causal_noalloc(const void* q, const void* k, const void* v, void* o, const float* S0,
                                    const float* z0, float* den_out, float* S_out, float* z_out, int64_t B, int64_t H,
                                    int64_t N, int64_t d, int chunk, la_dtype dt, void* stream) {
    size_t need = 0;
    la_status st = la_workspace_size(LA_OP_FWD_CAUSAL, B, H, N, d, chunk, dt, &need);
    if (st != LA_OK) return st;
    if (need > kScratchBytes)
        return la::fail_status(LA_ERR_WORKSPACE,
                               "this shape needs more workspace than the 64 MiB static scratch array holds; "
                               "call la_forward_causal with a workspace instead");
    void* ws = nullptr;
    if (need > 0 && (st = scratch_on_current_device(&ws)) != LA_OK) return st;
    return la::forward_causal_on(q, k, v, o, S0, z0, den_out, S_out, z_out, B, H, N, d, chunk, dt, ws, need, stream);
}

}  // extern "C"
