// The backward over views for callers that cannot allocate (code under
// graph capture, tight serving loops, harnesses that forbid allocation):
// rmsnorm_bwd_strided_noalloc runs rmsnorm_bwd_strided with its workspace
// taken from a fixed device array instead of the caller.
//
// The array holds the deterministic route's dw partial rows ([P, H], FP32 or
// FP64); its size is the largest workspace any default route asks for (P =
// 256 row blocks of H 8192 or 16384 FP64 sums: 32 MiB). A problem that would
// need more (only reachable through a tuning override) is refused before
// anything is enqueued. Each device that runs the entry point holds its own
// copy until the process ends; its address is looked up once per device,
// with that device current, and only that address is handed to the kernels
// (the array's name denotes a host-side stand-in in host code). Calls share
// the array: two calls that overlap on one device race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "rmsn_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (null on failure).
void* scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" int rmsnorm_bwd_strided_noalloc(const void* dy, rmsn_view_t dyv, const void* x,
                                           rmsn_view_t xv, const float* rstd, const void* w,
                                           rmsn_dtype_t w_dtype, int deterministic, void* dx,
                                           rmsn_view_t dxv, float* dw, hipStream_t stream) {
    int64_t rows = 0;
    if (xv.T >= 0 && xv.heads >= 1 && !__builtin_mul_overflow(xv.T, xv.heads, &rows) && rows > 0) {
        rmsn::Route rt;
        if (rmsn::route(1, rows, xv.H, w_dtype, deterministic, rmsn::kFormPlain, &rt) == RMSN_OK &&
            rt.workspace > kScratchBytes)
            return RMSN_ERR_SCRATCH;
    }
    void* ws = scratch_address();
    if (!ws) return RMSN_ERR_SCRATCH;
    return rmsnorm_bwd_strided(dy, dyv, x, xv, rstd, w, w_dtype, deterministic, dx, dxv, dw, ws,
                               kScratchBytes, stream);
}
