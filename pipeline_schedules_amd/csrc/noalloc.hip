// Device memory for pps_stage_create_noalloc: one fixed array per GPU, for
// callers that cannot allocate (code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc).  A stage created that way takes its
// stash pool, scratch, gradients and weight copies from this array instead
// of hipMalloc.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up per device with hipGetSymbolAddress, once,
// with that device current, and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "pps.h"

namespace {

constexpr size_t kScratchBytes = (size_t)PPS_NOALLOC_MAX_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
char* g_ptr[kMaxDevices] = {};

}  // namespace

namespace pps {

// This device's copy of the array, or PPS_EHIP / PPS_EINVAL.
int noalloc_scratch(char** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return PPS_EHIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return PPS_EINVAL;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return PPS_EHIP;
        }
        g_ptr[dev] = static_cast<char*>(p);
    }
    *out = g_ptr[dev];
    return PPS_OK;
}

}  // namespace pps
