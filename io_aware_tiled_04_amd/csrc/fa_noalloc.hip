// Allocation-free split-KV forward: the split partials go to a fixed device
// array of this file instead of a caller workspace.
//
// `scratch` is a file-scope device array.  In host code its name is only a
// host-side stand-in, never a device address: the device address of each
// GPU's copy comes from hipGetSymbolAddress, taken once per device (with
// that device current) on the first call there, and kept in `g_scratch`.
// Only that pointer is passed to the kernels.  Each GPU holds its copy of the
// array from then until the process ends, and every call on that GPU shares
// it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"
#include "fa_kernels.h"

namespace fa {
namespace {

static_assert(FA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) float scratch[FA_NOALLOC_SCRATCH_BYTES / 4];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

// Device address of the current device's scratch array (looked up once per
// device), or an error.
hipError_t noalloc_scratch(float** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = (float*)g_scratch[dev];
    return hipSuccess;
}

}  // namespace fa
