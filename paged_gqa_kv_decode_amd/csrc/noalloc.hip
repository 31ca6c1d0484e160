// Library-held scratch for vk_paged_gqa_decode_noalloc: the split-KV partials
// live in one file-scope device array of VK_NOALLOC_SCRATCH_BYTES instead of
// caller buffers, so the call allocates nothing.  Each GPU the library runs on
// holds its own copy of the array until the process ends.
//
// In host code the array's name is only a host-side stand-in: its device
// address is looked up once per device (with that device current) and only
// that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "vk_constants.h"
#include "vk_kernels.h"

namespace {

static __device__ __align__(256) unsigned char scratch[VK_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace vk {

hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace vk
