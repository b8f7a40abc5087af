// scratch.hip - device memory of the allocation-free decode entry point
// (attn_decode_splitk_noalloc): a fixed array in the library's code object,
// one copy per GPU, held until the process ends.
//
// Host code never uses the array's name as a device address (in host code it
// names a host-side stand-in): the address of each GPU's copy comes from
// hipGetSymbolAddress, called once per device with that device current, and
// is cached per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gqa_kernels.hpp"

namespace gqa {

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device: its copy of `scratch`, or null until first use

}  // namespace

size_t scratch_capacity_bytes() { return kScratchBytes; }

hipError_t scratch_device_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace gqa
