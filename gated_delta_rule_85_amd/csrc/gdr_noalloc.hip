// gdr_fwd_noalloc: the forward without a caller workspace, for callers that
// cannot allocate device memory (include/gdr.h).  Its scratch is the static
// device array below, one per GPU, held until the process ends.
//
// In host code `scratch` names a host-side stand-in of the device array, not
// a device address: its device address is looked up once per device, with
// that device current, by hipGetSymbolAddress, and only that address is ever
// handed to kernels.  This file holds no kernels, so the array is placed on
// a GPU only when that lookup loads this file's code object there.
#include <mutex>

#include "gdr.h"
#include "gdr_kernels.hpp"

namespace {

__device__ __align__(256) char scratch[GDR_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void *scratch_ptr[MAX_DEVICES];  // device address of `scratch` on each device, once looked up

// device address of this device's scratch array; null if it cannot be had
void *scratch_for(int dev) {
    if (dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return nullptr;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) return nullptr;
        scratch_ptr[dev] = p;
    }
    return scratch_ptr[dev];
}

}  // namespace

extern "C" int gdr_fwd_noalloc(const gdr_fwd_args *a, hipStream_t stream) {
    return gdr::fwd_impl(a, stream, scratch_for, GDR_SCRATCH_BYTES);
}
