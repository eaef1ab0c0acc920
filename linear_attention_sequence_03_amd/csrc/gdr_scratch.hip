// gdr_scratch.hip -- the fixed device scratch behind gdr_chunk_fwd_noalloc.
//
// One file-scope device array per GPU holds the chunk workspace (the per-chunk
// WY factors that the preparation kernels write and the state pass reads) for
// callers that cannot allocate device memory.  The runtime gives each device
// its own copy of the array when the library's code object is loaded there;
// its device address is looked up once per device, with that device current,
// and kept.  Host code never uses the array's name as an address: on the host
// it only names the symbol.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdr.h"
#include "gdr_launch.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace gdr {

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
    *out = nullptr;
    hipDevice_t dev = 0;
    hipError_t err = hipStreamGetDevice(stream, &dev);   // the null stream: the current device
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        int cur = 0;
        err = hipGetDevice(&cur);
        if (err != hipSuccess) return err;
        if (cur != dev && (err = hipSetDevice(dev)) != hipSuccess) return err;
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (err != hipSuccess) return err;
        if (back != hipSuccess) return back;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace gdr
