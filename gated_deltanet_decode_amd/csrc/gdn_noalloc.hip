// gdn_noalloc.hip -- the device scratch of gdn_tree_verify_ut_noalloc, the
// tree verify for callers that cannot allocate (code under graph capture,
// serving loops that forbid hipMalloc, harnesses that refuse allocation).
//
// The scratch is a file-scope device array, so each GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// never passes the array's name to a kernel (on the host it names a stand-in,
// not device memory): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "gdn.h"
#include "gdn_launch.hpp"

namespace gdn {

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];   // device address of `scratch` per device, once looked up
}  // namespace

hipError_t noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace gdn
