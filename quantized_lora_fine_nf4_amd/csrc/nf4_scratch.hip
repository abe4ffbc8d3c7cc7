// nf4_scratch.hip -- the fixed device scratch of nf4_layer_error_noalloc.
//
// That entry point is for callers that cannot allocate device memory: it
// runs the fused pass with its workspace (the descriptor table and the
// per-tile fp64 error partials) in this file-scope device array instead of a
// caller buffer.  Each GPU the library runs on holds its own copy of the
// array, at its own address, until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in):
// its device address is looked up once per device with hipGetSymbolAddress,
// with that device current, and that address is what the kernels get.
#include <hip/hip_runtime.h>

#include <mutex>

#include "nf4_launch.h"

namespace {

static __device__ __align__(256) unsigned char scratch[nf4k::kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace nf4k {

hipError_t scratch_pointer(void** out)
{
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace nf4k
