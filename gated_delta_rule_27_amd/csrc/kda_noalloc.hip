// kda_noalloc.hip -- the device-resident scratch of kda_chunk_bwd_noalloc.
//
// The backward pass keeps two per-chunk tables (states and state gradients)
// in a workspace.  Callers that cannot allocate get them from `scratch`, a
// static device array of KDA_BWD_NOALLOC_MAX_BYTES: each GPU the library
// runs on holds its own copy from the code object's load until the process
// ends.  In host code `scratch` names a host-side stand-in, not device
// memory, so its address is looked up with hipGetSymbolAddress once per
// device (with that device current) and only that address is ever handed
// to kernels.  Nothing here allocates.
#include <mutex>

#include "kda.h"
#include "kda_launch.h"

namespace kda {

namespace {

static __device__ __align__(256) unsigned char scratch[KDA_BWD_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace kda
