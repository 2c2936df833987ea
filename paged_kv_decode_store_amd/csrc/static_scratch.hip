// A fixed device buffer for callers that cannot allocate (code under graph
// capture, tight serving loops, harnesses that forbid allocation): the
// split-KV partials of the no-allocation attention entry point live here
// instead of in a caller-provided workspace.
//
// The array is a file-scope device variable, so each GPU the library runs
// on holds its own copy until the process ends.  In host code its name is
// only a stand-in: the device address is resolved once per device, with
// that device current, through hipGetSymbolAddress, and every use (kernel
// arguments, copies) goes through the resolved pointer.  All calls on one
// GPU share that GPU's copy.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"
#include "pkv.h"

namespace pkv {

namespace {

static __device__ __align__(256) unsigned char scratch[PKV_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace pkv
