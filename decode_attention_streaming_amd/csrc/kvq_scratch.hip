// kvq_scratch.hip -- the library's one statically allocated device buffer:
// scratch space for the decode-attention hand-off (per-stream hand-off words
// and partial entries) used by kvq_decode_attention_noalloc(), for callers
// that cannot allocate device memory.  Each GPU holds its own copy of the
// array, at its own address, from the moment the code object is loaded until
// the process ends.
#include <mutex>

#include "kvq_internal.h"

namespace kvq {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];  // device address of each GPU's copy, once set up

}  // namespace

hipError_t static_scratch(int device, hipStream_t st, void **out)
{
    if (device < 0 || device >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[device]) {
        // the array's name is a host-side stand-in: its device address comes
        // from the runtime, for the current device
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        // arrival counters start at zero (each call re-arms the ones it uses)
        e = launch_zero(static_cast<unsigned *>(p), kStaticScratchStreams * kCounterStride, st);
        if (e != hipSuccess)
            return e;
        g_ptr[device] = p;
    }
    *out = g_ptr[device];
    return hipSuccess;
}

}  // namespace kvq
