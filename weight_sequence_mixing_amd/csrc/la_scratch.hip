// la_scratch.hip -- the static device scratch of la_forward_causal_noalloc,
// for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array.  In host code its name is only a
// host-side stand-in, never a device address: the address on a device comes
// from hipGetSymbolAddress, called once per device with that device current
// and kept in a per-device table.  Every call on a device shares that
// device's array and finds the previous call's contents there; the forward
// writes every segment state before it reads it, so nothing needs clearing.
// Calls that overlap on one device race for it.
#include <mutex>
#include <vector>

#include "la_internal.h"

namespace la {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_ptr(void** out)
{
    static std::mutex mu;
    static std::vector<void*> ptrs;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if ((size_t)dev >= ptrs.size()) ptrs.resize((size_t)dev + 1, nullptr);
    if (!ptrs[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return hipSuccess;
}

}  // namespace la
