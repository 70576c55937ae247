// static_scratch.hip -- the fixed device workspace of gqa_attn_forward_noalloc:
// a file-scope device array that the split-KV partials of a call live in,
// for callers that cannot allocate device memory (HIP graph capture, serving
// loops, harnesses that forbid allocation).
//
// Each device the library runs on holds its own copy of the array (allocated
// when the code object loads, held until the process ends).  Host code never
// passes the array's name to a kernel: in host code the name is a host-side
// stand-in, not a device address.  The device address of this device's copy
// comes from hipGetSymbolAddress, once per device, with that device current.
#include "launch.h"

#include <atomic>

namespace gqa {

static __device__ __align__(256) char scratch[kStaticScratchBytes];

hipError_t static_scratch_ptr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::atomic<void*> ptrs[256];
    if (dev < 0 || dev >= 256) return hipErrorInvalidDevice;
    void* p = ptrs[dev].load();
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        ptrs[dev].store(p);  // every thread stores the same address
    }
    *out = p;
    return hipSuccess;
}

}  // namespace gqa
