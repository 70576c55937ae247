// validate.hip -- the length-check kernel that GQA_ATTN_VALIDATE=1 runs before
// the attention kernels of a forward call (debug mode): one workgroup checks
// every sequence with the predicate of lengths.h and writes the OR of the
// violation bits to `status`.
#include "launch.h"
#include "lengths.h"

#include <atomic>

namespace gqa {

__global__ __launch_bounds__(256) void length_check_kernel(LenCheck c, uint32_t* status) {
    __shared__ uint32_t s_err;
    if (threadIdx.x == 0) s_err = 0u;
    __syncthreads();
    uint32_t e = 0u;
    for (int b = threadIdx.x; b < c.batch; b += blockDim.x) e |= check_sequence(c, b);
    if (e) atomicOr(&s_err, e);  // LDS atomic
    __syncthreads();
    // one vector store of the result, every call (nothing to clear first)
    if (threadIdx.x == 0) *status = s_err;
}

hipError_t launch_length_check(const LenCheck& c, uint32_t* status, hipStream_t stream) {
    hipLaunchKernelGGL(length_check_kernel, dim3(1), dim3(256), 0, stream, c, status);
    return hipGetLastError();
}

// The check's result word, one per device (each device holds its own copy of
// a __device__ variable); its address comes from hipGetSymbolAddress.
__device__ uint32_t g_length_status;

hipError_t length_status_ptr(uint32_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::atomic<uint32_t*> ptrs[256];
    if (dev < 0 || dev >= 256) return hipErrorInvalidDevice;
    uint32_t* p = ptrs[dev].load();
    if (!p) {
        e = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(g_length_status));
        if (e != hipSuccess) return e;
        ptrs[dev].store(p);  // every thread stores the same address
    }
    *out = p;
    return hipSuccess;
}

}  // namespace gqa
