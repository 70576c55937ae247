// prefill_persist.hip -- launcher of the persistent prefill kernel (16-bit
// Q/K/V, online softmax, no mask / tree / paging): the claim counters are
// zeroed, `workgroups` persistent workgroups run, and for split-KV calls
// the combine kernel merges the key slices.
#include "prefill_persist.h"

namespace gqa {

template <typename TI, int D>
static hipError_t launch_persist_t(const AttnParams& p, int workgroups, hipStream_t stream) {
    hipLaunchKernelGGL(prefill_sched_reset_kernel, dim3(1), dim3(kSchedInts), 0, stream, p.sched,
                       kSchedInts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    main_kernel_begin(stream);
    hipLaunchKernelGGL((prefill_persist_kernel<TI, D>), dim3(workgroups), dim3(256), 0, stream, p);
    main_kernel_end(stream);
    if (p.n_splits > 1) {
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((prefill_combine_kernel<TI, D>), dim3(p.grid_x, p.hq), dim3(256), 0,
                           stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_prefill_persist(const AttnParams& p, int elem, int head_dim, int workgroups,
                                  hipStream_t stream) {
    if (elem == ELEM_BF16)
        return head_dim == 64 ? launch_persist_t<bf16, 64>(p, workgroups, stream)
                              : launch_persist_t<bf16, 128>(p, workgroups, stream);
    return head_dim == 64 ? launch_persist_t<f16, 64>(p, workgroups, stream)
                          : launch_persist_t<f16, 128>(p, workgroups, stream);
}

}  // namespace gqa
