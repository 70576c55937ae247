// prefill_pp.hip -- launcher of the ping-pong prefill kernel (16-bit Q/K/V,
// online softmax, no mask) and, for split-KV calls, of its combine kernel.
#include "prefill_pp.h"

namespace gqa {

template <typename TI, int D>
static hipError_t launch_pp_t(const AttnParams& p, int grid_x, int grid_y, hipStream_t stream) {
    const dim3 grid(grid_x, grid_y, p.n_splits > 1 ? p.n_splits : 1);
    main_kernel_begin(stream);
    hipLaunchKernelGGL((prefill_pp_kernel<TI, D>), grid, dim3(512), 0, stream, p);
    main_kernel_end(stream);
    if (p.n_splits > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((prefill_combine_kernel<TI, D>), dim3(grid_x, p.hq), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_prefill_pp(const AttnParams& p, int elem, int head_dim, int grid_x, int grid_y,
                             hipStream_t stream) {
    if (elem == ELEM_BF16)
        return head_dim == 64 ? launch_pp_t<bf16, 64>(p, grid_x, grid_y, stream)
                              : launch_pp_t<bf16, 128>(p, grid_x, grid_y, stream);
    return head_dim == 64 ? launch_pp_t<f16, 64>(p, grid_x, grid_y, stream)
                          : launch_pp_t<f16, 128>(p, grid_x, grid_y, stream);
}

}  // namespace gqa
