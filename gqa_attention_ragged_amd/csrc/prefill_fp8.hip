// prefill_fp8.hip -- the general prefill kernels for fp8 Q/K/V.
#include "prefill_impl.h"

namespace gqa {

hipError_t launch_prefill_fp8(const AttnParams& p, int head_dim, int grid_x, int grid_y,
                              hipStream_t stream) {
    return head_dim == 64 ? launch_t<fp8, 64>(p, grid_x, grid_y, stream)
                          : launch_t<fp8, 128>(p, grid_x, grid_y, stream);
}

}  // namespace gqa
