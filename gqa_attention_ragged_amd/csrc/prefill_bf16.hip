// prefill_bf16.hip -- the general prefill kernels for bf16 Q/K/V.
#include "prefill_impl.h"

namespace gqa {

hipError_t launch_prefill_bf16(const AttnParams& p, int head_dim, int grid_x, int grid_y,
                              hipStream_t stream) {
    return head_dim == 64 ? launch_t<bf16, 64>(p, grid_x, grid_y, stream)
                          : launch_t<bf16, 128>(p, grid_x, grid_y, stream);
}

}  // namespace gqa
