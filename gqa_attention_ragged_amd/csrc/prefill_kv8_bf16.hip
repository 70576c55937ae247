// prefill_kv8_bf16.hip -- the prefill kernels for bf16 Q over an fp8 E4M3FN KV cache.
#include "prefill_impl.h"

namespace gqa {

hipError_t launch_prefill_kv8_bf16(const AttnParams& p, int head_dim, int grid_x, int grid_y,
                                 hipStream_t stream) {
    return head_dim == 64 ? launch_kv8_t<bf16, 64>(p, grid_x, grid_y, stream)
                          : launch_kv8_t<bf16, 128>(p, grid_x, grid_y, stream);
}

}  // namespace gqa
