// prefill.hip -- launcher of the general prefill kernel (the kernels are
// templates in prefill_impl.h, instantiated per element type in
// prefill_f16.hip, prefill_bf16.hip and prefill_fp8.hip, and for 16-bit Q over
// an fp8 KV cache in prefill_kv8_{f16,bf16}.hip, so that they compile in
// parallel; each launches its split-KV combine itself).
#include "launch.h"

namespace gqa {

hipError_t launch_prefill(const AttnParams& p, int elem, int head_dim, int grid_x, int grid_y,
                          hipStream_t stream) {
    if (p.kv8)
        return elem == ELEM_BF16 ? launch_prefill_kv8_bf16(p, head_dim, grid_x, grid_y, stream)
                                 : launch_prefill_kv8_f16(p, head_dim, grid_x, grid_y, stream);
    if (elem == ELEM_F16) return launch_prefill_f16(p, head_dim, grid_x, grid_y, stream);
    if (elem == ELEM_BF16) return launch_prefill_bf16(p, head_dim, grid_x, grid_y, stream);
    return launch_prefill_fp8(p, head_dim, grid_x, grid_y, stream);
}

}  // namespace gqa
