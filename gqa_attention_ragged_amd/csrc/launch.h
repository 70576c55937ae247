// launch.h -- host-side entry points of the attention kernels (internal).
#pragma once
#include <hip/hip_runtime.h>

#include "device_common.h"

namespace gqa {

enum Elem { ELEM_F16 = 0, ELEM_BF16 = 1, ELEM_FP8 = 2 };

// Prefill / general kernel.  grid_x = number of query-row tiles (upper bound
// over the ragged batch), grid_y = H_q / heads_per_wg.  elem: Q/K/V type.
hipError_t launch_prefill(const AttnParams& p, int elem, int head_dim, int grid_x, int grid_y,
                          hipStream_t stream);

// Software-pipelined prefill for 16-bit Q/K/V, softmax, no Q/DQ, no mask,
// score scale > 0: `waves` (4 or 8) row groups of 32 rows per workgroup,
// heads_per_wg = gcd(G, waves), rows_per_wg = 32 * waves / heads_per_wg.  The
// split-KV combine (when n_splits > 1) is launched by launch_prefill_combine.
hipError_t launch_prefill_pipe(const AttnParams& p, int elem, int head_dim, int waves, int grid_x,
                               int grid_y, hipStream_t stream);
hipError_t launch_prefill_combine(const AttnParams& p, int elem, int head_dim, int grid_x,
                                  hipStream_t stream);

// The general prefill kernels of one element type (launch_prefill's parts).
hipError_t launch_prefill_f16(const AttnParams& p, int head_dim, int grid_x, int grid_y,
                              hipStream_t stream);
hipError_t launch_prefill_bf16(const AttnParams& p, int head_dim, int grid_x, int grid_y,
                               hipStream_t stream);
hipError_t launch_prefill_fp8(const AttnParams& p, int head_dim, int grid_x, int grid_y,
                              hipStream_t stream);

// Decode (query length 1) split-KV partial pass and its combine.
// q_elem: Q type (f16/bf16); kv_elem: K/V type (same as q, or fp8).
hipError_t launch_decode(const AttnParams& p, int q_elem, int kv_elem, int head_dim,
                         hipStream_t stream);

}  // namespace gqa
