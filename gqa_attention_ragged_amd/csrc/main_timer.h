// main_timer.h -- optional event pair around the main attention kernel of a
// call (the prefill attention kernel, or the decode split kernel), for
// measuring that kernel's own duration.  Host code only; no-ops unless a
// timing window was opened with gqa_attn_timer_start.
#pragma once
#include <hip/hip_runtime.h>

namespace gqa {
void main_kernel_begin(hipStream_t stream);
void main_kernel_end(hipStream_t stream);
}  // namespace gqa
