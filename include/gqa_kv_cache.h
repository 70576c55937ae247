/*
 * gqa_kv_cache.h -- C ABI of the KV-cache update (gfx950), the step that
 * writes new keys / values into the cache before decode or chunked prefill.
 *
 * The operation is TRT_KVCacheUpdate as the onnx-tensorrt "TensorRT Custom
 * Operator Schemas" page defines it (attributes update_form, mode "linear",
 * axis -2; inputs past_cache, update, write_indices, update_lengths; output
 * Y): Y is past_cache with the update rows of every sequence written along
 * the sequence axis of the [B, H, N, D] cache.
 *
 * Conventions that the page leaves open (fixed here):
 *   - write_indices absent: every sequence writes from position 0;
 *   - update_lengths absent (padded update only): every sequence writes all
 *     N_u rows of its update; present (cumulative [B+1], starting at 0):
 *     sequence b writes L_b = update_lengths[b+1] - update_lengths[b] rows,
 *     the first L_b rows of update[b] (padded) or rows update_lengths[b] ..
 *     update_lengths[b+1]-1 of the packed update;
 *   - row t of sequence b goes to position write_indices[b] + t of every
 *     head; rows whose position falls outside [0, N) are dropped;
 *   - every other element of Y equals past_cache.  Y may be past_cache
 *     itself (same pointer and strides: the update runs in place and writes
 *     only the update rows); otherwise Y must not overlap past_cache or the
 *     update, and the whole cache is copied into it first.
 *
 * The copy is bit-exact for every element type (f16, bf16, fp8 E4M3FN).
 * Ownership, streams and errors as in gqa_attn.h: caller-owned device
 * buffers, no allocation, no synchronization, asynchronous launch on the
 * caller's stream, host-detectable errors returned before any launch.
 */
#ifndef GQA_KV_CACHE_H
#define GQA_KV_CACHE_H

#include "gqa_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* past_cache: [B, H, N, D]; dtype f16, bf16 or fp8 E4M3FN.
 * update: padded [B, H, N_u, D] or packed [T, H, D] (update_form), the
 *      cache's dtype, H and D.
 * out: Y, [B, H, N, D] of the cache's dtype (may be past_cache, see above).
 * write_indices: device int32 [B] or NULL.
 * update_lengths: device int32 [B+1] cumulative or NULL; required when the
 *      update is packed.
 * Tensor rules as in gqa_attn.h (D contiguous, 16-byte aligned base and
 * strides), and D times the element size a multiple of 16 bytes.
 * Device-side preconditions (not checked on the host): update_lengths
 * monotone from 0 with update_lengths[B] <= T (packed) and L_b <= N_u
 * (padded). */
typedef struct {
    gqa_tensor_t past_cache;
    gqa_tensor_t update;
    gqa_tensor_t out;
    const int32_t* write_indices;
    const int32_t* update_lengths;
    int32_t update_form; /* gqa_form_t */
} gqa_kv_update_args_t;

/* Check every host-visible property of args; launches nothing, touches no
 * device memory.  Returns a gqa_status_t. */
int gqa_kv_cache_update_validate(const gqa_kv_update_args_t* args);

/* Y = TRT_KVCacheUpdate(args) on `stream` (a hipStream_t; NULL = the null
 * stream).  Needs no workspace.  Returns GQA_OK once the kernels are
 * enqueued; gqa_attn_last_error / gqa_attn_last_hip_error describe a
 * failure. */
int gqa_kv_cache_update(const gqa_kv_update_args_t* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_KV_CACHE_H */
