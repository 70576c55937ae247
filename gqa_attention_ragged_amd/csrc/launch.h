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

// Per-workgroup records of a prefill launch (AttnParams::wrec, kWorkRecInts
// ints each) for the n_wg = grid_x * grid_y * max(n_splits, 1) workgroups of
// launch_prefill's grid; p.batch <= 64.
hipError_t launch_prefill_plan(const AttnParams& p, int32_t* rec, int n_wg, hipStream_t stream);

// The 8-wave ping-pong prefill kernel (16-bit Q/K/V, online softmax, no
// mask; grid_x row tiles of rows_per_wg rows) and its split-KV combine.
hipError_t launch_prefill_pp(const AttnParams& p, int elem, int head_dim, int grid_x, int grid_y,
                             hipStream_t stream);
// Persistent prefill (16-bit, online softmax, no mask / tree / paging):
// zeroes p.sched (kSchedInts ints), then runs `workgroups` workgroups over
// the grid_x x grid_y x n_splits work items of p.
constexpr int kSchedInts = 8 * 16;
hipError_t launch_prefill_persist(const AttnParams& p, int elem, int head_dim, int workgroups,
                                  hipStream_t stream);

// The general prefill kernels of one element type (launch_prefill's parts).
hipError_t launch_prefill_f16(const AttnParams& p, int head_dim, int grid_x, int grid_y,
                              hipStream_t stream);
hipError_t launch_prefill_bf16(const AttnParams& p, int head_dim, int grid_x, int grid_y,
                               hipStream_t stream);
hipError_t launch_prefill_fp8(const AttnParams& p, int head_dim, int grid_x, int grid_y,
                              hipStream_t stream);
// 16-bit Q over an fp8 KV cache (p.kv8)
hipError_t launch_prefill_kv8_f16(const AttnParams& p, int head_dim, int grid_x, int grid_y,
                                  hipStream_t stream);
hipError_t launch_prefill_kv8_bf16(const AttnParams& p, int head_dim, int grid_x, int grid_y,
                                   hipStream_t stream);

// Decode (query length 1) split-KV partial pass and its combine.
// q_elem: Q type (f16/bf16); kv_elem: K/V type (same as q, or fp8).
hipError_t launch_decode(const AttnParams& p, int q_elem, int kv_elem, int head_dim,
                         hipStream_t stream);

// Length-check kernel (GQA_ATTN_VALIDATE=1): writes the OR of the
// violation bits of every sequence (lengths.h) to *status.
struct LenCheck;
hipError_t launch_length_check(const LenCheck& c, uint32_t* status, hipStream_t stream);
// Device address of this device's status word for the length check.
hipError_t length_status_ptr(uint32_t** out);

// The fixed device workspace of gqa_attn_forward_noalloc: 128 MiB per
// device (static_scratch.hip), and this device's address of it.
constexpr size_t kStaticScratchBytes = size_t(128) << 20;
hipError_t static_scratch_ptr(void** out);

// KV-cache update (TRT_KVCacheUpdate, linear mode).  Element strides; the
// row of (b, h, n) of the cache / output starts at base + b*sb + h*sh + n*sn
// elements; the packed update row r of head h at base + r*sn + h*sh.
struct KvUpdateParams {
    const char* upd;
    int64_t u_sb, u_sh, u_sn;
    const char* cache;
    int64_t c_sb, c_sh, c_sn;
    char* out;
    int64_t o_sb, o_sh, o_sn;
    const int32_t* wi;   // write indices [B] or null
    const int32_t* ul;   // cumulative update lengths [B+1] or null
    int32_t packed;
    int32_t B, H, N;     // cache extents
    int32_t n_u;         // padded update rows per sequence
    int64_t T;           // packed update rows
    int32_t es;          // element bytes
    int32_t row_bytes;   // D * es, a multiple of 16
    int32_t in_place;    // out is the cache: copy nothing but the update rows
};

hipError_t launch_kv_update(const KvUpdateParams& p, hipStream_t stream);

}  // namespace gqa
