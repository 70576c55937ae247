// prefill.hip -- launcher of the general prefill kernel and the plan kernel
// that writes its per-workgroup records (the attention kernels are
// templates in prefill_impl.h, instantiated per element type in
// prefill_f16.hip, prefill_bf16.hip and prefill_fp8.hip, and for 16-bit Q over
// an fp8 KV cache in prefill_kv8_{f16,bf16}.hip, so that they compile in
// parallel; each launches its split-KV combine itself).
#include "launch.h"
#include "tile_common.h"

namespace gqa {

// The per-workgroup records of the prefill grid (AttnParams::wrec), built
// once per call instead of in every workgroup: wave 0 of each block sorts
// the sequences into dispatch order (dispatch_order: longest KV first) and
// scans their row-tile counts; then each thread maps one workgroup id
// through the XCD remap to (dispatch position, head group, key slice) and
// the position to (sequence, row tile) -- the same map the kernel builds
// without records.  Batches of at most 64 sequences (host-checked).
__global__ __launch_bounds__(256) void prefill_plan_kernel(AttnParams p, int32_t* rec, int n_wg) {
    __shared__ int s_idx[64], s_n[64], s_incl[64];
    __shared__ SeqInfo s_si[64];
    const int tid = threadIdx.x;
    if (tid < 64) {
        const SeqInfo si = map_lane_info(p);
        int idx, n, incl;
        dispatch_order(p, p.rows_per_wg, si, idx, n, incl);
        s_idx[tid] = idx;
        s_n[tid] = n;
        s_incl[tid] = incl;
        s_si[tid] = si;
    }
    __syncthreads();
    const int L = blockIdx.x * 256 + tid;
    if (L >= n_wg) return;
    const int nx = p.grid_x, ny = p.grid_y, nz = p.n_splits > 1 ? p.n_splits : 1;
    int bx = L % nx, by = (L / nx) % ny, bz = L / (nx * ny);
    if (p.xcds > 1) xcd_remap(p.xcds, nx, ny, nz, bx, by, bz);
    const int hbase = by * p.heads_per_wg;
    i32x4 r0 = {-1, 0, 0, 0};
    i32x4 r1 = {0, 0, hbase, (hbase / p.group) | (bz << 16)};
    // the first sorted entry whose inclusive tile count exceeds bx (the
    // counts never decrease): its sequence holds position bx
    int lo = 0, hi = 64;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_incl[mid] > bx) hi = mid;
        else lo = mid + 1;
    }
    if (lo < 64) {
        const int n = s_n[lo], incl = s_incl[lo];
        const int b = s_idx[lo];
        const SeqInfo si = s_si[b];
        r0 = i32x4{b, n - 1 - (bx - (incl - n)), si.q_len, si.kv_len};
        r1[0] = si.q_start;
        r1[1] = si.kv_start;
    }
    i32x4* out = (i32x4*)(rec + (int64_t)L * kWorkRecInts);
    out[0] = r0;
    out[1] = r1;
}

hipError_t launch_prefill_plan(const AttnParams& p, int32_t* rec, int n_wg, hipStream_t stream) {
    if (n_wg <= 0) return hipSuccess;
    hipLaunchKernelGGL(prefill_plan_kernel, dim3((n_wg + 255) / 256), dim3(256), 0, stream, p, rec,
                       n_wg);
    return hipGetLastError();
}

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
