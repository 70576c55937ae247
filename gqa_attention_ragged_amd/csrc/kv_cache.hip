// kv_cache.hip -- the KV-cache update (TRT_KVCacheUpdate on the onnx-tensorrt
// "TensorRT Custom Operator Schemas" page, linear mode along the sequence
// axis of the [B, H, N, D] cache), gfx950.
//
// Byte copies of whole D-rows in 16-byte units: one thread moves one unit,
// grid-stride over the units.  Out of place, the cache is copied into Y
// first (same stream, so the scatter that follows overwrites it).  The
// scatter maps each update unit to (b, h, t), resolves the sequence's length
// and write index on the device, and writes the row at position
// write_index + t when that lies in [0, N).  Nothing else of Y is touched.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace gqa {

constexpr int kKvThreads = 256;

__global__ __launch_bounds__(kKvThreads) void kv_copy_kernel(KvUpdateParams p) {
    const int upr = p.row_bytes / 16;  // 16-byte units per row
    const int64_t total = (int64_t)p.B * p.H * p.N * upr;
    const int64_t stride = (int64_t)gridDim.x * kKvThreads;
    for (int64_t u = (int64_t)blockIdx.x * kKvThreads + threadIdx.x; u < total; u += stride) {
        const int64_t row = u / upr;
        const int c = (int)(u - row * upr);
        const int n = (int)(row % p.N);
        const int64_t bh = row / p.N;
        const int h = (int)(bh % p.H), b = (int)(bh / p.H);
        const u32x4 v = *(const u32x4*)(p.cache +
                                        ((int64_t)b * p.c_sb + (int64_t)h * p.c_sh + (int64_t)n * p.c_sn) * p.es +
                                        c * 16);
        *(u32x4*)(p.out + ((int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)n * p.o_sn) * p.es +
                  c * 16) = v;
    }
}

// Sequence of packed update row r: the b with ul[b] <= r < ul[b+1]
// (binary search over the cumulative lengths, here in LDS).
__device__ __forceinline__ int seq_of_row(const int32_t* ul, int B, int64_t r) {
    int lo = 0, hi = B;  // invariant: ul[lo] <= r < ul[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)ul[mid] <= r) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Cumulative update lengths cached per workgroup (packed updates of up to
// kKvLdsSeqs sequences; more read them from global memory).
constexpr int kKvLdsSeqs = 2048;

// IDX: index type of the unit arithmetic (32-bit when every unit index
// fits, which turns the per-unit divisions into 32-bit ones).
template <typename IDX>
__global__ __launch_bounds__(kKvThreads) void kv_scatter_kernel(KvUpdateParams p) {
    __shared__ int32_t s_ul[kKvLdsSeqs + 1];
    const IDX upr = (IDX)(p.row_bytes / 16);
    const IDX H = (IDX)p.H;
    const IDX rows = p.packed ? (IDX)(p.T * p.H) : (IDX)((int64_t)p.B * p.H * p.n_u);
    const IDX total = rows * upr;
    const IDX stride = (IDX)gridDim.x * kKvThreads;
    const int32_t* ul = p.ul;
    if (p.packed && p.B <= kKvLdsSeqs) {
        for (int i = threadIdx.x; i <= p.B; i += kKvThreads) s_ul[i] = p.ul[i];
        __syncthreads();
        ul = s_ul;
    }
    const int64_t last = p.packed ? (int64_t)ul[p.B] : 0;
    for (IDX u = (IDX)blockIdx.x * kKvThreads + threadIdx.x; u < total; u += stride) {
        const IDX row = u / upr;
        const int c = (int)(u - row * upr);
        int b, h, t;
        const char* src;
        if (p.packed) {
            const IDX r = row / H;
            h = (int)(row - r * H);
            if ((int64_t)r >= last) continue;  // beyond the last sequence's rows
            b = seq_of_row(ul, p.B, (int64_t)r);
            t = (int)((int64_t)r - ul[b]);
            src = p.upd + ((int64_t)r * p.u_sn + (int64_t)h * p.u_sh) * p.es;
        } else {
            const IDX nu = (IDX)p.n_u;
            const IDX bh = row / nu;
            t = (int)(row - bh * nu);
            b = (int)(bh / H);
            h = (int)(bh - (IDX)b * H);
            if (p.ul && t >= p.ul[b + 1] - p.ul[b]) continue;
            src = p.upd + ((int64_t)b * p.u_sb + (int64_t)h * p.u_sh + (int64_t)t * p.u_sn) * p.es;
        }
        const int64_t pos = (int64_t)(p.wi ? p.wi[b] : 0) + t;
        if (pos < 0 || pos >= p.N) continue;  // outside the cache: dropped
        const u32x4 v = *(const u32x4*)(src + c * 16);
        *(u32x4*)(p.out + ((int64_t)b * p.o_sb + (int64_t)h * p.o_sh + pos * p.o_sn) * p.es + c * 16) = v;
    }
}

static int grid_for(int64_t units) {
    const int64_t g = (units + kKvThreads - 1) / kKvThreads;
    return (int)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

hipError_t launch_kv_update(const KvUpdateParams& p, hipStream_t stream) {
    const int upr = p.row_bytes / 16;
    if (!p.in_place && (int64_t)p.B * p.H * p.N > 0) {
        hipLaunchKernelGGL(kv_copy_kernel, dim3(grid_for((int64_t)p.B * p.H * p.N * upr)),
                           dim3(kKvThreads), 0, stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t rows = p.packed ? p.T * p.H : (int64_t)p.B * p.H * p.n_u;
    if (rows > 0 && p.B > 0) {
        if (rows * upr < ((int64_t)1 << 31) - (int64_t)65536 * kKvThreads)
            hipLaunchKernelGGL(kv_scatter_kernel<uint32_t>, dim3(grid_for(rows * upr)),
                               dim3(kKvThreads), 0, stream, p);
        else
            hipLaunchKernelGGL(kv_scatter_kernel<int64_t>, dim3(grid_for(rows * upr)),
                               dim3(kKvThreads), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace gqa
