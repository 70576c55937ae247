// tile_common.h -- pieces shared by the prefill kernels: the ragged row-tile
// map, the swizzled row-major V layout in LDS and the gfx950 LDS transpose
// reads that turn it into MFMA operands.
#pragma once
#include "device_common.h"

namespace gqa {

// V is staged row-major; the 16-byte units of row `key` are XOR-swizzled so
// that the transpose reads of one instruction (8 keys x 64 bytes for 16-bit
// V, 16 keys x 32 bytes for fp8 V) spread evenly over the LDS banks.
template <typename C>
__device__ __forceinline__ int v_swz(int key) {
    if constexpr (C::FP8) return 2 * ((key / C::RPL) % (C::VUNITS / 2));
    else return 4 * ((key / C::RPL) % (C::VUNITS / 4));
}
// Byte offset of element d of V row `key`.
template <typename C>
__device__ __forceinline__ int v_addr(int key, int d) {
    const int byte = d * C::ES;
    return key * C::VROW + (((byte >> 4) ^ v_swz<C>(key)) << 4) + (byte & 15);
}

// Buffer load of 16 bytes per lane written straight into LDS (no registers):
// lane i's bytes land at lds + 16 i; a lane outside the descriptor's range
// writes zeros.  Completion is tracked by vmcnt.  (The builtin exists only
// for the device target; the host pass sees an empty body.)
__device__ __forceinline__ void buf_load_lds16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                             voff, 0, 0, 0);
#endif
}

typedef __fp16 lds_h4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
// LDS transpose reads (gfx950): within each group of 16 lanes,
// ds_read_b64_tr_b16 gives lane 4q+c the 16-bit element c of lanes 4k+q
// (k = 0..3) and ds_read_b64_tr_b8 gives lane 8q+c the byte c of lanes 2k+q
// (k = 0..7).  Pointing lane 4k+q (2k+q) at (key_k, d0 + 4q (8q)) of a
// row-major V hands lane i the keys key_k at d = d0 + i: one row of V^T.
__device__ __forceinline__ u32x2 tr16(const char* p) {
    lds_h4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) lds_h4*)p);
    return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x2 tr8(const char* p) {
    return __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)p));
}

// ------------------------------------------------------------------ tile map
// Dispatch position `pos` -> (b, row tile within b); sequence b has
// ceil(q_len_b / R) row tiles.  Positions run over the sequences by
// decreasing KV length (ties: lower index first; more than 64 sequences:
// index order), and within a sequence from its last row tile to its first,
// so the heaviest work items (long rows of long sequences under causal
// masking) start first and the lightest ones fill the tail.  Wave 0
// computes the map; the result lands in s_map[0..1] (b = -1 past the last
// tile).  Block-wide barrier included.
__device__ __forceinline__ void map_tile(const AttnParams& p, int pos, int R, int* s_map) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (wave == 0) {
        if (lane == 0) s_map[0] = -1;
        if (p.batch <= 64) {
            // Bitonic sort of the (KV length, index) pairs across the 64
            // lanes into dispatch order (longer first, then lower index;
            // lanes past the batch sort last), then an inclusive scan of the
            // row-tile counts in that order.
            int key = lane < p.batch ? kv_len_of(p, lane) : -1;
            int idx = lane;
            int n = lane < p.batch ? (q_len_of(p, lane) + R - 1) / R : 0;  // row tiles
#pragma unroll
            for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
                for (int stride = size >> 1; stride > 0; stride >>= 1) {
                    const int pk = __shfl_xor(key, stride), pi = __shfl_xor(idx, stride);
                    const int pn = __shfl_xor(n, stride);
                    // does the partner's pair come first in dispatch order?
                    const bool pfirst = pk > key || (pk == key && pi < idx);
                    const bool lower = (lane & stride) == 0;
                    const bool fwd = size == 64 || (lane & size) == 0;  // run direction
                    if (pfirst == (lower == fwd)) {
                        key = pk;
                        idx = pi;
                        n = pn;
                    }
                }
            }
            int incl = n;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(incl, off);
                if (lane >= off) incl += y;
            }
            const int ahead = incl - n;
            if (n > 0 && pos >= ahead && pos < incl) {
                s_map[0] = idx;
                s_map[1] = n - 1 - (pos - ahead);
            }
        } else {
            int acc = 0;
            for (int base = 0; base < p.batch; base += 64) {
                const int b = base + lane;
                int n = 0;
                if (b < p.batch) n = (q_len_of(p, b) + R - 1) / R;
                int incl = n;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int y = __shfl_up(incl, off);
                    if (lane >= off) incl += y;
                }
                const int excl = incl - n;
                if (n > 0 && pos >= acc + excl && pos < acc + incl) {
                    s_map[0] = b;
                    s_map[1] = n - 1 - (pos - acc - excl);
                }
                acc += __shfl(incl, 63);
                if (acc > pos) break;
            }
        }
    }
    __syncthreads();
}


}  // namespace gqa
