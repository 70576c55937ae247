// tile_common.h -- pieces shared by the prefill kernels: the ragged row-tile
// map, the swizzled row-major V layout in LDS and the gfx950 LDS transpose
// reads that turn it into MFMA operands.
#pragma once
#include "device_common.h"

#include <type_traits>

namespace gqa {

// V is staged row-major; the 16-byte units of row `key` are XOR-swizzled so
// that the transpose reads of one instruction (8 keys x 64 bytes for 16-bit
// V, 16 keys x 32 bytes for fp8 V) spread evenly over the LDS banks.  An fp8
// read's half-wave covers keys base + {0..3, 8..11} (key bits 0, 1 and 3) and
// one pair of units in each row; rows that share a 256-byte bank line differ
// in the key bits below RPL, so the swizzle takes the remaining ones (bits 1
// and 3 with two rows per line, bit 3 with four) to give the rows at one
// line position disjoint unit pairs.
template <typename C>
__device__ __forceinline__ int v_swz(int key) {
    if constexpr (C::FP8) {
        static_assert(C::RPL == 2 || C::RPL == 4, "fp8 V rows of 128 or 64 bytes");
        if constexpr (C::RPL == 2) return 2 * (((key >> 1) & 1) | (((key >> 3) & 1) << 1));
        else return 2 * ((key >> 3) & 1);
    } else {
        return 4 * ((key / C::RPL) % (C::VUNITS / 4));
    }
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

// The same copy issued as an instruction the compiler does not see as a
// write to LDS.  With the builtin the compiler guards LDS reads against the
// copies in flight itself, and for reads it cannot tell apart from the
// copied range (the transpose reads carry no alias information) it waits for
// every copy in flight -- including the ones issued for later tiles, which
// serializes the copy latency into the loop.  With this form it inserts no
// such wait: the caller must wait for the copy (s_waitcnt vmcnt) and make it
// visible to the other waves (barrier) before any wave reads the bytes.  The
// instruction has no register result; M0 carries the LDS address.
//
// The compiler does not check hazards into an asm block either, so the
// block opens with the wait states the instruction needs itself: an LDS DMA
// needs 1 after an SALU write of M0 (the compiler sets M0 right before the
// block), and a VMEM instruction reading an SGPR that a VALU instruction
// wrote needs 5.  VALU_RSRC: the descriptor's SGPRs may come from VALU
// instructions (v_readfirstlane when a page table supplies the base,
// v_readlane when they were spilled): s_nop 4 (5 wait states); otherwise
// s_nop 0.  Without them the load can take the previous contents of a
// descriptor SGPR as its base address.  The choice per kernel is checked on
// the compiled code (every copy, the wait states back to the last VALU write
// of its SGPRs and the last write of M0).
template <bool VALU_RSRC>
__device__ __forceinline__ void buf_load_lds16_async(__amdgpu_buffer_rsrc_t r, char* lds,
                                                     uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t m = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
    if constexpr (VALU_RSRC) {
        __asm__ volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff),
                         "s"(r), "{m0}"(m)
                         : "memory");
    } else {
        __asm__ volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff),
                         "s"(r), "{m0}"(m)
                         : "memory");
    }
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
// What a workgroup needs of its sequence: lengths and first rows in packed
// tensors (0 where the tensor is padded).
struct SeqInfo {
    int q_len, kv_len, q_start, kv_start;
};
__device__ __forceinline__ SeqInfo seq_info(const AttnParams& p, int b) {
    SeqInfo s;
    s.q_start = p.ql ? p.ql[b] : 0;
    s.q_len = p.ql ? p.ql[b + 1] - s.q_start : p.n_q;
    if (p.kv_packed) {
        s.kv_start = p.kl[b];
        s.kv_len = p.kl[b + 1] - s.kv_start;
    } else {
        s.kv_start = 0;
        s.kv_len = p.kl ? p.kl[b] : p.n_kv;
    }
    return s;
}

// Lane l receives v of lane l ^ M.  Inside a 16-lane row the exchange is a
// DPP move (quad permutations, the half-row mirror, the row rotation by 8),
// with no round trip through LDS; across rows it is a bpermute.
template <int M>
__device__ __forceinline__ int xor_lanes(int v) {
    if constexpr (M == 1) {
        return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    } else if constexpr (M == 2) {
        return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    } else if constexpr (M == 4) {
        // half-row mirror (l ^ 7), then quad reversal (l ^ 3)
        const int m = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
        return __builtin_amdgcn_update_dpp(0, m, 0x1B, 0xF, 0xF, false);
    } else if constexpr (M == 8) {
        return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
    } else {
        return __shfl_xor(v, M);
    }
}
// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each
// row (lanes without a source add 0), then each row adds the totals of the
// rows before it through the row broadcasts of lanes 15 and 31.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

// Wave 0's per-lane sequence values for the map below (lane l: sequence l
// when the batch has at most 64 sequences).  Called at kernel start so that
// the loads overlap the work before the map.
__device__ __forceinline__ SeqInfo map_lane_info(const AttnParams& p) {
    const int lane = threadIdx.x & 63;
    SeqInfo si = {0, -1, 0, 0};
    if (threadIdx.x < 64 && p.batch <= 64 && lane < p.batch) si = seq_info(p, lane);
    return si;
}

// Dispatch order of the sequences for the tile maps below (wave 0, at most
// 64 sequences: lane l holds sequence l's `si`): lane j receives the j-th
// sequence in dispatch order (`idx`, past the batch: an index >= batch),
// its row-tile count `n` (R rows per tile) and the inclusive scan `incl` of
// the counts in that order.
__device__ __forceinline__ void dispatch_order(const AttnParams& p, int R, const SeqInfo& si,
                                               int& idx, int& n, int& incl) {
    const int lane = threadIdx.x & 63;
    // Bitonic sort of the (KV length, index) pairs into dispatch
    // order (longer first, then lower index; lanes past the batch
    // sort last) over groups of NMAX = 16, 32 or 64 lanes, the
    // smallest that holds the batch (groups past the first hold
    // only empty lanes), then an inclusive scan of the row-tile
    // counts in that order.
    int key = si.kv_len;
    idx = lane;
    n = lane < p.batch ? (si.q_len + R - 1) / R : 0;  // row tiles
    const int nmax = p.batch <= 16 ? 16 : p.batch <= 32 ? 32 : 64;
    // one compare-exchange step with the partner lane ^ stride
    auto step = [&](auto stride_c, int size) {
        constexpr int stride = decltype(stride_c)::value;
        const int pk = xor_lanes<stride>(key), pi = xor_lanes<stride>(idx);
        const int pn = xor_lanes<stride>(n);
        // does the partner's pair come first in dispatch order?
        const bool pfirst = pk > key || (pk == key && pi < idx);
        const bool lower = (lane & stride) == 0;
        const bool fwd = size == nmax || (lane & size) == 0;  // run direction
        if (pfirst == (lower == fwd)) {
            key = pk;
            idx = pi;
            n = pn;
        }
    };
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S4 = std::integral_constant<int, 4>;
    using S8 = std::integral_constant<int, 8>;
    using S16 = std::integral_constant<int, 16>;
    using S32 = std::integral_constant<int, 32>;
    step(S1{}, 2);
    step(S2{}, 4), step(S1{}, 4);
    step(S4{}, 8), step(S2{}, 8), step(S1{}, 8);
    step(S8{}, 16), step(S4{}, 16), step(S2{}, 16), step(S1{}, 16);
    if (nmax >= 32) {
        step(S16{}, 32), step(S8{}, 32), step(S4{}, 32), step(S2{}, 32), step(S1{}, 32);
    }
    if (nmax == 64) {
        step(S32{}, 64), step(S16{}, 64), step(S8{}, 64), step(S4{}, 64), step(S2{}, 64);
        step(S1{}, 64);
    }
    incl = wave_incl_scan(n);
}

// XCD-aware remap of a workgroup's grid position (bx, by, bz) over X XCDs.
// Consecutive workgroup ids go to the XCDs in turn (id % X), each with its
// own L2; remapped, XCD x takes one contiguous block of the work items
// ordered (head group, split, row tile), so the K / V rows of a head group
// are fetched into one L2 rather than into all of them.
__device__ __forceinline__ void xcd_remap(int X, int nx, int ny, int nz, int& bx, int& by,
                                          int& bz) {
    const int n = nx * ny * nz, L = bx + nx * (by + ny * bz);
    const int xcd = L % X, k = L / X, q = n / X, r = n % X;
    const int li = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + k;
    bx = li % nx;
    bz = (li / nx) % nz;
    by = li / (nx * nz);
}

// Dispatch position `pos` -> (b, row tile within b); sequence b has
// ceil(q_len_b / R) row tiles.  Positions run over the sequences by
// decreasing KV length (ties: lower index first; more than 64 sequences:
// index order), and within a sequence from its last row tile to its first,
// so the heaviest work items (long rows of long sequences under causal
// masking) start first and the lightest ones fill the tail.  Wave 0
// computes the map from its lanes' `si` (map_lane_info); s_map[0..5]
// receives b (-1 past the last tile), the row tile, and b's q_len, kv_len,
// q_start and kv_start, so that the workgroup reads its sequence's lengths
// from LDS rather than from memory again.  Block-wide barrier included.
__device__ __forceinline__ void map_tile(const AttnParams& p, int pos, int R, int* s_map,
                                         const SeqInfo& si) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (wave == 0) {
        if (lane == 0) s_map[0] = -1;
        if (p.batch <= 64) {
            int idx, n, incl;
            dispatch_order(p, R, si, idx, n, incl);
            const int ahead = incl - n;
            const uint64_t hit = __ballot(n > 0 && pos >= ahead && pos < incl);
            if (hit != 0 && __builtin_amdgcn_readlane(idx, (int)__builtin_ctzll(hit)) < p.batch) {
                // the one matching lane (wave-uniform), then its sequence's
                // values from the lane that loaded them
                const int src = (int)__builtin_ctzll(hit);
                const int b = __builtin_amdgcn_readlane(idx, src);
                const int t = __builtin_amdgcn_readlane(n - 1 - (pos - ahead), src);
                const int ql = __builtin_amdgcn_readlane(si.q_len, b);
                const int kl = __builtin_amdgcn_readlane(si.kv_len, b);
                const int qs = __builtin_amdgcn_readlane(si.q_start, b);
                const int ks = __builtin_amdgcn_readlane(si.kv_start, b);
                if (lane == 0) {
                    s_map[0] = b;
                    s_map[1] = t;
                    s_map[2] = ql;
                    s_map[3] = kl;
                    s_map[4] = qs;
                    s_map[5] = ks;
                }
            }
        } else {
            int acc = 0;
            for (int base = 0; base < p.batch; base += 64) {
                const int b = base + lane;
                int n = 0;
                SeqInfo si = {0, 0, 0, 0};
                if (b < p.batch) {
                    si = seq_info(p, b);
                    n = (si.q_len + R - 1) / R;
                }
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
                    s_map[2] = si.q_len;
                    s_map[3] = si.kv_len;
                    s_map[4] = si.q_start;
                    s_map[5] = si.kv_start;
                }
                acc += __shfl(incl, 63);
                if (acc > pos) break;
            }
        }
    }
    __syncthreads();
}


}  // namespace gqa
