// decode.hip -- attention for query length 1 (autoregressive decode), gfx950.
//
// Same operator as the prefill kernel (onnx-tensorrt "TensorRT Custom
// Operator Schemas" page, TRT_Attention), specialised for padded Q with
// N_q = 1, softmax, no mask, and KV either in Q's type or an FP8 (E4M3FN)
// cache with per-tensor fp32 dequantization scales (TensorRT Edge-LLM
// "TensorRT Plugins Guide", AttentionPlugin: FP16 or FP8 KV cache).
//
// The step is bound by the HBM read of K and V, so the design is about
// keeping many bytes in flight on every CU:
//   * split-KV: workgroup (b, kv head, split) reads split_keys keys once for
//     all G = H_q / H_kv query heads that share them; the grid holds
//     B * H_kv * ceil(N_kv / split_keys) workgroups and those past a
//     sequence's length exit at once.  The split is the slowest grid
//     dimension: workgroups are dispatched in order, so the first splits of
//     every sequence (always busy) go first and the mostly empty last splits
//     trail at the end, instead of runs of empty workgroups between the busy
//     ones holding the dispatcher up (measured: 1.2 -> ~2 busy workgroups per
//     CU);
//   * the 4 waves of a workgroup each stream their own 32-key tiles with
//     coalesced 16-byte loads (K straight into MFMA operand registers, V
//     through a wave-private LDS transpose), no workgroup barrier in the
//     key loop;
//   * scores and outputs use 16x16x32 MFMAs with the G heads as the 16-wide
//     dimension (S^T = K Q^T, O^T = V^T P^T), online softmax in the exp2
//     domain;
//   * the waves merge (max, sum, O) through LDS and write one fp32 partial
//     per (b, head, split); a second kernel merges the splits with the
//     log-sum-exp rule  M = max m_s,  O = sum e^(m_s-M) O_s / sum e^(m_s-M) l_s
//     and writes the output row.
#include "device_common.h"
#include "launch.h"
#include "main_timer.h"

#include <type_traits>

namespace gqa {

// Order this wave's LDS traffic: every LDS access issued before completes
// before any issued after (the V tile is written and read by different lanes
// of the same wave).  Waits on LDS only (lgkmcnt(0)), never on the global
// loads in flight, and stops the compiler from moving memory operations
// across it.
__device__ __forceinline__ void lds_wave_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
}

typedef __fp16 lds_h4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) lds_h4* lds_h4_ptr;
typedef __attribute__((address_space(3))) u32x2* lds_u2_ptr;

// LDS transpose reads (gfx950).  Within each group of 16 lanes, lane L
// supplies an address; ds_read_b64_tr_b16 gives lane 4q+c the 16-bit element
// c of lanes 4k+q (k = 0..3), ds_read_b64_tr_b8 gives lane 8q+c the byte c of
// lanes 2k+q (k = 0..7).  With row-major V, pointing lane 4k+q (2k+q) at
// (key_k, d0 + 4q (8q)) hands lane i the values of keys key_k at d = d0 + i:
// a column of V, i.e. a row of V^T, as the MFMA A operand wants it.
__device__ __forceinline__ u32x2 lds_tr16(const char* p) {
    lds_h4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4_ptr)(p));
    return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x2 lds_tr8(const char* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                         (__attribute__((address_space(3))) i32x2*)(p)));
}

template <typename TQ, typename TKV, int D, bool PAGED = false>
struct Decode {
    static constexpr bool KV8 = std::is_same<TKV, fp8>::value;
    static constexpr int KES = KV8 ? 1 : 2;       // K/V element bytes
    static constexpr int KT = 32;                 // keys per wave tile
    static constexpr int ROWB = D * KES;          // bytes per V row (global and LDS)
    static constexpr int VCH = ROWB / 16;         // 16-byte chunks per V row
    static constexpr int VRPI = 64 / VCH;         // V rows per wave load
    static constexpr int VINS = KT / VRPI;        // V loads per lane per tile
    static constexpr int RPL = ROWB >= 256 ? 1 : 256 / ROWB;  // rows per 256-byte bank line
    static constexpr int WAVE_LDS = KT * ROWB;
    static constexpr int MERGE_FLOATS = D * 16 + 32;
    static constexpr int LDS_BYTES =
        4 * WAVE_LDS > 4 * MERGE_FLOATS * 4 ? 4 * WAVE_LDS : 4 * MERGE_FLOATS * 4;
    typedef typename Vec8<TQ>::type V8;
    typedef typename std::conditional<KV8, u32x2, u32x4>::type ChunkT;
    // K operand registers per 16-key block: 16-bit K, one 16-byte chunk (8
    // values) per k-step; fp8 K, one 16-byte chunk per two k-steps.
    static constexpr int KCH = KV8 ? D / 64 : D / 32;
    // Channel of the first of the 8 values lane group g feeds into k-step ks.
    // The dot product may pair channels with MFMA k-slots in any order, as
    // long as K and Q use the same one: fp8 K lanes take 16 contiguous bytes
    // (channels 64 (ks/2) + 16 g .. +15) that serve k-steps ks and ks+1.
    __device__ __forceinline__ static int kchan(int ks, int g) {
        return KV8 ? (ks >> 1) * 64 + g * 16 + (ks & 1) * 8 : ks * 32 + g * 8;
    }
    // The 8 K values of k-step ks out of the lane's chunks.
    __device__ __forceinline__ static ChunkT kpart(const u32x4 (&k)[KCH], int ks) {
        if constexpr (KV8) {
            const u32x4 c = k[ks >> 1];
            u32x2 r;
            r[0] = c[(ks & 1) * 2];
            r[1] = c[(ks & 1) * 2 + 1];
            return r;
        } else {
            return k[ks];
        }
    }

    // XOR swizzle of the 16-byte chunks of V row `key` in LDS, chosen so the
    // transpose reads of one instruction (16 keys x 32 bytes for 16-bit V,
    // 32 keys x 16 bytes for fp8 V) spread evenly over the LDS banks.
    __device__ __forceinline__ static int swz(int key) {
        if constexpr (KV8) return (key / RPL) % VCH;
        else return 2 * ((key / RPL) % (VCH / 2));
    }

    __device__ __forceinline__ static V8 to8(ChunkT c) {
        if constexpr (KV8) {
            return e4m3x8_to<TQ>(c);
        } else {
            return __builtin_bit_cast(V8, c);
        }
    }

    __device__ __forceinline__ static void run(const AttnParams& p, char* smem) {
        const int kvh = blockIdx.x, b = blockIdx.y, s = blockIdx.z;
        const int tid = threadIdx.x, lane = tid & 63;
        // wave index in a scalar register: everything derived from it is
        // wave-uniform, and branches on it are scalar branches
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int l16 = lane & 15, g = lane >> 4;
        const int G = p.group;
        if (q_len_of(p, b) <= 0) return;
        const int kv_len = kv_len_of(p, b);
        const int k0 = s * p.split_keys;
        if (k0 >= kv_len) return;
        const int k1 = min(k0 + p.split_keys, kv_len);

        // Q operand: lane (head l16, group g) holds Q[h][ks*32 + g*8 .. +7]
        V8 qreg[D / 32];
        {
            const bool ok = l16 < G;
            const char* qrow = (const char*)p.q.ptr +
                               (q_rowbase(p, b) + (int64_t)(kvh * G + (ok ? l16 : 0)) * p.q.sh) * 2;
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                V8 a = {};
                if (ok) a = *(const V8*)(qrow + kchan(ks, g) * 2);
                qreg[ks] = a;
            }
        }
        // paged KV: the head's offset inside a page (the page comes per tile)
        const int64_t kro = PAGED ? 0 : kv_rowbase(p, p.k, b), vro = PAGED ? 0 : kv_rowbase(p, p.v, b);
        const char* kbase = (const char*)p.k.ptr + (kro + (int64_t)kvh * p.k.sh) * KES;
        const char* vbase = (const char*)p.v.ptr + (vro + (int64_t)kvh * p.v.sh) * KES;
        const int32_t* ptk = p.ptab + (int64_t)b * 2 * p.ptab_pages;
        char* sv = smem + wave * WAVE_LDS;
        const float sc = p.scale * p.k_descale * kLog2e;

        f32x4 o[D / 16];
#pragma unroll
        for (int db = 0; db < D / 16; ++db) o[db] = f32x4{};
        float m_run = -INFINITY, l_run = 0.f;

        // V loads: lane -> (row lane / VCH of each group of VRPI rows, chunk lane % VCH)
        const int vrow = lane / VCH, vch = lane % VCH;
        // Q must be resident before the key loop (see the prefill kernel).
        __builtin_amdgcn_s_waitcnt(0x0F70);

        // Registers of one 32-key tile: K operand (2 blocks x D/32 steps) and
        // V chunks.  Two sets: the next tile is in flight while the current
        // one is computed.
        struct Tile {
            u32x4 k[2][KCH];
            u32x4 v[VINS];
        };
        // Rows [k0, k1) of this sequence, the split's keys: keys past the
        // split's end read as zero without touching memory (and are masked
        // below).  The window starts at the split (64-bit base), so a
        // sequence's rows may span more than 4 GiB; the host bounds one
        // split's span (plus the prefetch past its end) below 2^32 bytes.
        const __amdgpu_buffer_rsrc_t krs =
            make_rsrc(kbase + (int64_t)k0 * p.k.sn * KES, rows_bytes(k1 - k0, p.k.sn, D, KES));
        const __amdgpu_buffer_rsrc_t vrs =
            make_rsrc(vbase + (int64_t)k0 * p.v.sn * KES, rows_bytes(k1 - k0, p.v.sn, D, KES));
        // paged: the page pair of the next tile this wave loads, read from
        // the table one tile ahead (its latency then overlaps a tile's
        // compute instead of preceding the tile's loads); a wave loads its
        // tiles in increasing order, 4 * KT keys apart
        const int stride = 4 * KT;
        int pk_next = 0, pv_next = 0;
        auto fetch_pages = [&](int j) {
            if constexpr (PAGED) {
                // the table is read at a clamped index (a tile past the
                // split's end gets an empty range below)
                const int pi = min(j, k1 - 1) >> p.page_shift;
                pk_next = ptk[pi];
                pv_next = ptk[p.ptab_pages + pi];
            }
        };
        auto load = [&](Tile& t, int j0) {
            if constexpr (PAGED) {
                // a 32-key tile lies inside one page (pages hold a power of
                // two >= 32 keys)
                const int within = j0 & ((1 << p.page_shift) - 1);
                const int valid = min(k1 - j0, KT);
                const int pk = pk_next, pv = pv_next;
                fetch_pages(j0 + stride);
                const __amdgpu_buffer_rsrc_t kt = make_rsrc(
                    kbase + ((int64_t)pk * p.k.sb + (int64_t)within * p.k.sn) * KES,
                    rows_bytes(valid, p.k.sn, D, KES));
                const __amdgpu_buffer_rsrc_t vt = make_rsrc(
                    vbase + ((int64_t)pv * p.v.sb + (int64_t)within * p.v.sn) * KES,
                    rows_bytes(valid, p.v.sn, D, KES));
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int jj = kb * 16 + l16;
#pragma unroll
                    for (int kc = 0; kc < KCH; ++kc)
                        buf_load(kt, (uint32_t)(((int64_t)jj * p.k.sn + kchan(kc * (KV8 ? 2 : 1), g)) * KES),
                                 t.k[kb][kc]);
                }
#pragma unroll
                for (int i = 0; i < VINS; ++i) {
                    const int jj = i * VRPI + vrow;
                    buf_load(vt, (uint32_t)((int64_t)jj * p.v.sn * KES + vch * 16), t.v[i]);
                }
                return;
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int j = j0 - k0 + kb * 16 + l16;  // key within the split
#pragma unroll
                for (int kc = 0; kc < KCH; ++kc)
                    buf_load(krs, (uint32_t)(((int64_t)j * p.k.sn + kchan(kc * (KV8 ? 2 : 1), g)) * KES),
                             t.k[kb][kc]);
            }
#pragma unroll
            for (int i = 0; i < VINS; ++i) {
                const int j = j0 - k0 + i * VRPI + vrow;
                buf_load(vrs, (uint32_t)((int64_t)j * p.v.sn * KES + vch * 16), t.v[i]);
            }
        };
        auto compute = [&](const Tile& t, int j0) {
            // ---- S^T = K Q^T
            f32x4 st[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x4 acc = {};
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) acc = mfma16(to8(kpart(t.k[kb], ks)), qreg[ks], acc);
                st[kb] = acc;
            }
            // ---- V tile, row-major, into this wave's LDS (swizzled chunks)
#pragma unroll
            for (int i = 0; i < VINS; ++i) {
                const int row = i * VRPI + vrow;
                *(u32x4*)(sv + row * ROWB + ((vch ^ swz(row)) * 16)) = t.v[i];
            }
            // ---- predicate + online softmax (lane: head l16, keys kb*16 + g*4 + r)
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = j0 + kb * 16 + g * 4 + r;
                    float v = st[kb][r] * sc;
                    v = j < k1 ? v : -INFINITY;
                    st[kb][r] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - m_new);  // m_new is finite: key j0 is valid
            float ls = 0.f;
            V8 pb;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = fast_exp2(st[kb][r] - m_new);
                    ls += e;
                    pb[kb * 4 + r] = (TQ)e;
                }
            l_run = l_run * alpha + ls;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < D / 16; ++db) o[db] *= alpha;
            lds_wave_sync();
            // ---- O^T += V^T P^T.  A operand lane (d = l16, group g) element
            // e holds key (e/4)*16 + g*4 + e%4, the key pb[e] belongs to.
#pragma unroll
            for (int db = 0; db < D / 16; ++db) {
                V8 a;
                if constexpr (KV8) {
                    const int key = ((l16 >> 1) >> 2) * 16 + g * 4 + ((l16 >> 1) & 3);
                    const int d = db * 16 + 8 * (l16 & 1);
                    const u32x2 w = lds_tr8(sv + key * ROWB + (((d >> 4) ^ swz(key)) * 16) + (d & 15));
                    a = to8(w);
                } else {
                    const int d = db * 16 + 4 * (l16 & 3);
                    u32x2 lo, hi;
                    {
                        const int key = g * 4 + (l16 >> 2);
                        lo = lds_tr16(sv + key * ROWB + (((d >> 3) ^ swz(key)) * 16) + (d & 7) * 2);
                    }
                    {
                        const int key = 16 + g * 4 + (l16 >> 2);
                        hi = lds_tr16(sv + key * ROWB + (((d >> 3) ^ swz(key)) * 16) + (d & 7) * 2);
                    }
                    u32x4 w;
                    w[0] = lo[0]; w[1] = lo[1]; w[2] = hi[0]; w[3] = hi[1];
                    a = __builtin_bit_cast(V8, w);
                }
                o[db] = mfma16(a, pb, o[db]);
            }
            lds_wave_sync();
        };

        // Software pipeline over this wave's tiles: the loads of the next tile
        // (16-bit KV) or the next two (fp8 KV) are always issued before the
        // current one is computed (past the split's end they fall outside the
        // buffer range: zeros, no traffic).
        int j0 = k0 + wave * KT;
        if (j0 < k1) {
            fetch_pages(j0);
            if constexpr (KV8) {
                // an fp8 tile holds half the bytes of a 16-bit one: the loads
                // of the next two tiles are in flight while one is computed
                Tile a, bt, ct;
                load(a, j0);
                load(bt, j0 + stride);
                while (true) {
                    load(ct, j0 + 2 * stride);
                    compute(a, j0);
                    j0 += stride;
                    if (j0 >= k1) break;
                    load(a, j0 + 2 * stride);
                    compute(bt, j0);
                    j0 += stride;
                    if (j0 >= k1) break;
                    load(bt, j0 + 2 * stride);
                    compute(ct, j0);
                    j0 += stride;
                    if (j0 >= k1) break;
                }
            } else {
                Tile a, bt;
                load(a, j0);
                while (true) {
                    load(bt, j0 + stride);
                    compute(a, j0);
                    j0 += stride;
                    if (j0 >= k1) break;
                    load(a, j0 + stride);
                    compute(bt, j0);
                    j0 += stride;
                    if (j0 >= k1) break;
                }
            }
        }

        // ---- merge the 4 waves through LDS (reusing the V tiles' space)
        l_run += __shfl_xor(l_run, 16);
        l_run += __shfl_xor(l_run, 32);
        __syncthreads();
        float* mg = (float*)smem + wave * MERGE_FLOATS;
        if (g == 0) {
            mg[l16] = m_run;
            mg[16 + l16] = l_run;
        }
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) mg[32 + (db * 16 + g * 4 + r) * 16 + l16] = o[db][r];
        __syncthreads();
        const float* m0 = (const float*)smem;
        for (int idx = tid; idx < G * D; idx += 256) {
            const int hh = idx / D, d = idx % D;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < 4; ++w) M = fmaxf(M, m0[w * MERGE_FLOATS + hh]);
            const float Mu = M == -INFINITY ? 0.f : M;
            float L = 0.f, acc = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float* mw = m0 + w * MERGE_FLOATS;
                const float f = fast_exp2(mw[hh] - Mu);
                L += f * mw[16 + hh];
                acc += f * mw[32 + d * 16 + hh];
            }
            const int64_t slot = ((int64_t)b * p.hq + kvh * G + hh) * p.n_splits + s;
            p.part_o[slot * D + d] = acc;
            if (d == 0) {
                p.part_ml[slot * 2] = M;
                p.part_ml[slot * 2 + 1] = L;
            }
        }
    }
};

template <typename TQ, typename TKV, int D, bool PAGED>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(AttnParams p) {
    typedef Decode<TQ, TKV, D, PAGED> K;
    __shared__ __attribute__((aligned(16))) char smem[K::LDS_BYTES];
    K::run(p, smem);
}

// One thread per output element: merge the splits of (b, head).
template <typename TO, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(AttnParams p) {
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    if (q_len_of(p, b) <= 0) return;
    const int kv_len = kv_len_of(p, b);
    const int ns = kv_len > 0 ? (kv_len + p.split_keys - 1) / p.split_keys : 0;
    const int64_t slot0 = ((int64_t)b * p.hq + h) * p.n_splits;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, p.part_ml[(slot0 + s) * 2]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float f = fast_exp2(p.part_ml[(slot0 + s) * 2] - Mu);
        L += f * p.part_ml[(slot0 + s) * 2 + 1];
        acc += f * p.part_o[(slot0 + s) * D + d];
    }
    const float y = L > 0.f ? acc / L * p.v_descale : 0.f;
    TO* orow = (TO*)p.out + o_rowbase(p, b) + (int64_t)h * p.o_sh;
    orow[d] = (TO)y;
}

template <typename TQ, typename TKV, int D>
static hipError_t launch_t(const AttnParams& p, hipStream_t stream) {
    main_kernel_begin(stream);
    if (p.kv_paged)
        hipLaunchKernelGGL((decode_split_kernel<TQ, TKV, D, true>), dim3(p.hkv, p.batch, p.n_splits),
                           dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_split_kernel<TQ, TKV, D, false>), dim3(p.hkv, p.batch, p.n_splits),
                           dim3(256), 0, stream, p);
    main_kernel_end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<TQ, D>), dim3(p.hq, p.batch), dim3(D), 0, stream, p);
    return hipGetLastError();
}

template <typename TQ>
static hipError_t launch_q(const AttnParams& p, int kv_elem, int head_dim, hipStream_t stream) {
    if (kv_elem == ELEM_FP8)
        return head_dim == 64 ? launch_t<TQ, fp8, 64>(p, stream) : launch_t<TQ, fp8, 128>(p, stream);
    return head_dim == 64 ? launch_t<TQ, TQ, 64>(p, stream) : launch_t<TQ, TQ, 128>(p, stream);
}

hipError_t launch_decode(const AttnParams& p, int q_elem, int kv_elem, int head_dim,
                         hipStream_t stream) {
    if (q_elem == ELEM_F16) return launch_q<f16>(p, kv_elem, head_dim, stream);
    return launch_q<bf16>(p, kv_elem, head_dim, stream);
}

}  // namespace gqa
