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
//     sequence's length exit at once;
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

#include <type_traits>

namespace gqa {

template <typename TQ, typename TKV, int D>
struct Decode {
    static constexpr bool KV8 = std::is_same<TKV, fp8>::value;
    static constexpr int KES = KV8 ? 1 : 2;       // K/V element bytes
    static constexpr int KT = 32;                 // keys per wave tile
    static constexpr int VROW = KT * 2 + 16;      // LDS bytes per V^T row (16-bit)
    static constexpr int WAVE_LDS = D * VROW;
    static constexpr int CH = D / 8;              // 8-element chunks per row
    static constexpr int KG = 64 / CH;            // key groups per wave for V loads
    static constexpr int KPL = KT / KG;           // keys per lane for V loads
    static constexpr int MERGE_FLOATS = D * 16 + 32;
    typedef typename Vec8<TQ>::type V8;
    typedef typename std::conditional<KV8, u32x2, u32x4>::type ChunkT;

    // position of key o (0..31) in a V^T row: lane group g of the BMM2
    // A operand then holds the keys its S^T accumulators hold.
    __device__ static int vpos(int o) { return ((o & 15) >> 2) * 8 + (o >> 4) * 4 + (o & 3); }

    __device__ static V8 to8(ChunkT c) {
        if constexpr (KV8) {
            return e4m3x8_to<TQ>(c);
        } else {
            return __builtin_bit_cast(V8, c);
        }
    }

    __device__ static void run(const AttnParams& p, char* smem) {
        const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
        const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
                if (ok) a = *(const V8*)(qrow + (ks * 32 + g * 8) * 2);
                qreg[ks] = a;
            }
        }
        const char* kbase =
            (const char*)p.k.ptr + (kv_rowbase(p, p.k, b) + (int64_t)kvh * p.k.sh) * KES;
        const char* vbase =
            (const char*)p.v.ptr + (kv_rowbase(p, p.v, b) + (int64_t)kvh * p.v.sh) * KES;
        char* sv = smem + wave * WAVE_LDS;
        const float sc = p.scale * p.k_descale * kLog2e;

        f32x4 o[D / 16];
#pragma unroll
        for (int db = 0; db < D / 16; ++db) o[db] = f32x4{};
        float m_run = -INFINITY, l_run = 0.f;

        const int vch = lane % CH, vkg = lane / CH;
        for (int j0 = k0 + wave * KT; j0 < k1; j0 += 4 * KT) {
            // ---- issue loads: K operand (2 blocks x D/32 steps), V rows
            ChunkT ka[2][D / 32];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int j = j0 + kb * 16 + l16;
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    ka[kb][ks] = ChunkT{};
                    if (j < k1)
                        ka[kb][ks] = *(const ChunkT*)(kbase + ((int64_t)j * p.k.sn + ks * 32 + g * 8) * KES);
                }
            }
            ChunkT vr[KPL];
#pragma unroll
            for (int u = 0; u < KPL; ++u) {
                const int j = j0 + vkg * KPL + u;
                vr[u] = ChunkT{};
                if (j < k1) vr[u] = *(const ChunkT*)(vbase + ((int64_t)j * p.v.sn + vch * 8) * KES);
            }
            // ---- S^T = K Q^T
            f32x4 st[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x4 acc = {};
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) acc = mfma16(to8(ka[kb][ks]), qreg[ks], acc);
                st[kb] = acc;
            }
            // ---- V^T into this wave's LDS (16-bit), runs of 4 keys
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = vch * 8 + e;
#pragma unroll
                for (int run = 0; run < KPL / 4; ++run) {
                    V8 v0 = to8(vr[run * 4 + 0]), v1 = to8(vr[run * 4 + 1]);
                    V8 v2 = to8(vr[run * 4 + 2]), v3 = to8(vr[run * 4 + 3]);
                    typedef TQ T4 __attribute__((ext_vector_type(4)));
                    T4 w;
                    w[0] = v0[e]; w[1] = v1[e]; w[2] = v2[e]; w[3] = v3[e];
                    const int key = vkg * KPL + run * 4;
                    *(T4*)(sv + d * VROW + vpos(key) * 2) = w;
                }
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
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // ---- O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < D / 16; ++db) {
                V8 a = *(const V8*)(sv + (db * 16 + l16) * VROW + g * 16);
                o[db] = mfma16(a, pb, o[db]);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }

        // ---- merge the 4 waves through LDS
        l_run += __shfl_xor(l_run, 16);
        l_run += __shfl_xor(l_run, 32);
        float* mg = (float*)(smem + 4 * WAVE_LDS) + wave * MERGE_FLOATS;
        if (g == 0) {
            mg[l16] = m_run;
            mg[16 + l16] = l_run;
        }
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) mg[32 + (db * 16 + g * 4 + r) * 16 + l16] = o[db][r];
        __syncthreads();
        const float* m0 = (const float*)(smem + 4 * WAVE_LDS);
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

template <typename TQ, typename TKV, int D>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(AttnParams p) {
    typedef Decode<TQ, TKV, D> K;
    __shared__ __attribute__((aligned(16))) char smem[4 * K::WAVE_LDS + 4 * K::MERGE_FLOATS * 4];
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
    hipLaunchKernelGGL((decode_split_kernel<TQ, TKV, D>), dim3(p.n_splits, p.hkv, p.batch),
                       dim3(256), 0, stream, p);
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
