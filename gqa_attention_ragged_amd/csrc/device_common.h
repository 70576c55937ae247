// device_common.h -- gfx950 building blocks shared by the attention kernels:
// vector types, MFMA wrappers, E4M3FN conversions and the parameter blocks
// the host passes to each kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef _Float16 f16;
typedef __bf16 bf16;
struct fp8 { uint8_t bits; };  // OCP E4M3FN storage

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- parameters
// Element strides of a [rows, heads, D] view of a Q / K / V / Y tensor: row
// (b, h, i) lives at  base + rowbase(b) + h * sh + i * sn  where rowbase is
// b * sb for the padded form and cum[b] * sn for the packed form.
struct TensorView {
    const void* ptr;
    int64_t sb, sh, sn;
};

enum MaskKind { MASK_NONE = 0, MASK_BOOL = 1, MASK_F16 = 2, MASK_BF16 = 3, MASK_F32 = 4 };

struct AttnParams {
    TensorView q, k, v;
    void* out;
    int64_t o_sb, o_sh, o_sn;
    const void* mask;
    int64_t m_sb, m_sh, m_si, m_sj;  // 0 on broadcast dimensions
    int32_t mask_kind;
    int32_t mask_vec;                 // 1 if 4-key groups of the mask are aligned & contiguous
    int32_t mask_lds;                 // 1 if mask tiles are staged through LDS (see prefill)
    const int32_t* ql;                // cumulative query lengths or null
    const int32_t* kl;                // cumulative (packed KV) / per-batch (padded) / null
    int32_t q_packed, kv_packed;
    int32_t batch, n_q, n_kv;         // n_q / n_kv: padded extents
    int32_t causal;                   // 0 none, 1 upper_left, 2 lower_right
    int32_t norm_none;                // 1: TRT_normalization_op "none"
    int32_t qdq;                      // 0 off, 1 fp8, 2 int8
    int32_t qdq_nosat;                // 1: P / qscale cannot leave the range (no clamp)
    float scale, qscale, k_descale, v_descale;
    int32_t hq, hkv, group;           // group = hq / hkv
    int32_t heads_per_wg, rows_per_wg;
    // decode split-KV
    float* part_o;                    // [B, Hq, S, D] unnormalized O of each key slice
    float* part_ml;                   // [B, Hq, S, 2]
    int32_t split_keys, n_splits;
    int32_t xcds;                     // >1: prefill workgroups remapped over this many XCDs
    int32_t mirror;                   // prefill grid of one round: second half of the
                                      // heaviest-first positions taken in reverse
    const int32_t* tree;              // draft-token parents, token-aligned with Q's rows, or null
    // paged KV: k / v are page pools [P, H_kv, 2^page_shift, D]; ptab is the
    // page table [B, 2, ptab_pages] (K pages, then V pages, per sequence)
    const int32_t* ptab;
    int32_t ptab_pages, page_shift, kv_paged;
    // persistent prefill: the work-item grid (row-tile positions x head
    // groups; key slices = n_splits) and the per-XCD claim counters (16
    // ints apart, zeroed before each launch)
    int32_t grid_x, grid_y;
    int32_t* sched;
    int32_t kv8;                      // 1: fp8 E4M3FN K / V with 16-bit Q (prefill)
    // prefill: one record of kWorkRecInts per workgroup of the attention
    // grid (linear id x + nx (y + ny z)), written by the plan kernel before
    // the launch: sequence (-1: nothing to do), row tile, q_len, kv_len,
    // q_start, kv_start, first head of the workgroup's head group, and
    // kv head | key slice << 16.  Null: every workgroup builds its own map.
    const int32_t* wrec;
};
constexpr int kWorkRecInts = 8;

// ---------------------------------------------------------------- lengths
__device__ __forceinline__ int q_len_of(const AttnParams& p, int b) {
    return p.ql ? (p.ql[b + 1] - p.ql[b]) : p.n_q;
}
__device__ __forceinline__ int kv_len_of(const AttnParams& p, int b) {
    if (p.kv_packed) return p.kl[b + 1] - p.kl[b];
    return p.kl ? p.kl[b] : p.n_kv;
}
__device__ __forceinline__ int64_t q_rowbase(const AttnParams& p, int b) {
    return p.q_packed ? (int64_t)p.ql[b] * p.q.sn : (int64_t)b * p.q.sb;
}
__device__ __forceinline__ int64_t o_rowbase(const AttnParams& p, int b) {
    return p.q_packed ? (int64_t)p.ql[b] * p.o_sn : (int64_t)b * p.o_sb;
}
__device__ __forceinline__ int64_t kv_rowbase(const AttnParams& p, const TensorView& t, int b) {
    return p.kv_packed ? (int64_t)p.kl[b] * t.sn : (int64_t)b * t.sb;
}

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 32x32x64, both operands E4M3FN, no block scaling.
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <typename T> struct Vec8;
template <> struct Vec8<f16> { typedef f16x8 type; };
template <> struct Vec8<bf16> { typedef bf16x8 type; };

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ f16 to_t(float x, f16*) { return (f16)x; }
__device__ __forceinline__ bf16 to_t(float x, bf16*) { return (bf16)x; }

// acc[i] += v[2i] + v[2i+1] for the eight 16-bit values of an operand: one
// dot-product instruction per pair against (1, 1) (the products are exact,
// the sum is formed in fp32).
__device__ __forceinline__ void add_pairs(const f16x8& v, float (&acc)[4]) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 one = {(f16)1.f, (f16)1.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const h2 pr = {v[2 * i], v[2 * i + 1]};
        acc[i] = __builtin_amdgcn_fdot2(pr, one, acc[i], false);
    }
}
__device__ __forceinline__ void add_pairs(const bf16x8& v, float (&acc)[4]) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 one = {(bf16)1.f, (bf16)1.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const b2 pr = {v[2 * i], v[2 * i + 1]};
        acc[i] = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc[i], false);
    }
}

// Round |x| <= 448 to the nearest E4M3FN code (ties to even).  The hardware
// conversion rounds to nearest-even but does not saturate, so the input is
// clamped to the format's range first (saturating reading of Q/DQ).
__device__ __forceinline__ uint32_t f32_to_e4m3_pair(float a, float b) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false) &
           0xffffu;  // the upper half (a's bits) is masked off
}
// The same without the clamp, for inputs known to be in [0, 464): values in
// [448, 464) still round to 448, only larger ones would become NaN.
__device__ __forceinline__ uint32_t f32_to_e4m3_pair_unsat(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false) &
           0xffffu;  // the upper half (a's bits) is masked off
}
// Four fp32 values -> one dword of E4M3FN codes (a, b, c, d in bytes 0..3),
// round to nearest even; SAT clamps to +-448 first (see above).  The second
// conversion writes the high half-word and keeps the low one.
template <bool SAT>
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
    if (SAT) {
        a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
        b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
        c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
        d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    }
    // The first conversion keeps the upper half of its `old` operand, which
    // the second one overwrites: passing a's own bits (dead after this) lets
    // the result reuse a's register instead of zeroing a fresh one.
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}
template <int BYTE>
__device__ __forceinline__ float e4m3_to_f32(uint32_t word) {
    return __builtin_amdgcn_cvt_f32_fp8((int)word, BYTE);
}

// Eight E4M3FN codes (two dwords) -> eight 16-bit values (exact: every
// E4M3FN value is representable in f16 and bf16), two codes per
// v_cvt_scalef32_pk_{f16,bf16}_fp8 with scale 1 (byte 2i -> element 2i).
template <bool HI>
__device__ __forceinline__ void e4m3x2_to(uint32_t w, f16& a, f16& b) {
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
    a = v[0];
    b = v[1];
}
template <bool HI>
__device__ __forceinline__ void e4m3x2_to(uint32_t w, bf16& a, bf16& b) {
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
    a = v[0];
    b = v[1];
}
template <typename T>
__device__ __forceinline__ typename Vec8<T>::type e4m3x8_to(u32x2 w) {
    typename Vec8<T>::type r;
    T x[8];
    e4m3x2_to<false>(w[0], x[0], x[1]);
    e4m3x2_to<true>(w[0], x[2], x[3]);
    e4m3x2_to<false>(w[1], x[4], x[5]);
    e4m3x2_to<true>(w[1], x[6], x[7]);
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = x[i];
    return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions across the two halves of the wave (lane l with lane l ^ 32)
// with one v_permlane32_swap: of the two registers it returns, one holds the
// lane's own value and the other its partner's, so their max / sum is the
// pair's in every lane, without a round trip through LDS.
__device__ __forceinline__ float halves_max(float v) {
    const int x = __builtin_bit_cast(int, v);
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    const int a = r[0], b = r[1];  // copy out first: bit_cast of r[i] misreads the element
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float halves_sum(float v) {
    const int x = __builtin_bit_cast(int, v);
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    const int a = r[0], b = r[1];
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// ---------------------------------------------------------------- buffer loads
// A raw buffer resource over [base, base + bytes): loads whose range falls
// outside return zero and touch no memory, so predicated tile loads need no
// branches (branch-free loads also let the compiler count outstanding loads
// exactly instead of draining them all).
// `base` and `bytes` must be the same in every lane of the wave: they are
// read from the first active lane into scalar registers, which keeps the
// descriptor scalar (the compiler would otherwise wrap each load in a loop
// over the distinct descriptors of the wave whenever it computed either value
// with vector instructions).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, (int)n,
                                             0x00020000);
}
__device__ __forceinline__ void buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4& v) {
    v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2& v) {
    v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
// 16-byte buffer store; a lane outside the descriptor's range writes nothing.
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t off, const u32x4& v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
// Bytes from a window's first row to the end of its row n-1 (0 if n <= 0),
// for windows the host has bounded below 2^32 bytes (a key tile, a split, a
// query tile).
__device__ __forceinline__ uint32_t rows_bytes(int n, int64_t row_stride, int d, int es) {
    return n > 0 ? (uint32_t)(((int64_t)(n - 1) * row_stride + d) * es) : 0u;
}
// The same in 64 bits, for a whole sequence's rows (may exceed 4 GiB).
__device__ __forceinline__ int64_t rows_bytes64(int n, int64_t row_stride, int d, int es) {
    return n > 0 ? ((int64_t)(n - 1) * row_stride + d) * es : 0;
}
// A buffer range of `rem` bytes, clamped into the 32-bit range field (the
// loads through such a window stay within its first 2^32 - 1 bytes).
__device__ __forceinline__ uint32_t clamp_range(int64_t rem) {
    return rem <= 0 ? 0u : rem >= 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)rem;
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace gqa
