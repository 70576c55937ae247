// prefill_impl.h -- fused ragged GQA attention for query tiles (prefill, chunked
// context, and any query length), gfx950.
//
// Computes, per valid query row, BMM1 -> causal / length / mask predicate ->
// normalization (softmax or none) -> optional quantize-dequantize of the
// normalized scores -> BMM2, as the onnx-tensorrt "TensorRT Custom Operator
// Schemas" page defines TRT_Attention and TRT_QuantizedAttention.
//
// Work decomposition
//   * A workgroup is 4 waves.  Each wave owns 32 query rows of one query
//     head.  The waves of a workgroup share one KV head: with group size
//     G = H_q / H_kv they cover HW = gcd(G, 4) heads of the same KV group and
//     4 / HW blocks of 32 rows, so every K/V tile staged in LDS feeds 4 waves.
//   * blockIdx.x enumerates query-row tiles over the whole ragged batch
//     (sum_b ceil(q_len_b / rows_per_wg)); the tile -> (b, tile) map is
//     rebuilt on the device from the cumulative lengths, so the host never
//     reads device memory.  blockIdx.y enumerates head groups, blockIdx.z
//     key slices (split-KV).  When the head groups divide evenly over the
//     XCDs, workgroup ids are remapped so that each XCD works through whole
//     head groups (K/V cached in one L2).
//   * The key loop streams 64-key tiles through double-buffered LDS, copied
//     by buffer loads that write LDS directly: K row-major with padded rows,
//     V row-major with XOR-swizzled 16-byte units, read as the BMM2 operand
//     with the gfx950 LDS transpose loads.
//   * Scores are computed transposed, S^T = K Q^T, with 32x32 MFMA tiles, so
//     each lane owns one query row (lane % 32) and 16 of every 32 keys; the
//     row max / sum need one exchange with lane ^ 32 only.  O is likewise
//     accumulated transposed, O^T = V^T P^T.
//   * Softmax runs online in the exp2 domain (scale * log2 e folded into the
//     score scale), the published online-normalizer method (Milakov &
//     Gimelshein 2018, as used by FlashAttention-2).  With Q/DQ the
//     normalized P needs the final row max and sum, so a first pass over the
//     keys computes them and a second pass quantizes exactly.
//   * Padding is never read (loads are predicated on the valid lengths) and
//     output rows are only written when they are valid.
#pragma once
#include "device_common.h"
#include "launch.h"
#include "main_timer.h"
#include "tile_common.h"

#include <type_traits>

namespace gqa {

template <typename TI, int D>
struct Cfg {
    static constexpr bool FP8 = std::is_same<TI, fp8>::value;
    static constexpr int ES = FP8 ? 1 : 2;          // element bytes
    static constexpr int BN = 64;                   // keys per tile
    static constexpr int KROW = D * ES + 16;        // LDS bytes per K row (padded)
    static constexpr int VROW = D * ES;             // LDS bytes per V row (row-major, swizzled)
    static constexpr int KBYTES = BN * KROW;
    static constexpr int VBYTES = BN * VROW;
    static constexpr int STAGE = KBYTES + VBYTES;
    // K / V tiles are copied HBM -> LDS by buffer loads that write LDS
    // directly, 1 KiB (64 lanes x 16 bytes, contiguous) per instruction; the
    // 4 waves take the instructions of a tile round-robin.
    static constexpr int NKD = KBYTES / 1024;       // instructions per K tile
    static constexpr int NVD = VBYTES / 1024;       // instructions per V tile
    static constexpr int KMAX = (NKD + 3) / 4;      // per wave, at most
    static constexpr int VMAX = (NVD + 3) / 4;
    static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0, "tiles copy in whole KiB");
    static constexpr int QSTEPS = FP8 ? D / 64 : D / 16;  // BMM1 k-steps
    static constexpr int VUNITS = VROW / 16;        // 16-byte units per V row
    static constexpr int RPL = VROW >= 256 ? 1 : 256 / VROW;  // V rows per 256-byte bank line
    // Staged mask tile: 32 query rows x BN keys of a 1- or 2-byte mask
    // (row stride padded by 16 bytes against bank conflicts).
    static constexpr int MROW = BN * 2 + 16;
    static constexpr int MBYTES = 32 * MROW;
    // Q rows (input type) and O rows (16-bit output) as 16-byte chunks; one
    // 1 KiB copy instruction moves QRPI (ORPI) rows, 32 rows take QINS (OINS).
    static constexpr int QROW = D * ES, QCH = QROW / 16, QRPI = 64 / QCH, QINS = 32 / QRPI;
    static constexpr int OROW = D * 2, OCH = OROW / 16, ORPI = 64 / OCH, OINS = 32 / ORPI;
};

// Element e of an 8-element chunk, as raw bits.
__device__ __forceinline__ uint32_t chunk_elem(u32x4 c, int e) {
    return (c[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
}
__device__ __forceinline__ uint32_t chunk_elem(u32x2 c, int e) {
    return (c[e >> 2] >> ((e & 3) * 8)) & 0xffu;
}

// ------------------------------------------------------------------ mask
struct MaskGroup {
    float add[4];
    bool ok[4];
};

__device__ __forceinline__ float mask_scalar(const AttnParams& p, const char* row, int64_t j) {
    switch (p.mask_kind) {
    case MASK_BOOL: return ((const uint8_t*)row)[j * p.m_sj] ? 1.f : 0.f;
    case MASK_F16: return (float)((const f16*)row)[j * p.m_sj];
    case MASK_BF16: return (float)((const bf16*)row)[j * p.m_sj];
    default: return ((const float*)row)[j * p.m_sj];
    }
}

// Mask values for keys jg..jg+3 of one row; keys >= kv_len are not read.
__device__ __forceinline__ MaskGroup load_mask_group(const AttnParams& p, const char* row, int jg,
                                                     int kv_len) {
    MaskGroup m;
    const bool is_bool = p.mask_kind == MASK_BOOL;
    if (p.mask_vec && jg + 3 < kv_len) {
        if (is_bool) {
            uint32_t w = *(const uint32_t*)(row + (int64_t)jg);
#pragma unroll
            for (int u = 0; u < 4; ++u) { m.ok[u] = (w >> (8 * u)) & 0xff; m.add[u] = 0.f; }
        } else if (p.mask_kind == MASK_F32) {
            f32x4 w = *(const f32x4*)(row + (int64_t)jg * 4);
#pragma unroll
            for (int u = 0; u < 4; ++u) { m.add[u] = w[u]; m.ok[u] = true; }
        } else {
            u32x2 w = *(const u32x2*)(row + (int64_t)jg * 2);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                uint32_t h = (w[u >> 1] >> ((u & 1) * 16)) & 0xffffu;
                if (p.mask_kind == MASK_F16) {
                    m.add[u] = (float)__builtin_bit_cast(f16, (uint16_t)h);
                } else {
                    m.add[u] = __builtin_bit_cast(float, h << 16);
                }
                m.ok[u] = true;
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            m.add[u] = 0.f;
            m.ok[u] = false;
            if (jg + u < kv_len) {
                float x = mask_scalar(p, row, jg + u);
                if (is_bool) m.ok[u] = x != 0.f;
                else { m.add[u] = x; m.ok[u] = true; }
            }
        }
    }
    return m;
}

// ------------------------------------------------------------------ kernel
enum PassKind { PASS_STATS = 0, PASS_ONLINE = 1, PASS_FIXED = 2, PASS_NONE = 3 };
// Kernel modes: online softmax; softmax with Q/DQ of P (two passes);
// "none" normalization (with or without Q/DQ).
enum Mode { MODE_SOFTMAX = 0, MODE_SOFTMAX_QDQ = 1, MODE_NONE = 2, MODE_SOFTMAX_QDQ_NS = 3 };
constexpr float kLazyRescale = 8.0f;  // log2 units
// s_waitcnt immediate: vmcnt(0), expcnt / lgkmcnt not waited on.
constexpr int kWaitVmcnt0 = 0x0F70;
// s_waitcnt immediate: lgkmcnt(0) (LDS), vmcnt / expcnt not waited on.
constexpr int kWaitLgkmcnt0 = 0xC07F;

// Mask variants of the general kernel: none; read per lane from global memory
// (any kind and layout); staged through LDS as 16-bit additive values -- f16
// (an f16 mask, or a bool mask converted to 0 / -inf while staging) or bf16;
// no mask but tree decoding; staged bool masks in the fp8 kernels, whose
// mask type is then known at compile time (fewer registers: three
// workgroups per CU).  The tree rule is compiled only into the generic and
// tree variants (a tree with a mask takes the generic one).
enum MaskVariant { MK_NONE = 0, MK_GENERIC = 1, MK_LDS16 = 2, MK_LDS_BF16 = 3, MK_TREE = 4,
                   MK_LDS_BOOL = 5 };

template <typename TI, int D, int MK, bool PAGED = false, bool KV8 = false>
struct Prefill {
    static constexpr bool HAS_MASK = MK != MK_NONE && MK != MK_TREE;
    static constexpr bool TREE = MK == MK_GENERIC || MK == MK_TREE;  // tree rule compiled in
    static constexpr bool STAGED = MK == MK_LDS16 || MK == MK_LDS_BF16 || MK == MK_LDS_BOOL;
    typedef Cfg<TI, D> C;
    // MFMA element type: the input type for 16-bit inputs; E4M3FN codes for fp8.
    typedef typename std::conditional<C::FP8, f16, TI>::type T16;
    typedef typename std::conditional<C::FP8, f16, TI>::type TO;  // output element

    typedef typename Vec8<T16>::type V8;
    // fp8 kernels stage the mask tile as fp32 raw-score biases (0 / -inf for
    // bool masks, value * log2 e / scale for additive ones) that initialize
    // the BMM1 accumulators, so the mask costs no vector instruction per
    // score; 16-bit kernels (whose LDS holds only 16-bit values for two
    // workgroups per CU) stage the 16-bit values and add them per score.
    static constexpr bool MACC = STAGED && C::FP8;
    static_assert(MK != MK_LDS_BOOL || C::FP8, "compile-time bool staging: fp8 kernels");
    static constexpr int MROW = MACC ? C::BN * 4 + 16 : C::MROW;
    static constexpr int MBYTES = 32 * MROW;
    // Bytes per pipeline stage: K tile, V tile and (mask kernels) a mask tile.
    static constexpr int SSTAGE = C::STAGE + (HAS_MASK ? MBYTES : 0);
    // When a tile's copy instructions do not divide evenly over the 4 waves,
    // the waves without a last instruction skip it (a wave-uniform branch:
    // every wait for the copies is a wait for all of the wave's loads).
    // fp8 KV cache with 16-bit Q (KV8): K / V tiles are copied as E4M3FN codes
    // in unpadded rows of D bytes into small stages (an even number of 1 KiB
    // copies per wave: no spare) and converted once per tile, by the whole
    // workgroup, into the 16-bit tile (`t16`, layout of a 16-bit stage) that
    // the products read.  E4M3FN values are exact in f16 and bf16.
    static_assert(!KV8 || !C::FP8, "KV8: 16-bit Q");
    static constexpr int KES = KV8 ? 1 : C::ES;  // K / V bytes per element in memory
    static constexpr int K8BYTES = C::BN * D, V8BYTES = C::BN * D;
    static constexpr int STAGE8 = K8BYTES + V8BYTES;
    static constexpr int K8PW = K8BYTES / 4096, V8PW = V8BYTES / 4096;  // copies per wave
    static_assert(K8BYTES % 4096 == 0 && K8PW <= C::KMAX && V8PW <= C::VMAX, "KV8 copies");
    // Q / O tiles staged through LDS, row-major with XOR-swizzled 16-byte
    // chunks (chunk c of row r at c ^ (r mod chunks per row)) so that the
    // 32 rows of an operand read spread over the banks.  Each wave stages
    // 32 rows: Q in stage 1 (4 x 32 Q rows), O in stages 0 and 1 (2 waves
    // each).
    static_assert(4 * 32 * C::QROW <= SSTAGE && 2 * 32 * C::OROW <= SSTAGE, "Q / O staging fits");
    __device__ __forceinline__ static int q_swz(int row) { return row & (C::QCH - 1); }
    __device__ __forceinline__ static int o_swz(int row) { return row & (C::OCH - 1); }
    // BMM1 B operand held in registers for the whole kernel: 8 x 16-bit
    // values per k-step, or 32 E4M3FN codes per k-step.
    typedef typename std::conditional<C::FP8, i32x8, V8>::type QOp;
    typedef QOp QRegs[C::QSTEPS];
    typedef f32x16 ORegs[D / 32];

    // Per-workgroup state shared by the passes.
    struct Ctx {
        int b, q_len, kv_len, diag;
        int t0, t1;           // key tiles [t0, t1) of this workgroup
        bool causal;
        int wr0;              // first row of this wave
        bool wave_rows;       // wave has at least one valid row
        int wave_kv_end;      // keys this wave can see (causal)
        const char* kbase;    // K rows of (b, kv head)
        const char* vbase;
        int64_t kbytes, vbytes;         // bytes from row 0 to the end of the last valid key
        int64_t ktile, vtile;           // bytes per tile of BN keys
        uint32_t koff[C::KMAX], voff[C::VMAX];  // this lane's source offsets inside a tile
        const char* mrow;     // mask row of this lane's query row (or null)
        const char* mtile;    // staged mask: the workgroup's first mask row
        int64_t mvalid;       // staged mask: bytes up to the last valid (row, key)
        uint32_t moff;        // staged mask: this thread's load offset in a tile
        int mrow_l, mchunk;   // staged mask: this thread's (row, 16-byte chunk); row < 0: idle
        bool mbool;           // staged mask: bool source (converted to f16 0 / -inf)
        int i;                // this lane's query row
        bool tree;            // tree decoding: the last q_len keys are draft tokens
        int tbase;            // key of draft 0 (kv_len - q_len)
        // drafts on this row's ancestor chain, itself included: bit t % 32 of
        // word t / 32 is draft t (four words, no arrays: a lane-dependent
        // array index would put the context in scratch memory)
        uint32_t anc0, anc1, anc2, anc3;
        bool tree_over;       // row beyond the drafts this build resolves: its output is NaN
    };

    // Staged bool mask?  Known at compile time in the fp8 kernels (bool masks
    // take MK_LDS_BOOL there), a flag of the call in the 16-bit ones.
    __device__ __forceinline__ static bool mask_is_bool(const Ctx& c) {
        return MACC ? MK == MK_LDS_BOOL : c.mbool;
    }

    // Drafts per sequence whose ancestor chains the tree variants resolve
    // (two per lane).
    static constexpr int kMaxDrafts = 128;

    // Tree rule for draft t (key tbase + t) of this lane's row: the row's own
    // draft and its ancestors.
    // Both halves are read and the bit is picked arithmetically: a select
    // between two fields of the context would become a load through a
    // selected pointer, which keeps the whole context in scratch memory.
    __device__ __forceinline__ static bool tree_ok(const Ctx& c, int t) {
        const uint64_t lo = ((uint64_t)c.anc1 << 32) | c.anc0;
        const uint64_t hi = ((uint64_t)c.anc3 << 32) | c.anc2;
        const uint32_t sh = (uint32_t)t & 63u;
        const uint64_t b = ((lo >> sh) & (uint64_t)(t < 64)) |
                           ((hi >> sh) & (uint64_t)(t >= 64 && t < kMaxDrafts));
        return (b & 1u) != 0;
    }

    // Rows past the drafts the tree variants resolve output NaN: the result
    // is visibly undefined rather than computed by another rule.
    __device__ __forceinline__ static void poison_over(const Ctx& c, ORegs& o) {
        if constexpr (TREE) {
            if (c.tree_over) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[db][r] = __builtin_nanf("");
            }
        }
    }

    // A buffer window starting at tile `tile`: the wave-uniform base moves
    // with the tile (64-bit scalar arithmetic, so a sequence's rows may span
    // more than 4 GiB) and the range ends with the last valid key, so keys
    // >= kv_len read as zero and touch no memory.  One tile's loads reach at
    // most BN rows past the base (the host bounds that below 2^32 bytes).
    __device__ __forceinline__ static __amdgpu_buffer_rsrc_t window(const char* base,
                                                                    int64_t valid,
                                                                    int64_t stride, int tile) {
        const int64_t off = (int64_t)tile * stride;
        return make_rsrc(base + off, clamp_range(valid - off));
    }

    __device__ __forceinline__ static void load_mask(const AttnParams& p, const Ctx& c, int tile,
                                                     u32x4& rm) {
        const int es = p.mask_kind == MASK_BOOL ? 1 : 2;
        const int64_t off = (int64_t)tile * (C::BN * es);
        const __amdgpu_buffer_rsrc_t mr = make_rsrc(c.mtile + off, clamp_range(c.mvalid - off));
        if (MACC && mask_is_bool(c)) {
            u32x2 v;  // fp8 kernels stage bool masks in 8-byte chunks
            buf_load(mr, c.moff, v);
            rm[0] = v[0];
            rm[1] = v[1];
        } else {
            buf_load(mr, c.moff, rm);
        }
    }
    // Staged rows hold 16-bit additive values; a bool chunk (16 keys) becomes
    // 16 f16 values, 0 (may attend) or -inf.  fp8 kernels (MACC) store fp32
    // raw-score biases instead: 0 / -inf, or the additive value times kadd.
    __device__ __forceinline__ static void store_mask(char* stage, const Ctx& c, const u32x4& rm,
                                                      float kadd) {
        if (c.mrow_l < 0) return;
        char* row = stage + C::STAGE + c.mrow_l * MROW;
        if constexpr (MACC) {
            if (mask_is_bool(c)) {
                // 8 keys: byte b -> bias (b - 1) & 0xFF800000, i.e. -inf for
                // a zero byte and +0 for any other (b - 1 < 2^23)
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    const uint32_t x = rm[w];
                    f32x4 f;
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        f[u] = __builtin_bit_cast(float, (((x >> (8 * u)) & 0xffu) - 1u) & 0xFF800000u);
                    *(f32x4*)(row + c.mchunk * 32 + w * 16) = f;
                }
            } else {
#pragma unroll
                for (int w = 0; w < 4; w += 2) {
                    f32x4 f;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint32_t x = rm[w + (u >> 1)];
                        f[u] = staged_add((x >> ((u & 1) * 16)) & 0xffffu) * kadd;
                    }
                    *(f32x4*)(row + c.mchunk * 32 + w * 8) = f;
                }
            }
            return;
        }
        if (c.mbool) {
            u32x4 h[2];
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const uint32_t b0 = (rm[w] >> (16 * half)) & 0xffu;
                    const uint32_t b1 = (rm[w] >> (16 * half + 8)) & 0xffu;
                    h[w >> 1][(w & 1) * 2 + half] = (b0 ? 0u : 0xFC00u) | (b1 ? 0u : 0xFC000000u);
                }
            *(u32x4*)(row + c.mchunk * 32) = h[0];
            *(u32x4*)(row + c.mchunk * 32 + 16) = h[1];
        } else {
            *(u32x4*)(row + c.mchunk * 16) = rm;
        }
    }

    // One staged additive mask value as float.
    __device__ __forceinline__ static float staged_add(uint32_t h16) {
        if constexpr (MK == MK_LDS_BF16) return __builtin_bit_cast(float, h16 << 16);
        else return (float)__builtin_bit_cast(f16, (uint16_t)h16);
    }

    // Softmax on raw scores (scale > 0): the staged additive mask enters the
    // raw domain as s + add / scale', so that exp2(s' * sc) carries
    // add * log2 e; -inf removes the key.  kadd = log2 e / sc.
    __device__ __forceinline__ static void apply_mask_raw(f32x16 (&s)[2], const char* stage,
                                                          float kadd) {
        const int lane = threadIdx.x & 63, lg = lane >> 5;
        const char* src = stage + C::STAGE + (lane & 31) * MROW;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const u32x2 w = *(const u32x2*)(src + (kb * 32 + rq * 8 + lg * 4) * 2);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t h16 = (w[u >> 1] >> ((u & 1) * 16)) & 0xffffu;
                    s[kb][rq * 4 + u] = __builtin_fmaf(staged_add(h16), kadd, s[kb][rq * 4 + u]);
                }
            }
    }

    // Start the copy of tile `tile` (K, and V when with_v) into `stage`:
    // instruction j of the tile writes LDS bytes [j KiB, j KiB + 1 KiB) of the
    // K (V) region, lane i the 16 bytes at i * 16, read from the source offset
    // the lane was given for that position (padding lanes of K get an offset
    // beyond the range: zeros, no memory access).  Completion is waited for
    // with vmcnt before the barrier that publishes the stage.
    __device__ __forceinline__ static void dma_tile(const AttnParams& p, const Ctx& c, int tile,
                                                    bool with_v, char* stage, int wave) {
        __amdgpu_buffer_rsrc_t kr, vr;
        if constexpr (PAGED) {
            // the tile lies inside one page (pages hold a power of two >= BN
            // keys): its base comes from the page table, its range ends
            // with the sequence's last valid key
            const int row0 = tile * C::BN;
            const int pi = row0 >> p.page_shift;
            const int within = row0 & ((1 << p.page_shift) - 1);
            const uint32_t valid = rows_bytes(min(C::BN, c.kv_len - row0), p.k.sn, D, KES);
            const int32_t* pt = p.ptab + (int64_t)c.b * 2 * p.ptab_pages + pi;
            kr = make_rsrc(c.kbase + ((int64_t)pt[0] * p.k.sb + (int64_t)within * p.k.sn) * KES,
                           valid);
            vr = make_rsrc(c.vbase + ((int64_t)pt[p.ptab_pages] * p.v.sb +
                                      (int64_t)within * p.v.sn) * KES,
                           rows_bytes(min(C::BN, c.kv_len - row0), p.v.sn, D, KES));
        } else {
            kr = window(c.kbase, c.kbytes, c.ktile, tile);
            vr = window(c.vbase, c.vbytes, c.vtile, tile);
        }
        if constexpr (KV8) {
#pragma unroll
            for (int k = 0; k < K8PW; ++k)
                buf_load_lds16_async<PAGED>(kr, stage + (wave + 4 * k) * 1024, c.koff[k]);
            if (!with_v) return;
#pragma unroll
            for (int k = 0; k < V8PW; ++k)
                buf_load_lds16_async<PAGED>(vr, stage + K8BYTES + (wave + 4 * k) * 1024, c.voff[k]);
            return;
        }
#pragma unroll
        for (int k = 0; k < C::KMAX; ++k) {
            const int j = wave + 4 * k;
            if (4 * (k + 1) <= C::NKD || j < C::NKD)
                buf_load_lds16_async<PAGED>(kr, stage + j * 1024, c.koff[k]);
        }
        if (!with_v) return;
#pragma unroll
        for (int k = 0; k < C::VMAX; ++k) {
            const int j = wave + 4 * k;
            if (4 * (k + 1) <= C::NVD || j < C::NVD)
                buf_load_lds16_async<PAGED>(vr, stage + C::KBYTES + j * 1024, c.voff[k]);
        }
    }

    // KV8: the fp8 tile in `s8` (K then V, rows of D codes) into the 16-bit
    // tile `t16` (K rows padded, V rows with XOR-swizzled 16-byte units, as a
    // 16-bit stage): every thread converts 8-code chunks of whole rows.
    __device__ __forceinline__ static void convert_tile(const char* s8, char* t16) {
        constexpr int CPR = D / 8, NCH = C::BN * CPR;
        static_assert(NCH % 256 == 0, "chunks divide over the workgroup");
#pragma unroll
        for (int k = 0; k < NCH / 256; ++k) {
            const int i = (int)threadIdx.x + 256 * k, row = i / CPR, c8 = i % CPR;
            const u32x2 kw = *(const u32x2*)(s8 + row * D + c8 * 8);
            const u32x2 vw = *(const u32x2*)(s8 + K8BYTES + row * D + c8 * 8);
            *(V8*)(t16 + row * C::KROW + c8 * 16) = e4m3x8_to<T16>(kw);
            *(V8*)(t16 + C::KBYTES + row * C::VROW + ((c8 ^ v_swz<C>(row)) << 4)) = e4m3x8_to<T16>(vw);
        }
    }
    // Workgroup barrier after LDS writes that leaves the tile copies in flight.
    __device__ __forceinline__ static void lds_barrier() {
        __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    }

    // S^T tile (64 keys x 32 rows) for this wave from the staged K tile.  The
    // two 32-key blocks accumulate in alternation so that consecutive MFMAs
    // never wait on each other's result.
    __device__ __forceinline__ static void bmm1(const char* sK, const QRegs& qreg, f32x16 (&s)[2]) {
        const int lane = threadIdx.x & 63, lr = lane & 31, lg = lane >> 5;
        if constexpr (MACC) {
            // the staged raw-score biases of this lane's (row, keys)
            const char* mb = sK + C::STAGE + lr * MROW;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const f32x4 v = *(const f32x4*)(mb + (kb * 32 + rq * 8 + lg * 4) * 4);
#pragma unroll
                    for (int u = 0; u < 4; ++u) s[kb][rq * 4 + u] = v[u];
                }
        } else {
            s[0] = f32x16{};
            s[1] = f32x16{};
        }
        const char* row0 = sK + lr * C::KROW;
        const char* row1 = sK + (32 + lr) * C::KROW;
        if constexpr (C::FP8) {
            auto kop = [&](int ks, int kb) {
                const char* row = kb ? row1 : row0;
                const u32x4 lo = *(const u32x4*)(row + ks * 64 + lg * 32);
                const u32x4 hi = *(const u32x4*)(row + ks * 64 + lg * 32 + 16);
                i32x8 a;
                a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
                a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
                return a;
            };
            if constexpr (MACC) {
                // Staged biases occupy the accumulators before the MFMAs:
                // the two K operands of one 64-byte k-step at a time, the
                // next k-step's reads issued behind the current two MFMAs
                // (128 cycles of matrix work cover their latency) into the
                // same registers, 16 VGPRs fewer than reading the whole tile
                // first (sched_barrier keeps the order).
                i32x8 a0 = kop(0, 0), a1 = kop(0, 1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < C::QSTEPS; ++ks) {
                    s[0] = mfma32_fp8(a0, qreg[ks], s[0]);
                    s[1] = mfma32_fp8(a1, qreg[ks], s[1]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (ks + 1 < C::QSTEPS) {
                        a0 = kop(ks + 1, 0);
                        a1 = kop(ks + 1, 1);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            } else {
                // every K operand of the tile read before the first MFMA,
                // which then waits for its own reads only
                i32x8 a[C::QSTEPS][2];
#pragma unroll
                for (int ks = 0; ks < C::QSTEPS; ++ks) {
                    a[ks][0] = kop(ks, 0);
                    a[ks][1] = kop(ks, 1);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < C::QSTEPS; ++ks) {
                    s[0] = mfma32_fp8(a[ks][0], qreg[ks], s[0]);
                    s[1] = mfma32_fp8(a[ks][1], qreg[ks], s[1]);
                }
            }
        } else {
            // Explicit software pipeline (the source order is the
            // instruction order: sched_barrier keeps the scheduler from
            // sinking each operand read to its MFMA, which exposed the LDS
            // latency on every MFMA): the K operands of k-step ks + LA are
            // read while k-step ks's two MFMAs run.
            constexpr int KS = C::QSTEPS, LA = 2;
            V8 ka[LA + 1][2];
#pragma unroll
            for (int ks = 0; ks < LA; ++ks) {
                ka[ks][0] = *(const V8*)(row0 + (ks * 16 + lg * 8) * 2);
                ka[ks][1] = *(const V8*)(row1 + (ks * 16 + lg * 8) * 2);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + LA < KS) {
                    const int n = ks + LA;
                    ka[n % (LA + 1)][0] = *(const V8*)(row0 + (n * 16 + lg * 8) * 2);
                    ka[n % (LA + 1)][1] = *(const V8*)(row1 + (n * 16 + lg * 8) * 2);
                }
                s[0] = mfma32(ka[ks % (LA + 1)][0], qreg[ks], s[0]);
                s[1] = mfma32(ka[ks % (LA + 1)][1], qreg[ks], s[1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // Whether the tile is fully allowed by the lengths and the causal rule
    // (the mask aside) for every row of this wave.
    __device__ __forceinline__ static bool cl_full(const AttnParams& p, const Ctx& c, int tile) {
        const int j0 = tile * C::BN;
        return j0 + C::BN <= c.kv_len && c.wr0 + 32 <= c.q_len &&
               !(p.causal && j0 + C::BN - 1 > c.wr0 + c.diag) &&
               !(TREE && c.tree && j0 + C::BN > c.tbase);
    }

    // Mask-free kernels: mark the keys a row may not see with -inf and keep
    // the other raw scores (the scale is applied inside the exp2 argument).
    // Key j of this lane's row is allowed iff j < lim, one compare per score.
    __device__ __forceinline__ static void predicate_raw(const Ctx& c, int tile, f32x16 (&s)[2]) {
        const int lane = threadIdx.x & 63, lg = lane >> 5;
        int lim = c.i < c.q_len ? c.kv_len : 0;
        if (c.causal) lim = min(lim, c.i + c.diag + 1);
        const int rel = lim - (tile * C::BN + lg * 4);  // key offset limit for this lane
        if (TREE && c.tree) {
            const int t0 = tile * C::BN + lg * 4 - c.tbase;  // draft index of offset 0
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
                    const bool ok = off < rel && (t0 + off < 0 || tree_ok(c, t0 + off));
                    s[kb][r] = ok ? s[kb][r] : -INFINITY;
                }
            return;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
                s[kb][r] = off < rel ? s[kb][r] : -INFINITY;
            }
    }

    // Scale the raw scores and apply the causal / length / mask predicate.
    // Disallowed entries become -inf (softmax) or 0 (none).
    __device__ __forceinline__ static void predicate(const AttnParams& p, const Ctx& c, int tile,
                                                     f32x16 (&s)[2], float sc, float ac,
                                                     bool none_norm, const char* stage) {
        const int lane = threadIdx.x & 63, lg = lane >> 5;
        const int j0 = tile * C::BN;
        const bool row_ok = c.i < c.q_len;
        const float off = none_norm ? 0.f : -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int jg = j0 + kb * 32 + rq * 8 + lg * 4;
                MaskGroup mg;
                if constexpr (MACC) {
                    // the bias is in the scores already; -inf marks a removed key
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        mg.add[u] = s[kb][rq * 4 + u] == -INFINITY ? -INFINITY : 0.f;
                        mg.ok[u] = true;
                    }
                } else if constexpr (STAGED) {
                    // staged tile: row = this lane's row within the 32-row tile
                    const char* src = stage + C::STAGE + (lane & 31) * MROW;
                    const int ko = kb * 32 + rq * 8 + lg * 4;
                    const u32x2 w = *(const u32x2*)(src + ko * 2);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        mg.add[u] = staged_add((w[u >> 1] >> ((u & 1) * 16)) & 0xffffu);
                        mg.ok[u] = true;
                    }
                } else if (HAS_MASK && row_ok) {
                    mg = load_mask_group(p, c.mrow, jg, c.kv_len);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) { mg.add[u] = 0.f; mg.ok[u] = true; }
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int j = jg + u;
                    const int r = rq * 4 + u;
                    bool a = row_ok && j < c.kv_len && (p.causal == 0 || j <= c.i + c.diag);
                    if (TREE && c.tree && j >= c.tbase) a = a && tree_ok(c, j - c.tbase);
                    float v = s[kb][r] * sc;
                    if (MK == MK_GENERIC && p.mask_kind == MASK_BOOL) {
                        a = a && mg.ok[u];
                    } else if (HAS_MASK) {
                        a = a && !(__builtin_isinf(mg.add[u]) && mg.add[u] < 0.f);
                        v += mg.add[u] * ac;
                    }
                    s[kb][r] = a ? v : off;
                }
            }
        }
    }

    // BMM2 A operand for k-step ks (16 keys) and d-block db (32 values of d):
    // lane (d = db*32 + lane%32, g = lane/32) gets keys
    // ks*16 + (e/4)*8 + g*4 + e%4 for e = 0..7 -- the keys whose
    // probabilities the same lane holds in its S^T accumulator.
    __device__ __forceinline__ static V8 v_operand(const char* sV, int ks, int db) {
        const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 5, dh = (lane >> 4) & 1;
        const int d = db * 32 + dh * 16 + 4 * (l16 & 3);
        const int key = ks * 16 + g * 4 + (l16 >> 2);
        const u32x2 lo = tr16(sV + v_addr<C>(key, d));
        const u32x2 hi = tr16(sV + v_addr<C>(key + 8, d));
        u32x4 w;
        w[0] = lo[0]; w[1] = lo[1]; w[2] = hi[0]; w[3] = hi[1];
        return __builtin_bit_cast(V8, w);
    }

    // P^T of one tile as the four 16-bit BMM2 B operands (one per 16-key
    // k-step): lane (row, group g) holds keys ks*16 + (e/4)*8 + g*4 + e%4.
    __device__ __forceinline__ static void p_operands(const f32x16 (&pv)[2], V8 (&b)[4]) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) b[ks][e] = to_t(pv[ks >> 1][(ks & 1) * 8 + e], (T16*)nullptr);
    }

    // 16-bit BMM2: O^T += V^T P^T over one 64-key tile, as an explicit
    // software pipeline (source order = instruction order): each V operand
    // (two transpose reads) is read LA MFMAs ahead of its use.
    __device__ __forceinline__ static void bmm2_ops(const char* sV, const V8 (&b)[4], ORegs& o) {
        constexpr int DB = D / 32, NC = 4 * DB, LA = 3;
        V8 va[LA + 1];
#pragma unroll
        for (int i = 0; i < LA; ++i) va[i] = v_operand(sV, i / DB, i % DB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            if (i + LA < NC) va[(i + LA) % (LA + 1)] = v_operand(sV, (i + LA) / DB, (i + LA) % DB);
            o[i % DB] = mfma32(va[i % (LA + 1)], b[i / DB], o[i % DB]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __device__ __forceinline__ static void bmm2_16(const char* sV, const f32x16 (&pv)[2], ORegs& o) {
        V8 b[4];
        p_operands(pv, b);
        bmm2_ops(sV, b, o);
    }

    // "none" normalization keeps unbounded scores: split each into a 16-bit
    // high part and a 16-bit remainder so BMM2 keeps ~fp32 accuracy.
    __device__ __forceinline__ static void bmm2_16_split(const char* sV, const f32x16 (&pv)[2], ORegs& o) {
        const int lane = threadIdx.x & 63, lr = lane & 31, lg = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            V8 bh, bl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = pv[ks >> 1][(ks & 1) * 8 + e];
                T16 h = to_t(x, (T16*)nullptr);
                bh[e] = h;
                bl[e] = to_t(x - (float)h, (T16*)nullptr);
            }
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const V8 a = v_operand(sV, ks, db);
                o[db] = mfma32(a, bh, o[db]);
                o[db] = mfma32(a, bl, o[db]);
            }
        }
    }

    // fp8 BMM2: P' codes (E4M3FN) against V^T codes, one 64-key k-step.
    // fp8 BMM2 A operand for d-block db: four 8-key transpose reads; read t
    // holds keys key(t, g, k).
    __device__ __forceinline__ static i32x8 v_operand_fp8(const char* sV, int db) {
        const int lane = threadIdx.x & 63, lg = lane >> 5;
        const int l16 = lane & 15, dh = (lane >> 4) & 1, k = l16 >> 1;
        const int d = db * 32 + dh * 16 + 8 * (l16 & 1);
        i32x8 a;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int key = (t >> 1) * 32 + ((t & 1) * 2 + (k >> 2)) * 8 + lg * 4 + (k & 3);
            const u32x2 w = tr8(sV + v_addr<C>(key, d));
            a[2 * t] = (int)w[0];
            a[2 * t + 1] = (int)w[1];
        }
        return a;
    }
    // fp8 BMM2 over the tile's one 64-key k-step, each d-block's operand
    // read LA MFMAs ahead of its use (source order = instruction order).
    __device__ __forceinline__ static void bmm2_fp8(const char* sV, const i32x8& codes, ORegs& o) {
        constexpr int DB = D / 32, LA = DB > 2 ? 2 : 1;
        i32x8 va[LA + 1];
#pragma unroll
        for (int i = 0; i < LA; ++i) va[i] = v_operand_fp8(sV, i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            if (db + LA < DB) va[(db + LA) % (LA + 1)] = v_operand_fp8(sV, db + LA);
            o[db] = mfma32_fp8(va[db % (LA + 1)], codes, o[db]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Quantize x (= P / qscale) and return the dequantized code value
    // (without the qscale factor, which the epilogue applies).
    template <bool SAT = true>
    __device__ __forceinline__ static float qdq_value(float x, int kind) {
        if (kind == 1) {
            uint32_t code = SAT ? f32_to_e4m3_pair(x, 0.f) : f32_to_e4m3_pair_unsat(x, 0.f);
            return e4m3_to_f32<0>(code);
        }
        float r = __builtin_rintf(x);
        return SAT ? __builtin_amdgcn_fmed3f(r, -128.f, 127.f) : r;
    }

    // One sweep over the key tiles of this workgroup.
    // SAT: the quantized scores may exceed the format's range and are
    // saturated; without it the caller guarantees x = P / qscale stays below
    // the rounding limit (P <= 1), and the clamp is left out.
    // PRIMED: the copy of the first tile into st0 was started by the caller
    // (with the mask tile's registers in rm0).
    // The score scale sc is positive: the caller moves a non-positive scale
    // onto Q.
    template <int KIND, bool SAT = true, bool PRIMED = false>
    __device__ __forceinline__ static void sweep(const AttnParams& p, const Ctx& c,
                                                 char* __restrict__ st0, char* __restrict__ st1,
                                                 const QRegs& qreg, float sc, float ac,
                                                 float& m_run, float& l_run, float inv, ORegs& o,
                                                 const u32x4& rm0 = u32x4{},
                                                 char* __restrict__ t16 = nullptr) {
        const bool with_v = KIND != PASS_STATS;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const float kadd = ac / sc;  // staged mask weight on raw scores
        u32x4 rm = {};
        const bool mlds = STAGED;
        if (c.t0 < c.t1) {
            if constexpr (PRIMED) {
                if (mlds) store_mask(st0, c, rm0, kadd);
            } else {
                dma_tile(p, c, c.t0, with_v, st0, wave);
                if (mlds) load_mask(p, c, c.t0, rm);
                if (mlds) store_mask(st0, c, rm, kadd);
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        // Loop body for tile `it` computed from `stage` while tile it+1 is
        // staged into `nstage`; unrolled by two below so that both stage
        // addresses are compile-time LDS offsets.
        auto body = [&](int it, char* __restrict__ stage_in, char* __restrict__ nstage) {
            const bool more = it + 1 < c.t1;
            if (more) dma_tile(p, c, it + 1, with_v, nstage, wave);
            if (mlds && more) load_mask(p, c, it + 1, rm);
            // KV8: the products read the 16-bit tile converted from this
            // tile's codes (the previous tile's barrier freed it)
            char* const stage = KV8 ? t16 : stage_in;
            if constexpr (KV8) {
                convert_tile(stage_in, t16);
                lds_barrier();
            }
            const int j0 = it * C::BN;
            if (c.wave_rows && j0 < c.wave_kv_end) {
                f32x16 s[2];
                bmm1(stage, qreg, s);
                if (KIND == PASS_NONE) {
                    predicate(p, c, it, s, sc, ac, true, stage);
                    if (p.qdq) {
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int r = 0; r < 16; ++r) s[kb][r] = qdq_value(s[kb][r] * inv, p.qdq);
                        if constexpr (C::FP8) {
                            i32x8 codes;
#pragma unroll
                            for (int w = 0; w < 8; ++w) {
                                const int kb = w >> 2, r0 = (w & 3) * 4;
                                codes[w] = (int)f32x4_to_e4m3<true>(s[kb][r0], s[kb][r0 + 1],
                                                                    s[kb][r0 + 2], s[kb][r0 + 3]);
                            }
                            bmm2_fp8(stage + C::KBYTES, codes, o);
                        } else {
                            bmm2_16(stage + C::KBYTES, s, o);
                        }
                    } else {
                        bmm2_16_split(stage + C::KBYTES, s, o);
                    }
                } else {
                    // Softmax in the exp2 domain.  On a fully allowed tile the
                    // raw dot products are kept and the score scale is folded
                    // into the exp2 argument (fma); otherwise the predicate
                    // scales them and marks disallowed keys with -inf.
                    float eff = sc;
                    if constexpr (STAGED) {
                        // staged mask on raw scores, lengths / causal only
                        // where the tile is not fully allowed
                        if constexpr (!MACC) apply_mask_raw(s, stage, kadd);
                        if (!cl_full(p, c, it)) predicate_raw(c, it, s);
                    } else if constexpr (HAS_MASK) {
                        predicate(p, c, it, s, sc, ac, false, stage);
                        eff = 1.f;
                    } else {
                        if (!cl_full(p, c, it)) predicate_raw(c, it, s);
                    }
                    // row max over the lane's 32 scores: four independent chains
                    float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], s[kb][r]);
                    float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])) * eff;
                    if (KIND != PASS_FIXED) {
                        mx = halves_max(mx);
                        // Lazy rescaling: the reference max only moves when a
                        // row's max grows by more than 2^8, so exp2 values stay
                        // <= 256 and the O / l rescale is skipped for the wave
                        // on most tiles.  O / l is unchanged by the choice of
                        // reference.
                        const bool upd = mx > m_run + kLazyRescale;
                        if (__any(upd)) {
                            const float m_new = upd ? mx : m_run;
                            const float alpha = upd ? fast_exp2(m_run - m_new) : 1.f;
                            l_run *= alpha;
                            if (KIND == PASS_ONLINE) {
#pragma unroll
                                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                                    for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
                            }
                            m_run = m_new;
                        }
                        const float m_use = m_run == -INFINITY ? 0.f : m_run;
                        float l4[4] = {0.f, 0.f, 0.f, 0.f};
                        if constexpr (KIND == PASS_ONLINE && !C::FP8) {
                            // P in the BMM2 operand type; the row sum adds
                            // those rounded values (dot products with one),
                            // so l normalizes exactly the P that BMM2 uses
#pragma unroll
                            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                                for (int r = 0; r < 16; ++r)
                                    s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], eff, -m_use));
                            V8 pb[4];
                            p_operands(s, pb);
#pragma unroll
                            for (int ks = 0; ks < 4; ++ks) add_pairs(pb[ks], l4);
                            l_run += (l4[0] + l4[1]) + (l4[2] + l4[3]);
                            bmm2_ops(stage + C::KBYTES, pb, o);
                        } else {
#pragma unroll
                            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                                for (int r = 0; r < 16; ++r) {
                                    const float e = fast_exp2(__builtin_fmaf(s[kb][r], eff, -m_use));
                                    s[kb][r] = e;
                                    l4[r & 3] += e;
                                }
                            l_run += (l4[0] + l4[1]) + (l4[2] + l4[3]);
                            if (KIND == PASS_ONLINE) bmm2_16(stage + C::KBYTES, s, o);
                        }
                    } else {
                        // reference max and sum known: P = exp2(s - m) / l,
                        // x = P / qscale = exp2(s - m) * inv = exp2(s - m')
                        // with m' = m - log2(inv) (inv = 0: m' = +inf, x = 0)
                        const float m_use = m_run == -INFINITY ? 0.f : m_run;
                        const float m_q = m_use - __builtin_amdgcn_logf(inv);
                        if constexpr (C::FP8) {
                            i32x8 codes;
#pragma unroll
                            for (int w = 0; w < 8; ++w) {
                                const int kb = w >> 2, r0 = (w & 3) * 4;
                                float x0 = fast_exp2(__builtin_fmaf(s[kb][r0], eff, -m_q));
                                float x1 = fast_exp2(__builtin_fmaf(s[kb][r0 + 1], eff, -m_q));
                                float x2 = fast_exp2(__builtin_fmaf(s[kb][r0 + 2], eff, -m_q));
                                float x3 = fast_exp2(__builtin_fmaf(s[kb][r0 + 3], eff, -m_q));
                                codes[w] = (int)f32x4_to_e4m3<SAT>(x0, x1, x2, x3);
                            }
                            bmm2_fp8(stage + C::KBYTES, codes, o);
                        } else {
#pragma unroll
                            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                                for (int r = 0; r < 16; ++r)
                                    s[kb][r] = qdq_value<SAT>(
                                        fast_exp2(__builtin_fmaf(s[kb][r], eff, -m_q)), p.qdq);
                            bmm2_16(stage + C::KBYTES, s, o);
                        }
                    }
                }
            }
            if (mlds && more) store_mask(nstage, c, rm, kadd);
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's part of tile it+1 landed
            __syncthreads();
        };
        int it = c.t0;
        for (; it + 1 < c.t1; it += 2) {
            body(it, st0, st1);
            body(it + 1, st1, st0);
        }
        if (it < c.t1) body(it, st0, st1);
    }

    // Source offsets of the 16 bytes this lane writes in each tile-copy
    // instruction (they depend on the lane and the row strides only).
    __device__ __forceinline__ static void set_copy_offsets(const AttnParams& p, Ctx& c, int wave,
                                                            int lane) {
        if constexpr (KV8) {
            // source of the 16 bytes this lane writes in each copy: rows of
            // D codes, unpadded, in both tiles
#pragma unroll
            for (int k = 0; k < C::KMAX; ++k) {
                const int pos = (wave + 4 * k) * 1024 + lane * 16;
                c.koff[k] = k < K8PW ? (uint32_t)((int64_t)(pos / D) * p.k.sn + pos % D) : 0xFFFFFFF0u;
            }
#pragma unroll
            for (int k = 0; k < C::VMAX; ++k) {
                const int pos = (wave + 4 * k) * 1024 + lane * 16;
                c.voff[k] = k < V8PW ? (uint32_t)((int64_t)(pos / D) * p.v.sn + pos % D) : 0xFFFFFFF0u;
            }
        } else {
            // source of the 16 LDS bytes this lane writes in each copy
            // instruction: K rows are padded (positions in the pad read as
            // zeros), V rows are swizzled (position -> logical 16-byte unit)
#pragma unroll
            for (int k = 0; k < C::KMAX; ++k) {
                const int pos = (wave + 4 * k) * 1024 + lane * 16;
                const int row = pos / C::KROW, byte = pos % C::KROW;
                c.koff[k] = pos < C::KBYTES && byte < D * C::ES
                                ? (uint32_t)((int64_t)row * p.k.sn * C::ES + byte)
                                : 0xFFFFFFF0u;
            }
#pragma unroll
            for (int k = 0; k < C::VMAX; ++k) {
                const int pos = (wave + 4 * k) * 1024 + lane * 16;
                const int row = pos / C::VROW, unit = (pos % C::VROW) / 16;
                c.voff[k] = pos < C::VBYTES
                                ? (uint32_t)((int64_t)row * p.v.sn * C::ES + ((unit ^ v_swz<C>(row)) << 4))
                                : 0xFFFFFFF0u;
            }
        }
    }

    template <int MODE>
    __device__ __forceinline__ static void run(const AttnParams& p, char* __restrict__ st0,
                                               char* __restrict__ st1,
                                               char* __restrict__ t16 = nullptr) {
        __shared__ int s_map[6];
        const int tid = threadIdx.x, lane = tid & 63;
        // wave index in a scalar register: everything derived from it is
        // wave-uniform, and branches on it are scalar branches
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lr = lane & 31, lg = lane >> 5;
        const int R = p.rows_per_wg;
        // This workgroup's record, when the plan kernel wrote them: the loads
        // are issued first and the lane offsets below computed while they
        // are in flight.
        i32x4 rec0 = {-1, 0, 0, 0}, rec1 = {0, 0, 0, 0};
        if (p.wrec) {
            const int L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
            const i32x4* rp = (const i32x4*)(p.wrec + (int64_t)L * kWorkRecInts);
            rec0 = rp[0];
            rec1 = rp[1];
        }
        Ctx c;
        set_copy_offsets(p, c, wave, lane);
        int b, tile, q_start, kv_start, hbase, kvh, bz;
        if (p.wrec) {
            // (b, row tile, ...) are workgroup-uniform: read into scalar
            // registers, so every address and buffer descriptor built from
            // them is scalar too (a descriptor in vector registers needs a
            // loop per load)
            b = __builtin_amdgcn_readfirstlane(rec0[0]);
            if (b < 0) return;  // beyond the last tile of the batch (grid is an upper bound)
            tile = __builtin_amdgcn_readfirstlane(rec0[1]);
            c.q_len = __builtin_amdgcn_readfirstlane(rec0[2]);
            c.kv_len = __builtin_amdgcn_readfirstlane(rec0[3]);
            q_start = __builtin_amdgcn_readfirstlane(rec1[0]);
            kv_start = __builtin_amdgcn_readfirstlane(rec1[1]);
            hbase = __builtin_amdgcn_readfirstlane(rec1[2]);
            const int kz = __builtin_amdgcn_readfirstlane(rec1[3]);
            kvh = kz & 0xFFFF;
            bz = kz >> 16;
        } else {
            const SeqInfo si = map_lane_info(p);  // loads in flight during the remap
            int bx = blockIdx.x, by = blockIdx.y;
            bz = blockIdx.z;
            if (p.xcds > 1) xcd_remap(p.xcds, gridDim.x, gridDim.y, gridDim.z, bx, by, bz);
            // A grid of one round (a slot for every workgroup): an XCD hands
            // its workgroups to its CUs round-robin, so in heaviest-first
            // order the two workgroups of a CU were of similar weight; the
            // second half of the positions, reversed, pairs the heaviest
            // with the lightest (tree decoding +4%).
            if (p.mirror && bx >= (int)gridDim.x / 2) bx = gridDim.x - 1 - (bx - (int)gridDim.x / 2);
            // dispatch position -> (sequence, row tile), heaviest first
            map_tile(p, bx, R, s_map, si);
            b = __builtin_amdgcn_readfirstlane(s_map[0]);
            if (b < 0) return;
            tile = __builtin_amdgcn_readfirstlane(s_map[1]);
            c.q_len = __builtin_amdgcn_readfirstlane(s_map[2]);
            c.kv_len = __builtin_amdgcn_readfirstlane(s_map[3]);
            q_start = __builtin_amdgcn_readfirstlane(s_map[4]);
            kv_start = __builtin_amdgcn_readfirstlane(s_map[5]);
            hbase = by * p.heads_per_wg;
            kvh = hbase / p.group;
        }
        c.b = b;
        c.diag = p.causal == 1 ? 0 : c.kv_len - c.q_len;
        c.causal = p.causal != 0;
        c.tree = TREE && p.tree != nullptr;
        c.tbase = c.kv_len - c.q_len;
        c.anc0 = c.anc1 = c.anc2 = c.anc3 = 0u;
        c.tree_over = false;
        const int row0 = tile * R;
        // heads per workgroup: 1, 2 or 4 (a power of two)
        const int hw = p.heads_per_wg, hsh = __builtin_ctz((unsigned)hw);
        const int h = hbase + (wave & (hw - 1));
        c.wr0 = row0 + (wave >> hsh) * 32;
        c.i = c.wr0 + lr;
        c.wave_rows = c.wr0 < c.q_len;
        if (TREE && c.tree) {
            // Ancestor sets of the sequence's first 128 drafts by pointer
            // jumping, lane l holding drafts l and l + 64: a draft's set A
            // starts as itself and its jump J as its parent; each round
            // A |= A of J, J = J of J doubles the chain length covered, so 7
            // rounds cover any chain of 128.  Parents precede their children,
            // so every jump of draft l (< 64) stays below 64: its set lives
            // in the low 64 bits and needs its own half only.
            const int64_t prow = p.q_packed ? (int64_t)q_start : (int64_t)b * p.n_q;
            const int d1 = lane + 64;
            const int par0 = lane < c.q_len ? p.tree[prow + lane] : -1;
            const int par1 = d1 < c.q_len ? p.tree[prow + d1] : -1;
            int j0 = (par0 >= 0 && par0 < lane) ? par0 : -1;
            int j1 = (par1 >= 0 && par1 < d1) ? par1 : -1;
            // draft l: words 0, 1 of its set; draft l + 64: words 0..3
            const uint32_t self = 1u << (lane & 31);
            uint32_t a0w0 = lane < c.q_len && lane < 32 ? self : 0u;
            uint32_t a0w1 = lane < c.q_len && lane >= 32 ? self : 0u;
            uint32_t a1w0 = 0u, a1w1 = 0u;
            uint32_t a1w2 = d1 < c.q_len && lane < 32 ? self : 0u;
            uint32_t a1w3 = d1 < c.q_len && lane >= 32 ? self : 0u;
#pragma unroll
            for (int round = 0; round < 7; ++round) {
                // every lane reads its sources' values of this round first
                const int s0 = j0 >= 0 ? j0 : lane;
                const uint32_t f0 = __shfl(a0w0, s0), f1 = __shfl(a0w1, s0);
                const int fj = __shfl(j0, s0);
                const int s1 = j1 >= 0 ? (j1 & 63) : lane;
                const uint32_t g0 = __shfl(a0w0, s1), g1 = __shfl(a0w1, s1);
                const int gj = __shfl(j0, s1);
                const uint32_t h0 = __shfl(a1w0, s1), h1 = __shfl(a1w1, s1);
                const uint32_t h2 = __shfl(a1w2, s1), h3 = __shfl(a1w3, s1);
                const int hj = __shfl(j1, s1);
                if (j0 >= 0) {
                    a0w0 |= f0;
                    a0w1 |= f1;
                    j0 = fj;
                }
                if (j1 >= 64) {  // the jump lands on a draft of the upper half
                    a1w0 |= h0;
                    a1w1 |= h1;
                    a1w2 |= h2;
                    a1w3 |= h3;
                    j1 = hj;
                } else if (j1 >= 0) {
                    a1w0 |= g0;
                    a1w1 |= g1;
                    j1 = gj;
                }
            }
            // this lane's row: draft i's set from lane i % 64
            const int mine = c.i & 63;
            const uint32_t m0 = __shfl(a0w0, mine), m1 = __shfl(a0w1, mine);
            const uint32_t u0 = __shfl(a1w0, mine), u1 = __shfl(a1w1, mine);
            const uint32_t u2 = __shfl(a1w2, mine), u3 = __shfl(a1w3, mine);
            if (c.i < 64) {
                c.anc0 = m0;
                c.anc1 = m1;
            } else if (c.i < kMaxDrafts) {
                c.anc0 = u0;
                c.anc1 = u1;
                c.anc2 = u2;
                c.anc3 = u3;
            } else {
                c.tree_over = c.i < c.q_len;
            }
        }
        const int wg_last = min(row0 + R, c.q_len) - 1;
        int kv_end = c.kv_len;
        if (p.causal) kv_end = min(kv_end, wg_last + c.diag + 1);
        kv_end = max(kv_end, 0);
        c.t0 = 0;
        c.t1 = (kv_end + C::BN - 1) / C::BN;
        // split-KV: this workgroup takes one slice of the keys.  Slices
        // cover fixed key ranges: a row tile whose keys fit in one slice is
        // computed whole by slice 0 and written as final output; the others
        // write fp32 partials for the combine kernel.  Slices past the keys
        // of this row tile have nothing to do.
        int nsl = 1;
        if (p.n_splits > 1) {
            const int per = p.split_keys / C::BN;
            nsl = (c.t1 + per - 1) / per;
            if (bz >= max(nsl, 1)) return;
            c.t0 = min(bz * per, c.t1);
            c.t1 = min(c.t0 + per, c.t1);
        }
        const int wave_last = min(c.wr0 + 32, c.q_len) - 1;
        c.wave_kv_end = c.kv_len;
        if (p.causal) c.wave_kv_end = min(c.wave_kv_end, wave_last + c.diag + 1);
        // paged KV: the head's offset inside a page (the page comes per tile)
        const int64_t kro = PAGED ? 0
                            : p.kv_packed ? (int64_t)kv_start * p.k.sn : (int64_t)b * p.k.sb;
        const int64_t vro = PAGED ? 0
                            : p.kv_packed ? (int64_t)kv_start * p.v.sn : (int64_t)b * p.v.sb;
        c.kbase = (const char*)p.k.ptr + (kro + (int64_t)kvh * p.k.sh) * KES;
        c.vbase = (const char*)p.v.ptr + (vro + (int64_t)kvh * p.v.sh) * KES;
        c.kbytes = rows_bytes64(c.kv_len, p.k.sn, D, KES);
        c.vbytes = rows_bytes64(c.kv_len, p.v.sn, D, KES);
        c.ktile = (int64_t)C::BN * p.k.sn * KES;
        c.vtile = (int64_t)C::BN * p.v.sn * KES;
        c.mrow = nullptr;
        c.mtile = nullptr;
        c.mvalid = 0;
        c.moff = 0;
        c.mrow_l = -1;
        c.mchunk = 0;
        c.mbool = p.mask_kind == MASK_BOOL;  // MK_LDS_BOOL: the host launched it for a bool mask
        if constexpr (STAGED) {
            // 32 rows x BN keys; 16-bit: 8 chunks of 16 B per row (all 256
            // threads); bool: 4 chunks of 16 B per row (threads 0..127),
            // or in the fp8 kernels, whose staging expands each byte to four,
            // 8 chunks of 8 B (all 256 threads)
            const int es = p.mask_kind == MASK_BOOL ? 1 : 2;
            const int chunk = MACC && mask_is_bool(c) ? 8 : 16;
            const int cpr = C::BN * es / chunk;
            if (tid < 32 * cpr) {
                c.mrow_l = tid / cpr;
                c.mchunk = tid % cpr;
            }
            c.mtile = (const char*)p.mask + ((int64_t)b * p.m_sb + (int64_t)row0 * p.m_si) * es;
            const int rows = min(c.q_len - row0, 32);
            // The window ends with the last valid row's keys rounded up to a
            // whole 16-byte chunk (the mask's key extent is a multiple of 16
            // bytes, so the rounded end stays inside that row): a partially
            // valid chunk would otherwise be range-checked out as zeros.
            const int64_t kend = ((int64_t)c.kv_len * es + 15) & ~(int64_t)15;
            c.mvalid = rows > 0 && c.kv_len > 0 ? (int64_t)(rows - 1) * p.m_si * es + kend : 0;
            c.moff = c.mrow_l >= 0 ? (uint32_t)((int64_t)c.mrow_l * p.m_si * es + c.mchunk * chunk)
                                   : 0xFFFFFFF0u;  // idle threads: out of range, no access
        }
        if (HAS_MASK) {
            const int mes = p.mask_kind == MASK_BOOL ? 1 : (p.mask_kind == MASK_F32 ? 4 : 2);
            c.mrow = (const char*)p.mask +
                     ((int64_t)b * p.m_sb + (int64_t)h * p.m_sh + (int64_t)c.i * p.m_si) * mes;
        }

        // The copy of the first key tile (and its mask tile) starts before the
        // Q loads, so that the two latencies overlap.
        constexpr bool kFirstWithV = MODE != MODE_SOFTMAX_QDQ && MODE != MODE_SOFTMAX_QDQ_NS;
        u32x4 rm0 = {};
        if (c.t0 < c.t1) {
            dma_tile(p, c, c.t0, kFirstWithV, st0, wave);
            if constexpr (STAGED) load_mask(p, c, c.t0, rm0);
        }

        // ---- Q operand (B of S^T = K Q^T): lane (row lr, group lg).  The
        // wave's 32 rows are copied into its slice of stage 1 (free until the
        // key loop starts) by loads that write LDS directly, each moving
        // 1 KiB of whole rows, then read in operand layout.
        QRegs qreg;
        {
            char* qs = (KV8 ? t16 : st1) + wave * 32 * C::QROW;  // KV8: the free 16-bit tile
            const int nrows = max(0, min(32, c.q_len - c.wr0));
            const __amdgpu_buffer_rsrc_t qr = make_rsrc(
                (const char*)p.q.ptr +
                    ((p.q_packed ? (int64_t)q_start * p.q.sn : (int64_t)b * p.q.sb) +
                     (int64_t)h * p.q.sh + (int64_t)c.wr0 * p.q.sn) * C::ES,
                rows_bytes(nrows, p.q.sn, D, C::ES));
#pragma unroll
            for (int k = 0; k < C::QINS; ++k) {
                const int row = k * C::QRPI + lane / C::QCH;
                const int ch = (lane % C::QCH) ^ q_swz(row);  // source chunk of this position
                buf_load_lds16(qr, qs + k * 1024,
                               (uint32_t)((int64_t)row * p.q.sn * C::ES + ch * 16));
            }
            // Q (and the first tile) must be resident before the key loop:
            // otherwise the compiler cannot tell the Q loads from the tile
            // copies of the loop and waits for all of them before the first
            // MFMA.
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            const char* qrow = qs + lr * C::QROW;
#pragma unroll
            for (int ks = 0; ks < C::QSTEPS; ++ks) {
                if constexpr (C::FP8) {
                    // 32 bytes: chunks 4 ks + 2 lg and 4 ks + 2 lg + 1
                    const int c0 = ks * 4 + lg * 2;
                    const u32x4 lo = *(const u32x4*)(qrow + ((c0 ^ q_swz(lr)) << 4));
                    const u32x4 hi = *(const u32x4*)(qrow + (((c0 + 1) ^ q_swz(lr)) << 4));
                    i32x8 a;
                    a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
                    a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
                    qreg[ks] = a;
                } else {
                    // 16 bytes: chunk 2 ks + lg
                    qreg[ks] = *(const V8*)(qrow + (((ks * 2 + lg) ^ q_swz(lr)) << 4));
                }
            }
            // the operand reads complete before the barrier that lets the
            // key loop's copies overwrite stage 1
            __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
        }

        ORegs o;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
        float m_run = -INFINITY, l_run = 0.f;
        const bool none_norm = MODE == MODE_NONE;
        float sc = none_norm ? p.scale * p.k_descale : p.scale * p.k_descale * kLog2e;
        const float ac = none_norm ? 1.f : kLog2e;
        // The softmax sweeps keep raw dot products and fold the scale into
        // the exp2 argument, which needs a positive scale.  A negative scale
        // moves onto Q (sign bits flipped: every dot product changes sign
        // exactly); a zero scale zeroes Q and takes scale 1 (all scores 0).
        if (sc <= 0.f) {
            const bool neg = sc < 0.f;
            const uint32_t flip = C::FP8 ? 0x80808080u : 0x80008000u;
#pragma unroll
            for (int ks = 0; ks < C::QSTEPS; ++ks) {
                if constexpr (C::FP8) {
#pragma unroll
                    for (int w = 0; w < 8; ++w) {
                        const uint32_t x = (uint32_t)qreg[ks][w];
                        qreg[ks][w] = neg ? (int)(x ^ flip) : 0;
                    }
                } else {
                    u32x4 u = __builtin_bit_cast(u32x4, qreg[ks]);
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint32_t x = u[w];
                        u[w] = neg ? x ^ flip : 0u;
                    }
                    qreg[ks] = __builtin_bit_cast(V8, u);
                }
            }
            sc = neg ? -sc : 1.f;
        }
        float factor = p.v_descale;

        if constexpr (MODE == MODE_NONE) {
            const float inv = p.qdq ? 1.f / p.qscale : 1.f;
            sweep<PASS_NONE, true, true>(p, c, st0, st1, qreg, sc, ac, m_run, l_run, inv, o, rm0);
            poison_over(c, o);
            if (p.qdq) factor *= p.qscale;
        } else if constexpr (MODE == MODE_SOFTMAX_QDQ || MODE == MODE_SOFTMAX_QDQ_NS) {
            sweep<PASS_STATS, true, true>(p, c, st0, st1, qreg, sc, ac, m_run, l_run, 0.f, o, rm0);
            const float l_tot = halves_sum(l_run);
            const float inv = l_tot > 0.f ? 1.f / (l_tot * p.qscale) : 0.f;
            sweep<PASS_FIXED, MODE == MODE_SOFTMAX_QDQ>(p, c, st0, st1, qreg, sc, ac, m_run, l_run, inv, o);
            poison_over(c, o);
            factor *= p.qscale;
        } else {
            sweep<PASS_ONLINE, true, true>(p, c, st0, st1, qreg, sc, ac, m_run, l_run, 0.f, o, rm0,
                                           t16);
            poison_over(c, o);
            const float l_tot = halves_sum(l_run);
            if (nsl > 1) {
                // split-KV: unnormalized O with its reference max and sum
                // (exp2 domain); the combine kernel merges the slices.
                if (c.i < c.q_len) {
                    const int64_t row = (p.q_packed ? (int64_t)q_start : (int64_t)b * p.n_q) + c.i;
                    const int64_t slot = (row * p.hq + h) * p.n_splits + bz;
                    float* po = p.part_o + slot * D;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
#pragma unroll
                        for (int rq = 0; rq < 4; ++rq) {
                            f32x4 w;
#pragma unroll
                            for (int u = 0; u < 4; ++u) w[u] = o[db][rq * 4 + u];
                            *(f32x4*)(po + db * 32 + rq * 8 + lg * 4) = w;
                        }
                    if (lg == 0) {
                        p.part_ml[slot * 2] = m_run;
                        p.part_ml[slot * 2 + 1] = l_tot;
                    }
                }
                return;
            }
            factor *= l_tot > 0.f ? 1.f / l_tot : 0.f;
        }

        // ---- epilogue: lane (row lr, group lg) holds O^T[d][row] for
        // d = db*32 + rq*8 + lg*4 + u.  The wave's 32 output rows go through
        // its slice of the stages (free after the key loop's last barrier)
        // so that every store writes 1 KiB of whole rows.
        {
            char* os = KV8 ? t16 + wave * 32 * C::OROW
                           : (wave < 2 ? st0 : st1) + (wave & 1) * 32 * C::OROW;
            typedef TO TO4 __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    TO4 w;
#pragma unroll
                    for (int u = 0; u < 4; ++u) w[u] = to_t(o[db][rq * 4 + u] * factor, (TO*)nullptr);
                    const int ch = (db * 4 + rq) ^ o_swz(lr);
                    *(TO4*)(os + lr * C::OROW + ch * 16 + lg * 8) = w;
                }
            const int nrows = min(32, c.q_len - c.wr0);
            char* obase = (char*)p.out +
                          ((p.q_packed ? (int64_t)q_start * p.o_sn : (int64_t)b * p.o_sb) +
                           (int64_t)h * p.o_sh + (int64_t)c.wr0 * p.o_sn) * 2;
#pragma unroll
            for (int k = 0; k < C::OINS; ++k) {
                const int row = k * C::ORPI + lane / C::OCH;
                const int ch = lane % C::OCH;
                const u32x4 w = *(const u32x4*)(os + row * C::OROW + ((ch ^ o_swz(row)) << 4));
                if (row < nrows) *(u32x4*)(obase + (int64_t)row * p.o_sn * 2 + ch * 16) = w;
            }
        }
    }
};

// Two workgroups per CU (<= 256 VGPRs per wave), except the 16-bit "none"
// normalization kernels at D = 128, whose split BMM2 needs more registers:
// one workgroup per CU, so that no kernel uses scratch memory (scratch loads
// would share vmcnt with the direct-to-LDS tile copies that the key loop
// waits on by hand).  The fp8 Q/DQ kernels with a staged bool mask fit
// three (<= 168 VGPRs, 3 x 52 KB of LDS), as the mask-free fp8 kernels do by
// themselves; the online fp8 one would spill there and keeps two.
template <typename TI, int D, int MODE, int MK>
constexpr int kPrefillWgsPerCu =
    MODE == MODE_NONE && D == 128 && !std::is_same<TI, fp8>::value ? 1
    : MK == MK_LDS_BOOL && (MODE == MODE_SOFTMAX_QDQ || MODE == MODE_SOFTMAX_QDQ_NS) ? 3
                                                                                     : 2;

template <typename TI, int D, int MODE, int MK, bool PAGED = false>
__global__ __launch_bounds__(256, (kPrefillWgsPerCu<TI, D, MODE, MK>)) void prefill_kernel(AttnParams p) {
    // two separate stage arrays: the compiler then knows that the copy into
    // one stage never aliases the reads of the other, and does not wait for
    // the copy before computing on the current stage
    typedef Prefill<TI, D, MK, PAGED> P;
    __shared__ __attribute__((aligned(16))) char st0[P::SSTAGE];
    __shared__ __attribute__((aligned(16))) char st1[P::SSTAGE];
    P::template run<MODE>(p, st0, st1);
}

// fp8 KV cache with 16-bit Q: online softmax; fp8 stages for the copies and
// one 16-bit tile for the products (and the Q / O staging).
template <typename TI, int D, int MK, bool PAGED>
__global__ __launch_bounds__(256, 2) void prefill_kv8_kernel(AttnParams p) {
    typedef Prefill<TI, D, MK, PAGED, true> P;
    static_assert(4 * 32 * P::C::QROW <= P::C::STAGE && 4 * 32 * P::C::OROW <= P::C::STAGE,
                  "Q / O staging fits the 16-bit tile");
    __shared__ __attribute__((aligned(16))) char st0[P::STAGE8];
    __shared__ __attribute__((aligned(16))) char st1[P::STAGE8];
    __shared__ __attribute__((aligned(16))) char t16[P::C::STAGE];
    P::template run<MODE_SOFTMAX>(p, st0, st1, t16);
}

// Split-KV combine: one workgroup per (row tile, query head) merges the
// key slices of each row with the log-sum-exp rule
//   M = max m_s,  O = sum 2^(m_s - M) O_s / sum 2^(m_s - M) l_s
// (exp2 domain) and writes the valid rows of Y.
template <typename TO, int D>
__global__ __launch_bounds__(256) void prefill_combine_kernel(AttnParams p) {
    // CT threads per (row, head), each owning D / CT consecutive values of
    // d: every thread reads the slices' (m, l), then issues its 16-byte
    // partial loads of all slices before it needs them, so the reads of a
    // workgroup are in flight together.
    constexpr int CT = 8, DPT = D / CT;
    __shared__ int s_map[6];
    const int R = p.rows_per_wg;
    map_tile(p, blockIdx.x, R, s_map, map_lane_info(p));
    const int b = __builtin_amdgcn_readfirstlane(s_map[0]);
    if (b < 0) return;
    const int h = blockIdx.y;
    const int q_len = __builtin_amdgcn_readfirstlane(s_map[2]);
    const int row0 = __builtin_amdgcn_readfirstlane(s_map[1]) * R;
    // slices with work for this row tile, as the attention kernel counts
    // them; one slice: the attention kernel wrote the final rows itself
    const int kv_len = __builtin_amdgcn_readfirstlane(s_map[3]);
    int kv_end = kv_len;
    if (p.causal) {
        const int diag = p.causal == 1 ? 0 : kv_len - q_len;
        kv_end = min(kv_end, min(row0 + R, q_len) - 1 + diag + 1);
    }
    const int per = p.split_keys / 64;
    const int S = (max(kv_end, 0) + 64 * per - 1) / (64 * per);
    if (S <= 1) return;
    const int SS = p.n_splits;  // slot stride
    const int q_start = __builtin_amdgcn_readfirstlane(s_map[4]);
    const int64_t rbase = p.q_packed ? (int64_t)q_start : (int64_t)b * p.n_q;
    const int part = threadIdx.x % CT;
    for (int r = threadIdx.x / CT; r < R; r += 256 / CT) {
        const int i = row0 + r;
        if (i >= q_len) break;
        const int64_t slot0 = ((rbase + i) * p.hq + h) * SS;
        const float2* ml = (const float2*)p.part_ml + slot0;
        float M = -INFINITY;
        for (int sp = 0; sp < S; ++sp) M = fmaxf(M, ml[sp].x);
        const float Mu = M == -INFINITY ? 0.f : M;
        float acc[DPT];
#pragma unroll
        for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
        float L = 0.f;
#pragma unroll 4
        for (int sp = 0; sp < S; ++sp) {
            const float2 v = ml[sp];
            const float w = fast_exp2(v.x - Mu);
            L += w * v.y;
            const f32x4* src = (const f32x4*)(p.part_o + (slot0 + sp) * D + part * DPT);
#pragma unroll
            for (int k = 0; k < DPT / 4; ++k) {
                const f32x4 x = src[k];
#pragma unroll
                for (int u = 0; u < 4; ++u) acc[k * 4 + u] += w * x[u];
            }
        }
        const float inv = L > 0.f ? p.v_descale / L : 0.f;
        TO* orow = (TO*)p.out + (p.q_packed ? (int64_t)q_start * p.o_sn : (int64_t)b * p.o_sb) +
                   (int64_t)h * p.o_sh + (int64_t)i * p.o_sn + part * DPT;
#pragma unroll
        for (int e = 0; e < DPT; ++e) orow[e] = (TO)(acc[e] * inv);
    }
}

template <typename TI, int D, int MODE>
static void launch_m_kernel(const AttnParams& p, int grid_x, int grid_y, hipStream_t stream) {
    const dim3 grid(grid_x, grid_y, p.n_splits > 1 ? p.n_splits : 1);
    if constexpr (MODE == MODE_SOFTMAX && !std::is_same<TI, fp8>::value) {
        // paged KV: online softmax only (host-checked); masks are read per
        // lane (generic variant)
        if (p.kv_paged) {
            if (p.mask_kind != MASK_NONE)
                hipLaunchKernelGGL((prefill_kernel<TI, D, MODE, MK_GENERIC, true>), grid, dim3(256),
                                   0, stream, p);
            else if (p.tree)
                hipLaunchKernelGGL((prefill_kernel<TI, D, MODE, MK_TREE, true>), grid, dim3(256), 0,
                                   stream, p);
            else
                hipLaunchKernelGGL((prefill_kernel<TI, D, MODE, MK_NONE, true>), grid, dim3(256), 0,
                                   stream, p);
            return;
        }
    }
    if (p.mask_kind == MASK_NONE && p.tree)
        hipLaunchKernelGGL((prefill_kernel<TI, D, MODE, MK_TREE>), grid, dim3(256), 0, stream, p);
    else if (p.mask_kind == MASK_NONE)
        hipLaunchKernelGGL((prefill_kernel<TI, D, MODE, MK_NONE>), grid, dim3(256), 0, stream, p);
    else if (!p.mask_lds)
        hipLaunchKernelGGL((prefill_kernel<TI, D, MODE, MK_GENERIC>), grid, dim3(256), 0, stream, p);
    else if (p.mask_kind == MASK_BF16)
        hipLaunchKernelGGL((prefill_kernel<TI, D, MODE, MK_LDS_BF16>), grid, dim3(256), 0, stream, p);
    else if (std::is_same<TI, fp8>::value && p.mask_kind == MASK_BOOL)
        hipLaunchKernelGGL((prefill_kernel<TI, D, MODE, (std::is_same<TI, fp8>::value ? MK_LDS_BOOL : MK_LDS16)>),
                           grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_kernel<TI, D, MODE, MK_LDS16>), grid, dim3(256), 0, stream, p);
}
template <typename TI, int D, int MODE>
static void launch_m(const AttnParams& p, int grid_x, int grid_y, hipStream_t stream) {
    main_kernel_begin(stream);
    launch_m_kernel<TI, D, MODE>(p, grid_x, grid_y, stream);
    main_kernel_end(stream);
}

// fp8 KV cache with 16-bit Q (online softmax; masks read per lane), then the
// split-KV merge when the keys are split.
template <typename TI, int D>
static hipError_t launch_kv8_t(const AttnParams& p, int grid_x, int grid_y, hipStream_t stream) {
    const dim3 grid(grid_x, grid_y, p.n_splits > 1 ? p.n_splits : 1);
    main_kernel_begin(stream);
    if (p.kv_paged) {
        if (p.mask_kind != MASK_NONE)
            hipLaunchKernelGGL((prefill_kv8_kernel<TI, D, MK_GENERIC, true>), grid, dim3(256), 0, stream, p);
        else if (p.tree)
            hipLaunchKernelGGL((prefill_kv8_kernel<TI, D, MK_TREE, true>), grid, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((prefill_kv8_kernel<TI, D, MK_NONE, true>), grid, dim3(256), 0, stream, p);
    } else {
        if (p.mask_kind != MASK_NONE)
            hipLaunchKernelGGL((prefill_kv8_kernel<TI, D, MK_GENERIC, false>), grid, dim3(256), 0, stream, p);
        else if (p.tree)
            hipLaunchKernelGGL((prefill_kv8_kernel<TI, D, MK_TREE, false>), grid, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((prefill_kv8_kernel<TI, D, MK_NONE, false>), grid, dim3(256), 0, stream, p);
    }
    main_kernel_end(stream);
    if (p.n_splits > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((prefill_combine_kernel<TI, D>), dim3(grid_x, p.hq), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

template <typename TI, int D>
static hipError_t launch_t(const AttnParams& p, int grid_x, int grid_y, hipStream_t stream) {
    const int mode = p.norm_none ? MODE_NONE : (p.qdq ? MODE_SOFTMAX_QDQ : MODE_SOFTMAX);
    if (mode == MODE_NONE) {
        launch_m<TI, D, MODE_NONE>(p, grid_x, grid_y, stream);
    } else if (mode == MODE_SOFTMAX_QDQ || std::is_same<TI, fp8>::value) {
        // fp8 Q/K/V always carry fp8 Q/DQ of the scores (host-checked)
        if (p.qdq_nosat)
            launch_m<TI, D, MODE_SOFTMAX_QDQ_NS>(p, grid_x, grid_y, stream);
        else
            launch_m<TI, D, MODE_SOFTMAX_QDQ>(p, grid_x, grid_y, stream);
    } else {
        if constexpr (!std::is_same<TI, fp8>::value) {
            launch_m<TI, D, MODE_SOFTMAX>(p, grid_x, grid_y, stream);
            if (p.n_splits > 1) {
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
                typedef typename std::conditional<std::is_same<TI, bf16>::value, bf16, f16>::type TO;
                hipLaunchKernelGGL((prefill_combine_kernel<TO, D>), dim3(grid_x, p.hq), dim3(256), 0,
                                   stream, p);
            }
        }
    }
    return hipGetLastError();
}

}  // namespace gqa
