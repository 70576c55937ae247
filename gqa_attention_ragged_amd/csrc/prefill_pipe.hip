// prefill_pipe.hip -- software-pipelined prefill kernel for 16-bit Q/K/V
// with softmax normalization and no Q/DQ of the scores (TRT_Attention as the
// onnx-tensorrt "TensorRT Custom Operator Schemas" page defines it, with the
// default normalization), gfx950.
//
// Work decomposition
//   * One workgroup of 4 waves per CU (1 wave per SIMD, up to 512 registers
//     per lane).  Each wave owns NG row groups of 32 query rows that share
//     one KV head: two query heads of the same 32 positions when the group
//     size G = H_q / H_kv is even, else 64 consecutive positions of one head.
//     The 8 row groups of a workgroup cover HW = gcd(G, 8) heads of one KV
//     group and 8 / HW blocks of 32 positions, so a 64-key K/V tile staged in
//     LDS feeds 8 row groups and every K / V operand read from LDS feeds two
//     MFMAs: half the LDS traffic per MFMA of a one-group-per-wave layout.
//   * S^T = K Q^T and O^T = V^T P^T on 32x32x16 MFMAs, so each lane owns one
//     query row per group (lane % 32) and 16 of every 32 keys; the row max
//     and sum need one exchange with lane ^ 32.
//   * The key loop is software-pipelined inside each wave:
//         phase A: S(n+1) = K(n+1) Q^T      on the matrix cores, while the
//                  vector unit turns S(n) into P(n) (exp2, row sums, packing)
//         phase B: O += V(n)^T P(n)^T       on the matrix cores, while the
//                  vector unit takes the row max of S(n+1)
//     so that the softmax work of one tile hides under the MFMAs of the
//     other.  The compiler is told the interleaving with scheduling-group
//     barriers.  K and V have two LDS slots each; the K tile two ahead and
//     the V tile one ahead are fetched with buffer loads during the phases
//     and written to LDS at the end of the iteration (one barrier per tile).
//   * Online softmax in the exp2 domain (the online-normalizer method of
//     Milakov & Gimelshein 2018, as in FlashAttention-2) with lazy rescaling:
//     the reference max moves only when a row max grows by more than 2^8.
//     Row sums are taken over the packed 16-bit P (dot2 with ones), i.e. over
//     exactly the weights BMM2 applies.
//   * Causal / length limits are applied only on tiles that are not fully
//     allowed for the whole wave (the diagonal and the ragged tail).
//   * Split-KV: blockIdx.z selects a slice of the key tiles; the partial O,
//     max and sum go to a workspace merged by the prefill combine kernel.
#include "device_common.h"
#include "launch.h"
#include "tile_common.h"

namespace gqa {

template <int D, int NT>
struct PipeCfg {
    static constexpr bool FP8 = false;
    static constexpr int ES = 2;
    static constexpr int BN = 64;                   // keys per tile
    static constexpr int KROW = D * 2 + 16;         // LDS bytes per K row (padded)
    static constexpr int VROW = D * 2;              // LDS bytes per V row (swizzled)
    static constexpr int KBYTES = BN * KROW;
    static constexpr int VBYTES = BN * VROW;
    static constexpr int CHUNKS = D / 8;            // 16-byte chunks per row
    static constexpr int KPT = BN * CHUNKS / NT;    // rows per loader thread
    static constexpr int QSTEPS = D / 16;           // BMM1 k-steps
    static constexpr int DB = D / 32;               // 32-wide d blocks of O
    static constexpr int VUNITS = VROW / 16;
    static constexpr int RPL = VROW >= 256 ? 1 : 256 / VROW;
    static constexpr int LDS = 2 * KBYTES + 2 * VBYTES;
};

// v_dot2 accumulation of a packed pair with (1, 1): acc + x.lo + x.hi.
__device__ __forceinline__ float sum_pair(bf16x8 v, int i, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 x = {v[2 * i], v[2 * i + 1]};
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
}
__device__ __forceinline__ float sum_pair(f16x8 v, int i, float acc) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 x = {v[2 * i], v[2 * i + 1]};
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(x, one, acc, false);
}

// Placed in the body of a rarely taken branch: the compiler may not execute
// an asm statement speculatively, so the branch stays a branch instead of
// being turned into selects that run its (vector-wide, hence "cheap" to the
// compiler) arithmetic on every tile.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100;

// NG row groups of 32 rows per wave, NW waves per workgroup.
template <typename T, int D, int NG, int NW>
struct Pipe {
    static constexpr int NT = 64 * NW;
    typedef PipeCfg<D, NT> C;
    typedef typename Vec8<T>::type V8;
    typedef f32x16 SRegs[NG][2];          // [group][32-key block]
    typedef V8 PRegs[NG][4];              // [group][16-key k-step]
    typedef f32x16 ORegs[NG][C::DB];      // [group][d block]

    // S^T(n) for both groups from the K tile in `sK`.
    __device__ __forceinline__ static void bmm1(const char* sK, const V8 (&q)[NG][C::QSTEPS],
                                                SRegs& s) {
        const int lane = threadIdx.x & 63, lr = lane & 31, lg = lane >> 5;
#pragma unroll
        for (int g = 0; g < NG; ++g) s[g][0] = s[g][1] = f32x16{};
        const char* row0 = sK + lr * C::KROW + lg * 16;
        const char* row1 = row0 + 32 * C::KROW;
#pragma unroll
        for (int ks = 0; ks < C::QSTEPS; ++ks) {
            const V8 a0 = *(const V8*)(row0 + ks * 32);
            const V8 a1 = *(const V8*)(row1 + ks * 32);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                s[g][0] = mfma32(a0, q[g][ks], s[g][0]);
                s[g][1] = mfma32(a1, q[g][ks], s[g][1]);
            }
        }
    }

    // BMM2 A operand (V^T) for k-step ks and d block db: lane (d = db*32 +
    // lane%32, g = lane/32) gets keys ks*16 + (e/4)*8 + g*4 + e%4, the keys
    // whose probabilities the same lane holds in its S^T accumulator.
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

    __device__ __forceinline__ static void bmm2(const char* sV, const PRegs& pr, ORegs& o) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                const V8 a = v_operand(sV, ks, db);
#pragma unroll
                for (int g = 0; g < NG; ++g) o[g][db] = mfma32(a, pr[g][ks], o[g][db]);
            }
    }

    // P = exp2(S * sc - m) packed to 16 bits; l += the row sums of P.
    __device__ __forceinline__ static void exp_pack(const SRegs& s, float sc, const float (&m)[NG],
                                                    PRegs& pr, float (&l)[NG]) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float mu = m[g] == -INFINITY ? 0.f : m[g];
            float l2[2] = {0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                V8 v;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = (T)fast_exp2(__builtin_fmaf(s[g][ks >> 1][(ks & 1) * 8 + e], sc, -mu));
                pr[g][ks] = v;
#pragma unroll
                for (int i = 0; i < 4; ++i) l2[i & 1] = sum_pair(v, i, l2[i & 1]);
            }
            l[g] += l2[0] + l2[1];
        }
    }

    // Row max of the raw scores of both groups, scaled to the exp2 domain and
    // combined with the other half of the wave.
    __device__ __forceinline__ static void row_max(const SRegs& s, float sc, float (&mx)[NG]) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], s[g][kb][r]);
            mx[g] = halves_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])) * sc);
        }
    }

    // Keys at or beyond lim[g] (per lane) become -inf in tile `tile`.
    __device__ __forceinline__ static void predicate(SRegs& s, int tile, const int (&lim)[NG]) {
        keep_branch();
        const int lg = (threadIdx.x & 63) >> 5;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int rel = lim[g] - (tile * C::BN + lg * 4);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
                    s[g][kb][r] = off < rel ? s[g][kb][r] : -INFINITY;
                }
        }
    }

    // Lazy rescale after a new row max: the reference moves only when the
    // max grew by more than 2^kLazy; O and l follow the reference.
    __device__ __forceinline__ static void rescale(const float (&mx)[NG], float (&m)[NG],
                                                   float (&l)[NG], ORegs& o) {
        constexpr float kLazy = 8.0f;
        bool up[NG], any = false;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            up[g] = mx[g] > m[g] + kLazy;
            any = any || up[g];
        }
        if (__any(any)) {
            keep_branch();
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const float m_new = up[g] ? mx[g] : m[g];
                const float alpha = up[g] ? fast_exp2(m[g] - m_new) : 1.f;
                l[g] *= alpha;
#pragma unroll
                for (int db = 0; db < C::DB; ++db) o[g][db] *= alpha;
                m[g] = m_new;
            }
        }
    }

    // An empty asm that uses P: keeps its computation in phase A, next to the
    // BMM1 MFMAs it is interleaved with, instead of letting the compiler sink
    // it past the predicate branch to its use in BMM2.
    __device__ __forceinline__ static void pin(const PRegs& pr) {
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) asm volatile("" ::"v"(pr[g][ks]));
    }

    // Interleaving of phase A (BMM1 of the next tile + exp / pack / sum of
    // the current one): the K operand reads run a few MFMAs ahead of their
    // use, and every MFMA is followed by a share of the vector work.
    __device__ __forceinline__ static void schedule_a() {
        constexpr int MA = 2 * NG * C::QSTEPS;   // MFMAs
        constexpr int DA = 2 * C::QSTEPS;        // K operand reads
        constexpr int LEAD = 4;                  // reads issued ahead
        constexpr int EVERY = MA / DA;           // MFMAs per further read
        constexpr int VA = (100 * NG + MA - 1) / MA;
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, LEAD, 0);
        int left = DA - LEAD;
#pragma unroll
        for (int i = 0; i < MA; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgValu, VA, 0);
            if (left > 0 && i % EVERY == EVERY - 1) {
                __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
                --left;
            }
        }
    }
    // Phase B (BMM2 of the current tile + row max of the next one): two V^T
    // transpose reads per A operand, issued three operands ahead.
    __device__ __forceinline__ static void schedule_b() {
        constexpr int MB = 4 * C::DB * NG;       // MFMAs
        constexpr int DBR = 8 * C::DB;           // V^T reads
        constexpr int LEAD = 6;
        constexpr int PER = DBR / MB > 0 ? DBR / MB : 1;  // reads per MFMA after the lead
        int left = DBR - LEAD;
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, LEAD, 0);
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgValu, 2, 0);
            if (left > 0) {
                __builtin_amdgcn_sched_group_barrier(kSgDsRead, PER, 0);
                left -= PER;
            }
        }
    }

    __device__ __forceinline__ static void run(const AttnParams& p, char* smem) {
        __shared__ int s_map[2];
        const int tid = threadIdx.x, lane = tid & 63;
        // wave index in a scalar register: everything derived from it is
        // wave-uniform, and branches on it are scalar branches
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lr = lane & 31, lg = lane >> 5;
        const int R = p.rows_per_wg;  // 32 * 8 / heads_per_wg
        // Row tiles in reverse order: the heaviest causal tiles go first.
        const int tile = gridDim.x - 1 - blockIdx.x;
        map_tile(p, tile, R, s_map);
        const int b = __builtin_amdgcn_readfirstlane(s_map[0]);
        if (b < 0) return;
        const int row0 = __builtin_amdgcn_readfirstlane(s_map[1]) * R;
        const int q_len = q_len_of(p, b), kv_len = kv_len_of(p, b);
        const bool causal = p.causal != 0;
        const int diag = p.causal == 1 ? 0 : kv_len - q_len;
        const int hw = p.heads_per_wg;

        // row groups of this wave: (query head, first position)
        int hg[NG], pos[NG], lim[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int r = NG * wave + g;
            hg[g] = blockIdx.y * hw + r % hw;
            pos[g] = row0 + (r / hw) * 32;
            const int i = pos[g] + lr;
            lim[g] = causal ? min(kv_len, i + diag + 1) : kv_len;
        }
        const int kvh = (blockIdx.y * hw) / p.group;

        // key tiles [t0, t1) of this workgroup
        const int wg_last = min(row0 + R, q_len) - 1;
        int kv_end = causal ? min(kv_len, wg_last + diag + 1) : kv_len;
        kv_end = max(kv_end, 0);
        int t0 = 0, t1 = (kv_end + C::BN - 1) / C::BN;
        if (p.n_splits > 1) {
            const int per = p.split_keys / C::BN;
            t0 = min((int)blockIdx.z * per, t1);
            t1 = min(t0 + per, t1);
        }
        // keys below full_end are allowed for every row of this wave
        const int full_end = causal ? min(kv_len, pos[0] + diag + 1) : kv_len;  // pos[0] is the lowest

        // K / V buffer windows (bytes up to the end of the last valid key)
        const char* kbase =
            (const char*)p.k.ptr + (kv_rowbase(p, p.k, b) + (int64_t)kvh * p.k.sh) * 2;
        const char* vbase =
            (const char*)p.v.ptr + (kv_rowbase(p, p.v, b) + (int64_t)kvh * p.v.sh) * 2;
        const uint32_t kbytes = rows_bytes(kv_len, p.k.sn, D, 2);
        const uint32_t vbytes = rows_bytes(kv_len, p.v.sn, D, 2);
        const uint32_t ktile = (uint32_t)((int64_t)C::BN * p.k.sn * 2);
        const uint32_t vtile = (uint32_t)((int64_t)C::BN * p.v.sn * 2);
        uint32_t koff[C::KPT], voff[C::KPT];
        const int ch = tid % C::CHUNKS, kg = tid / C::CHUNKS;
#pragma unroll
        for (int kk = 0; kk < C::KPT; ++kk) {
            koff[kk] = (uint32_t)(((int64_t)(kg * C::KPT + kk) * p.k.sn + ch * 8) * 2);
            voff[kk] = (uint32_t)(((int64_t)(kg * C::KPT + kk) * p.v.sn + ch * 8) * 2);
        }
        // Tile `t` of K (V) into registers; tiles outside [t0, t1) read as
        // zeros and touch no memory.
        u32x4 rk[C::KPT], rv[C::KPT];
        auto load_k_into = [&](int t, u32x4 (&dst)[C::KPT]) {
            const uint32_t off = (uint32_t)t * ktile;
            const uint32_t valid = (t < t1 && kbytes > off) ? kbytes - off : 0u;
            const __amdgpu_buffer_rsrc_t r = make_rsrc(kbase + off, valid);
#pragma unroll
            for (int kk = 0; kk < C::KPT; ++kk) buf_load(r, koff[kk], dst[kk]);
        };
        auto load_k = [&](int t) { load_k_into(t, rk); };
        auto load_v = [&](int t) {
            const uint32_t off = (uint32_t)t * vtile;
            const uint32_t valid = (t < t1 && vbytes > off) ? vbytes - off : 0u;
            const __amdgpu_buffer_rsrc_t r = make_rsrc(vbase + off, valid);
#pragma unroll
            for (int kk = 0; kk < C::KPT; ++kk) buf_load(r, voff[kk], rv[kk]);
        };
        auto store_k = [&](int slot) {
            char* sK = smem + slot * C::KBYTES;
#pragma unroll
            for (int kk = 0; kk < C::KPT; ++kk)
                *(u32x4*)(sK + (kg * C::KPT + kk) * C::KROW + ch * 16) = rk[kk];
        };
        auto store_v = [&](int slot) {
            char* sV = smem + 2 * C::KBYTES + slot * C::VBYTES;
#pragma unroll
            for (int kk = 0; kk < C::KPT; ++kk) *(u32x4*)(sV + v_addr<C>(kg * C::KPT + kk, ch * 8)) = rv[kk];
        };
        auto k_slot = [&](int slot) -> const char* { return smem + slot * C::KBYTES; };
        auto v_slot = [&](int slot) -> const char* { return smem + 2 * C::KBYTES + slot * C::VBYTES; };

        // ---- Q operands (B of S^T = K Q^T) for both groups
        V8 q[NG][C::QSTEPS];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const char* qb =
                (const char*)p.q.ptr + (q_rowbase(p, b) + (int64_t)hg[g] * p.q.sh) * 2;
            const __amdgpu_buffer_rsrc_t r = make_rsrc(qb, rows_bytes(q_len, p.q.sn, D, 2));
            const uint32_t qoff = (uint32_t)(((int64_t)(pos[g] + lr) * p.q.sn + lg * 8) * 2);
#pragma unroll
            for (int ks = 0; ks < C::QSTEPS; ++ks) {
                u32x4 w;
                buf_load(r, qoff + ks * 32, w);
                q[g][ks] = __builtin_bit_cast(V8, w);
            }
        }

        const float sc = p.scale * p.k_descale * kLog2e;  // > 0 (host-checked)
        ORegs o;
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int db = 0; db < C::DB; ++db) o[g][db] = f32x16{};
        float m[NG], l[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            m[g] = -INFINITY;
            l[g] = 0.f;
        }

        const int ntiles = t1 - t0;
        if (ntiles > 0) {
            // ---- prologue: K(t0), V(t0) and K(t0+1) staged; S(t0) and its max
            // (one round trip: Q, K(t0), V(t0), K(t0+1) are in flight together)
            u32x4 rk1[C::KPT];
            load_k(t0);
            load_v(t0);
            load_k_into(t0 + 1, rk1);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q, K, V resident
            store_k(0);
            store_v(0);
#pragma unroll
            for (int kk = 0; kk < C::KPT; ++kk) rk[kk] = rk1[kk];
            store_k(1);
            __syncthreads();
            SRegs s;
            bmm1(k_slot(0), q, s);
            if ((t0 + 1) * C::BN > full_end) predicate(s, t0, lim);
            {
                float mx[NG];
                row_max(s, sc, mx);
                rescale(mx, m, l, o);
            }
            __syncthreads();  // slot 0 of K is rewritten in the first iteration

            // ---- steady state: iteration u consumes S(n), n = t0 + u, and
            // produces S(n+1); unrolled by two so that the score registers
            // swap roles instead of being copied.
            auto iteration = [&](int u, SRegs& cur, SRegs& nxt) {
                const int n = t0 + u;
                load_k(n + 2);
                load_v(n + 1);
                PRegs pr;
                // phase A: S(n+1) on the matrix cores, P(n) on the vector unit
                bmm1(k_slot((u + 1) & 1), q, nxt);
                exp_pack(cur, sc, m, pr, l);
                schedule_a();
                pin(pr);
                if ((n + 2) * C::BN > full_end) predicate(nxt, n + 1, lim);
                // phase B: O += V(n)^T P(n)^T, row max of S(n+1)
                bmm2(v_slot(u & 1), pr, o);
                float mx[NG];
                row_max(nxt, sc, mx);
                schedule_b();
                rescale(mx, m, l, o);
                __builtin_amdgcn_s_waitcnt(0x0F70);
                store_k(u & 1);        // K(n+2): slot of K(n), read in iteration u-1
                store_v((u + 1) & 1);  // V(n+1): slot of V(n-1), read in iteration u-1
                __syncthreads();
            };
            SRegs s2;
            int u = 0;
            for (; u + 2 < ntiles; u += 2) {
                iteration(u, s, s2);
                iteration(u + 1, s2, s);
            }
            if (u + 1 < ntiles) {
                iteration(u, s, s2);
                ++u;
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    s[g][0] = s2[g][0];
                    s[g][1] = s2[g][1];
                }
            }
            // ---- last tile
            {
                PRegs pr;
                exp_pack(s, sc, m, pr, l);
                bmm2(v_slot((ntiles - 1) & 1), pr, o);
            }
        }

        // ---- epilogue
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float l_tot = halves_sum(l[g]);
            const int i = pos[g] + lr;
            if (i >= q_len) continue;
            if (p.n_splits > 1) {
                // split-KV: unnormalized O with its reference max and sum
                // (exp2 domain); the combine kernel merges the slices.
                const int64_t row = (p.q_packed ? (int64_t)p.ql[b] : (int64_t)b * p.n_q) + i;
                const int64_t slot = (row * p.hq + hg[g]) * p.n_splits + blockIdx.z;
                float* po = p.part_o + slot * D;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        f32x4 w;
#pragma unroll
                        for (int u = 0; u < 4; ++u) w[u] = o[g][db][rq * 4 + u];
                        *(f32x4*)(po + db * 32 + rq * 8 + lg * 4) = w;
                    }
                if (lg == 0) {
                    p.part_ml[slot * 2] = m[g];
                    p.part_ml[slot * 2 + 1] = l_tot;
                }
                continue;
            }
            const float factor = l_tot > 0.f ? p.v_descale / l_tot : 0.f;
            T* orow = (T*)p.out + o_rowbase(p, b) + (int64_t)hg[g] * p.o_sh + (int64_t)i * p.o_sn;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    typedef T T4 __attribute__((ext_vector_type(4)));
                    T4 w;
#pragma unroll
                    for (int u = 0; u < 4; ++u) w[u] = (T)(o[g][db][rq * 4 + u] * factor);
                    *(T4*)(orow + db * 32 + rq * 8 + lg * 4) = w;
                }
        }
    }
};

// NW = 8: one workgroup per CU; NW = 4: two per CU (two waves per SIMD either
// way, so at most 256 registers per lane).
template <typename T, int D, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void prefill_pipe_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(16))) char smem[Pipe<T, D, 1, NW>::C::LDS];
    Pipe<T, D, 1, NW>::run(p, smem);
}

template <typename T, int D>
static hipError_t launch_pipe_t(const AttnParams& p, int waves, int grid_x, int grid_y,
                                hipStream_t stream) {
    const dim3 grid(grid_x, grid_y, p.n_splits > 1 ? p.n_splits : 1);
    if (waves == 8)
        hipLaunchKernelGGL((prefill_pipe_kernel<T, D, 8>), grid, dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_pipe_kernel<T, D, 4>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_prefill_pipe(const AttnParams& p, int elem, int head_dim, int waves, int grid_x,
                               int grid_y, hipStream_t stream) {
    if (elem == ELEM_F16)
        return head_dim == 64 ? launch_pipe_t<f16, 64>(p, waves, grid_x, grid_y, stream)
                              : launch_pipe_t<f16, 128>(p, waves, grid_x, grid_y, stream);
    return head_dim == 64 ? launch_pipe_t<bf16, 64>(p, waves, grid_x, grid_y, stream)
                          : launch_pipe_t<bf16, 128>(p, waves, grid_x, grid_y, stream);
}

}  // namespace gqa
