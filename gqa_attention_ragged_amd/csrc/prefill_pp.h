// prefill_pp.h -- the prefill kernel for 16-bit Q/K/V with online softmax and
// no mask, as a two-group ping-pong over the matrix cores (gfx950).
//
// Same operator and same per-tile arithmetic as prefill_impl.h (BMM1 on
// 32x32 MFMA tiles computed transposed, S^T = K Q^T; online softmax in the
// exp2 domain with lazy rescaling; O^T = V^T P^T), organized for overlap:
//
//   * A workgroup is 8 waves, two per SIMD, one workgroup per CU.  Waves
//     0..3 (group P) and 4..7 (group Q) each own 32 query rows of one head;
//     all eight share the K / V tiles of one KV head.
//   * Per 64-key tile k a wave runs A(k) = BMM1 (scores of tile k), B(k) =
//     softmax (VALU: predicate, max, exp2, sums, conversion of P), C(k) =
//     BMM2 (O += P V).  Its work alternates between a matrix phase
//     [C(k-1), A(k)] (32 MFMAs) and a vector phase [B(k)].  The two groups
//     are one phase apart and a workgroup barrier separates the phases, so
//     on every SIMD one wave issues MFMAs while the other runs its softmax:
//     the exp2 / fma / max work of the softmax (about half the matrix time
//     per tile) executes under the other wave's MFMAs instead of beside its
//     own.
//   * K / V tiles stream through four LDS stages by direct-to-LDS buffer
//     loads two tiles ahead (each wave issues 1/8 of a tile's copies), so a
//     tile's copy has two steps (four phases) to land.
#pragma once
#include "prefill_impl.h"

namespace gqa {

template <typename TI, int D>
struct PingPong {
    typedef Prefill<TI, D, MK_NONE, false> P;
    typedef typename P::C C;
    typedef typename P::Ctx Ctx;
    typedef typename P::QRegs QRegs;
    typedef typename P::ORegs ORegs;
    typedef typename P::V8 V8;
    typedef typename P::T16 T16;
    typedef typename P::TO TO;
    static_assert(!C::FP8, "16-bit inputs only");

    static constexpr int NW = 8;                       // waves per workgroup
    static constexpr int KM = (C::NKD + NW - 1) / NW;  // K copy instructions per wave and tile
    static constexpr int VM = (C::NVD + NW - 1) / NW;  // V copy instructions per wave and tile
    static constexpr int NCOPY = KM + VM;              // copy instructions per wave and tile
    static constexpr int SSTAGE = C::STAGE;
    // waves without a last copy instruction issue one (out of range: no
    // memory access) into a spare KiB, so the copy has no wave-dependent branch
    static constexpr int SPARE = (C::NKD % NW || C::NVD % NW) ? 1024 : 0;
    // Q rows staged at the start (stages 2 and 3, four waves each), O rows at
    // the end (stages 0 and 1)
    static_assert(4 * 32 * C::QROW <= SSTAGE && 4 * 32 * C::OROW <= SSTAGE, "Q / O staging fits");

    typedef V8 PRegs[4];  // P^T of one tile as the BMM2 B operands, one per 16-key k-step

    // Row strides of K and V in bytes (the copy offsets are recomputed for
    // every tile from them rather than held in registers through the loop).
    struct Copy {
        uint32_t kstride, vstride;
    };

    // Start the copy of tile `tile` into `stage`: instruction j writes LDS
    // bytes [j KiB, j KiB + 1 KiB) of the K (V) region, lane i the 16 bytes
    // at i * 16, read from the source offset of that position (K's row
    // padding and positions past the tile read out of range: zeros, no
    // memory access; V rows are swizzled).
    __device__ __forceinline__ static void dma(const Ctx& c, const Copy& cp, int tile, char* stage,
                                               int wave) {
        const __amdgpu_buffer_rsrc_t kr = P::window(c.kbase, c.kbytes, c.ktile, tile);
        const __amdgpu_buffer_rsrc_t vr = P::window(c.vbase, c.vbytes, c.vtile, tile);
        int lane = threadIdx.x & 63;
        __asm__ volatile("" : "+v"(lane));  // recomputed here, not kept through the loop
#pragma unroll
        for (int k = 0; k < KM; ++k) {
            const int j = wave + NW * k;
            const int dst = NW * (k + 1) <= C::NKD || j < C::NKD ? j * 1024 : SSTAGE;
            const int pos = j * 1024 + lane * 16;
            const int row = pos / C::KROW, byte = pos % C::KROW;
            const uint32_t off =
                pos < C::KBYTES && byte < D * C::ES ? (uint32_t)row * cp.kstride + byte : 0xFFFFFFF0u;
            buf_load_lds16_async<true>(kr, stage + dst, off);
        }
#pragma unroll
        for (int k = 0; k < VM; ++k) {
            const int j = wave + NW * k;
            const int dst = NW * (k + 1) <= C::NVD || j < C::NVD ? C::KBYTES + j * 1024 : SSTAGE;
            const int pos = j * 1024 + lane * 16;
            const int row = pos / C::VROW, unit = (pos % C::VROW) / 16;
            const uint32_t off = pos < C::VBYTES
                                     ? (uint32_t)row * cp.vstride + ((unit ^ v_swz<C>(row)) << 4)
                                     : 0xFFFFFFF0u;
            buf_load_lds16_async<true>(vr, stage + dst, off);
        }
    }

    // B(k): predicate (partial tiles), online max / rescale, exp2, row sums,
    // and P^T converted to the 16-bit BMM2 operands.
    __device__ __forceinline__ static void softmax(const AttnParams& p, const Ctx& c, int tile,
                                                   f32x16 (&s)[2], float sc, float& m_run,
                                                   float& l_run, ORegs& o, PRegs& pb) {
        if (!P::cl_full(p, c, tile)) P::predicate_raw(c, tile, s);
        float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], s[kb][r]);
        float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])) * sc;
        mx = halves_max(mx);
        // lazy rescaling: the reference max moves only when a row max grows
        // by more than 2^8 (O / l does not depend on the reference)
        const bool upd = mx > m_run + kLazyRescale;
        if (__any(upd)) {
            const float m_new = upd ? mx : m_run;
            const float alpha = upd ? fast_exp2(m_run - m_new) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
            m_run = m_new;
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = fast_exp2(__builtin_fmaf(s[ks >> 1][(ks & 1) * 8 + e], sc, -m_use));
                l4[e & 3] += x;
                pb[ks][e] = to_t(x, (T16*)nullptr);
            }
        l_run += (l4[0] + l4[1]) + (l4[2] + l4[3]);
    }

    // K operand of BMM1 k-step ks for the two 32-key blocks of a tile.
    __device__ __forceinline__ static void k_operands(const char* sK, int ks, int lane, V8& a0,
                                                      V8& a1) {
        const int lr = lane & 31, lg = lane >> 5;
        a0 = *(const V8*)(sK + lr * C::KROW + (ks * 16 + lg * 8) * 2);
        a1 = *(const V8*)(sK + (32 + lr) * C::KROW + (ks * 16 + lg * 8) * 2);
    }
    // BMM2 A operand for k-step ks and d-block db (as Prefill::v_operand,
    // with the lane index given).
    __device__ __forceinline__ static V8 v_operand(const char* sV, int ks, int db, int lane) {
        const int l16 = lane & 15, g = lane >> 5, dh = (lane >> 4) & 1;
        const int d = db * 32 + dh * 16 + 4 * (l16 & 3);
        const int key = ks * 16 + g * 4 + (l16 >> 2);
        const u32x2 lo = tr16(sV + v_addr<C>(key, d));
        const u32x2 hi = tr16(sV + v_addr<C>(key + 8, d));
        u32x4 w;
        w[0] = lo[0]; w[1] = lo[1]; w[2] = hi[0]; w[3] = hi[1];
        return __builtin_bit_cast(V8, w);
    }

    // The matrix phase's products in an explicit software pipeline (the
    // source order is the instruction order: sched_barrier keeps the
    // scheduler from sinking the operand reads to their MFMAs, which would
    // expose the LDS latency on every MFMA):
    //   C: O^T += V^T P^T over the 4 x D/32 (k-step, d-block) operands, each
    //      read (two transpose reads) three MFMAs ahead of its use;
    //   A: S^T = K Q^T, the next k-step's K operands read while this one's
    //      two MFMAs run, the two key blocks' accumulators alternating.
    template <bool DO_C, bool DO_A>
    __device__ __forceinline__ static void products(const char* sV, const char* sK,
                                                    const QRegs& qreg, const PRegs& pb, ORegs& o,
                                                    f32x16 (&s)[2]) {
        constexpr int DB = D / 32;
        constexpr int NC = 4 * DB;  // BMM2 MFMAs
        constexpr int KS = C::QSTEPS;
        constexpr int LA = 3;       // BMM2 read-ahead (operands)
        V8 va[LA + 1];
        V8 ka[2][2];
        // the operand addresses derive from the lane index read here (opaque
        // to the compiler): one set per stage hoisted out of the loop would
        // not fit the registers
        int lane = threadIdx.x & 63;
        __asm__ volatile("" : "+v"(lane));
        if constexpr (DO_C) {
#pragma unroll
            for (int i = 0; i < LA; ++i) va[i] = v_operand(sV, i / DB, i % DB, lane);
        } else {
            k_operands(sK, 0, lane, ka[0][0], ka[0][1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (DO_C) {
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                if (i + LA < NC) va[(i + LA) % (LA + 1)] = v_operand(sV, (i + LA) / DB, (i + LA) % DB, lane);
                else if (DO_A && i + LA == NC) k_operands(sK, 0, lane, ka[0][0], ka[0][1]);
                o[i % DB] = mfma32(va[i % (LA + 1)], pb[i / DB], o[i % DB]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (DO_A) {
            s[0] = f32x16{};
            s[1] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + 1 < KS) k_operands(sK, ks + 1, lane, ka[(ks + 1) & 1][0], ka[(ks + 1) & 1][1]);
                s[0] = mfma32(ka[ks & 1][0], qreg[ks], s[0]);
                s[1] = mfma32(ka[ks & 1][1], qreg[ks], s[1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // One step of the ping-pong for tile k, with tile k in stage `cur`, tile
    // k-1 in `prev` and tile k+2 copied into `next`.
    struct State {
        f32x16 s[2];
        PRegs pb;
        ORegs o;
        float m_run, l_run;
    };

    __device__ __forceinline__ static bool has_work(const Ctx& c, int tile) {
        return c.wave_rows && tile >= c.t0 && tile < c.t1 && tile * C::BN < c.wave_kv_end;
    }

    __device__ __forceinline__ static void matrix_phase(const Ctx& c, int k, const char* cur,
                                                        const char* prev, const QRegs& qreg,
                                                        State& st) {
        const bool hc = has_work(c, k - 1), ha = has_work(c, k);
        if (hc && ha) products<true, true>(prev + C::KBYTES, cur, qreg, st.pb, st.o, st.s);
        else if (hc) products<true, false>(prev + C::KBYTES, cur, qreg, st.pb, st.o, st.s);
        else if (ha) products<false, true>(prev + C::KBYTES, cur, qreg, st.pb, st.o, st.s);
    }

    __device__ __forceinline__ static void vector_phase(const AttnParams& p, const Ctx& c, int k,
                                                        float sc, State& st) {
        if (has_work(c, k)) softmax(p, c, k, st.s, sc, st.m_run, st.l_run, st.o, st.pb);
    }

    // Workgroup barrier that leaves the tile copies in flight: the s_barrier
    // alone (a __syncthreads() would also wait for every outstanding load),
    // with this wave's LDS reads complete and no memory access moved across.
    __device__ __forceinline__ static void barrier() {
        __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    }
    // Wait until at most one tile's copies (this wave's) are in flight, or
    // none when no later tile's copy was issued.
    __device__ __forceinline__ static void wait_copies(bool one_in_flight) {
        if (one_in_flight) __builtin_amdgcn_s_waitcnt(0x0F70 | (NCOPY & 0xF) | ((NCOPY >> 4) << 14));
        else __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }

    // Step k of a wave, with tile k in stage `cur`, tile k-1 in `prev` and
    // tile k+2 copied into `next`: the matrix phase [C(k-1), A(k)], then
    // the vector phase [B(k)], each opened by a workgroup barrier.  Every
    // wave runs the same steps; group Q runs them one phase after group P
    // (it passes one extra barrier first), so each barrier interval pairs
    // one group's matrix phase with the other's vector phase.  Before a
    // barrier a wave's copies of every tile up to the one the next phase of
    // either group reads have landed: tile k before the matrix phase (tile
    // k+1 may be in flight) and tile k+1 before the vector phase (tile k+2
    // may be).
    template <int J>
    __device__ __forceinline__ static void step(const AttnParams& p, const Ctx& c, const Copy& cp,
                                                int k, char* __restrict__ s0, char* __restrict__ s1,
                                                char* __restrict__ s2, char* __restrict__ s3,
                                                const QRegs& qreg, float sc, int wave, State& st) {
        char* const stg[4] = {s0, s1, s2, s3};
        char* cur = stg[J];
        char* prev = stg[(J + 3) & 3];
        char* next = stg[(J + 2) & 3];
        wait_copies(k + 1 < c.t1);
        barrier();
        if (k + 2 < c.t1) dma(c, cp, k + 2, next, wave);
        matrix_phase(c, k, cur, prev, qreg, st);
        wait_copies(k + 2 < c.t1);
        barrier();
        vector_phase(p, c, k, sc, st);
    }

    __device__ __forceinline__ static void run(const AttnParams& p, char* __restrict__ st0,
                                               char* __restrict__ st1, char* __restrict__ st2,
                                               char* __restrict__ st3) {
        __shared__ int s_map[6];
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int grp = wave >> 2;  // 0: group P, 1: group Q (one of each per SIMD)
        const int lr = lane & 31, lg = lane >> 5;
        const int R = p.rows_per_wg;
        const SeqInfo si = map_lane_info(p);
        int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
        if (p.xcds > 1) {
            // XCD x takes one contiguous block of the work items ordered (head
            // group, split, row tile), so a head group's K / V rows are fetched
            // into one L2
            const int nx = gridDim.x, ny = gridDim.y, nz = gridDim.z, X = p.xcds;
            const int n = nx * ny * nz, L = bx + nx * (by + ny * bz);
            const int xcd = L % X, kk = L / X, q = n / X, r = n % X;
            const int li = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + kk;
            bx = li % nx;
            bz = (li / nx) % nz;
            by = li / (nx * nz);
        }
        map_tile(p, bx, R, s_map, si);
        const int b = __builtin_amdgcn_readfirstlane(s_map[0]);
        if (b < 0) return;

        Ctx c;
        c.b = b;
        c.q_len = __builtin_amdgcn_readfirstlane(s_map[2]);
        c.kv_len = __builtin_amdgcn_readfirstlane(s_map[3]);
        const int q_start = __builtin_amdgcn_readfirstlane(s_map[4]);
        const int kv_start = __builtin_amdgcn_readfirstlane(s_map[5]);
        c.diag = p.causal == 1 ? 0 : c.kv_len - c.q_len;
        c.causal = p.causal != 0;
        c.tree = false;
        c.tbase = 0;
        c.anc0 = c.anc1 = c.anc2 = c.anc3 = 0u;
        c.tree_over = false;
        const int row0 = __builtin_amdgcn_readfirstlane(s_map[1]) * R;
        const int hw = p.heads_per_wg;
        const int h = by * hw + (wave % hw);
        const int kvh = (by * hw) / p.group;
        c.wr0 = row0 + (wave / hw) * 32;
        c.i = c.wr0 + lr;
        c.wave_rows = c.wr0 < c.q_len;
        const int wg_last = min(row0 + R, c.q_len) - 1;
        int kv_end = c.kv_len;
        if (p.causal) kv_end = min(kv_end, wg_last + c.diag + 1);
        kv_end = max(kv_end, 0);
        c.t0 = 0;
        c.t1 = (kv_end + C::BN - 1) / C::BN;
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
        const int64_t kro = p.kv_packed ? (int64_t)kv_start * p.k.sn : (int64_t)b * p.k.sb;
        const int64_t vro = p.kv_packed ? (int64_t)kv_start * p.v.sn : (int64_t)b * p.v.sb;
        c.kbase = (const char*)p.k.ptr + (kro + (int64_t)kvh * p.k.sh) * C::ES;
        c.vbase = (const char*)p.v.ptr + (vro + (int64_t)kvh * p.v.sh) * C::ES;
        c.kbytes = rows_bytes64(c.kv_len, p.k.sn, D, C::ES);
        c.vbytes = rows_bytes64(c.kv_len, p.v.sn, D, C::ES);
        c.ktile = (int64_t)C::BN * p.k.sn * C::ES;
        c.vtile = (int64_t)C::BN * p.v.sn * C::ES;
        c.mrow = nullptr;
        c.mtile = nullptr;
        c.mvalid = 0;
        c.moff = 0;
        c.mrow_l = -1;
        c.mchunk = 0;
        c.mbool = false;
        // a tile's rows span < 2^32 bytes (host-checked): 32-bit row strides
        Copy cp;
        cp.kstride = (uint32_t)(p.k.sn * C::ES);
        cp.vstride = (uint32_t)(p.v.sn * C::ES);

        // the first two tiles' copies start before the Q loads
        if (c.t0 < c.t1) dma(c, cp, c.t0, st0, wave);
        if (c.t0 + 1 < c.t1) dma(c, cp, c.t0 + 1, st1, wave);

        // ---- Q operand: the wave's 32 rows through its slice of stage 2 / 3
        QRegs qreg;
        {
            char* qs = (wave < 4 ? st2 : st3) + (wave & 3) * 32 * C::QROW;
            const int nrows = max(0, min(32, c.q_len - c.wr0));
            const __amdgpu_buffer_rsrc_t qr = make_rsrc(
                (const char*)p.q.ptr +
                    ((p.q_packed ? (int64_t)q_start * p.q.sn : (int64_t)b * p.q.sb) +
                     (int64_t)h * p.q.sh + (int64_t)c.wr0 * p.q.sn) * C::ES,
                rows_bytes(nrows, p.q.sn, D, C::ES));
#pragma unroll
            for (int k = 0; k < C::QINS; ++k) {
                const int row = k * C::QRPI + lane / C::QCH;
                const int ch = (lane % C::QCH) ^ P::q_swz(row);
                buf_load_lds16(qr, qs + k * 1024, (uint32_t)((int64_t)row * p.q.sn * C::ES + ch * 16));
            }
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            const char* qrow = qs + lr * C::QROW;
#pragma unroll
            for (int ks = 0; ks < C::QSTEPS; ++ks)
                qreg[ks] = *(const V8*)(qrow + (((ks * 2 + lg) ^ P::q_swz(lr)) << 4));
            // the operand reads complete before the first step's barrier, after
            // which stage 2 receives tile t0 + 2
            __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
        }

        State st;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) st.o[db] = f32x16{};
        st.m_run = -INFINITY;
        st.l_run = 0.f;
        float sc = p.scale * p.k_descale * kLog2e;
        // the exp2 argument folds the scale in, which needs it positive: a
        // negative scale moves onto Q (sign bits flipped), a zero scale
        // zeroes Q and takes scale 1
        if (sc <= 0.f) {
            const bool neg = sc < 0.f;
#pragma unroll
            for (int ks = 0; ks < C::QSTEPS; ++ks) {
                u32x4 u = __builtin_bit_cast(u32x4, qreg[ks]);
#pragma unroll
                for (int w = 0; w < 4; ++w) u[w] = neg ? u[w] ^ 0x80008000u : 0u;
                qreg[ks] = __builtin_bit_cast(V8, u);
            }
            sc = neg ? -sc : 1.f;
        }

        // ---- the ping-pong over steps t0 .. t1 (step t1 only finishes
        // C(t1-1)); group Q starts one phase late, group P ends one phase late
        if (grp == 1) barrier();
        for (int k = c.t0; k <= c.t1;) {
            step<0>(p, c, cp, k, st0, st1, st2, st3, qreg, sc, wave, st);
            if (++k > c.t1) break;
            step<1>(p, c, cp, k, st0, st1, st2, st3, qreg, sc, wave, st);
            if (++k > c.t1) break;
            step<2>(p, c, cp, k, st0, st1, st2, st3, qreg, sc, wave, st);
            if (++k > c.t1) break;
            step<3>(p, c, cp, k, st0, st1, st2, st3, qreg, sc, wave, st);
            ++k;
        }
        if (grp == 0) barrier();
        __syncthreads();  // every stage is free for the O staging
        // The epilogue's addresses derive from the lane index read again here
        // (opaque to the compiler): computed before the loop they would stay
        // in registers through it.
        int elane = lane;
        __asm__ volatile("" : "+v"(elane));
        const int elr = elane & 31, elg = elane >> 5;

        const float l_tot = halves_sum(st.l_run);
        if (nsl > 1) {
            // split-KV: unnormalized O with its reference max and sum (exp2
            // domain) for the combine kernel
            if (c.wr0 + elr < c.q_len) {
                const int64_t row = (p.q_packed ? (int64_t)q_start : (int64_t)b * p.n_q) + c.wr0 + elr;
                const int64_t slot = (row * p.hq + h) * p.n_splits + bz;
                float* po = p.part_o + slot * D;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        f32x4 w;
#pragma unroll
                        for (int u = 0; u < 4; ++u) w[u] = st.o[db][rq * 4 + u];
                        *(f32x4*)(po + db * 32 + rq * 8 + elg * 4) = w;
                    }
                if (elg == 0) {
                    p.part_ml[slot * 2] = st.m_run;
                    p.part_ml[slot * 2 + 1] = l_tot;
                }
            }
            return;
        }
        const float factor = p.v_descale * (l_tot > 0.f ? 1.f / l_tot : 0.f);

        // ---- epilogue: whole-row stores through the wave's slice of stage 0 / 1
        {
            char* os = (wave < 4 ? st0 : st1) + (wave & 3) * 32 * C::OROW;
            typedef TO TO4 __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    TO4 w;
#pragma unroll
                    for (int u = 0; u < 4; ++u) w[u] = to_t(st.o[db][rq * 4 + u] * factor, (TO*)nullptr);
                    const int ch = (db * 4 + rq) ^ P::o_swz(elr);
                    *(TO4*)(os + elr * C::OROW + ch * 16 + elg * 8) = w;
                }
            const int nrows = min(32, c.q_len - c.wr0);
            char* obase = (char*)p.out +
                          ((p.q_packed ? (int64_t)q_start * p.o_sn : (int64_t)b * p.o_sb) +
                           (int64_t)h * p.o_sh + (int64_t)c.wr0 * p.o_sn) * 2;
#pragma unroll
            for (int k = 0; k < C::OINS; ++k) {
                const int row = k * C::ORPI + elane / C::OCH;
                const int ch = elane % C::OCH;
                const u32x4 w = *(const u32x4*)(os + row * C::OROW + ((ch ^ P::o_swz(row)) << 4));
                if (row < nrows) *(u32x4*)(obase + (int64_t)row * p.o_sn * 2 + ch * 16) = w;
            }
        }
    }
};

template <typename TI, int D>
__global__ __launch_bounds__(512, 1) void prefill_pp_kernel(AttnParams p) {
    typedef PingPong<TI, D> K;
    // four separate stage arrays: the compiler then knows that the copy into
    // one stage never aliases the reads of another
    __shared__ __attribute__((aligned(16))) char st0[K::SSTAGE + K::SPARE];
    __shared__ __attribute__((aligned(16))) char st1[K::SSTAGE + K::SPARE];
    __shared__ __attribute__((aligned(16))) char st2[K::SSTAGE + K::SPARE];
    __shared__ __attribute__((aligned(16))) char st3[K::SSTAGE + K::SPARE];
    K::run(p, st0, st1, st2, st3);
}

}  // namespace gqa
