// prefill_persist.h -- persistent form of the 16-bit prefill kernel for the
// plain case: online softmax, no mask, no tree, contiguous (unpaged) K / V.
//
// Same operator and per-tile arithmetic as Prefill (prefill_impl.h): S^T =
// K Q^T on 32x32 MFMA tiles, online softmax in the exp2 domain with lazy
// rescaling, O^T += V^T P^T.  What differs is how a workgroup gets its work.
//
// A freshly launched workgroup waits for two memory round trips before its
// first MFMA (the sequence lengths for its tile map, then its Q rows and
// first K / V tile), and its CU meanwhile runs the other workgroup alone; on
// short ragged sequences that costs about three key tiles of compute per
// workgroup.  Here the grid is two workgroups per CU and each works through
// a stream of work items (row tile, head group, key slice):
//   * Items are ordered as the one-shot kernel orders its workgroups: XCD x
//     takes one contiguous block of the items, row tiles of the longest
//     sequences first.  A workgroup's first two items are fixed (its index j
//     among the gx workgroups of its XCD, then j + gx); after that it claims
//     items from a per-XCD counter (atomic add), so whichever workgroup
//     finishes first takes the next item, as the hardware dispatcher would.
//   * The claim for the item after next is issued at the start of an item
//     and read at its end (the atomic's round trip is hidden), and the next
//     item's map entry is resolved at the start of the current item.
//   * While a workgroup computes the last key tile of an item it copies the
//     next item's first K / V tile into the stage the item no longer needs,
//     and loads the next item's Q rows straight into the Q operand registers
//     (their last use was that tile's BMM1).  The output rows go through the
//     stage of the last tile, so the next item starts without waiting.
#pragma once
#include "prefill_impl.h"

namespace gqa {

template <typename TI, int D>
struct Persist {
    typedef Prefill<TI, D, MK_NONE, false> P;
    typedef typename P::C C;
    typedef typename P::Ctx Ctx;
    typedef typename P::QRegs QRegs;
    typedef typename P::ORegs ORegs;
    typedef typename P::V8 V8;
    typedef typename P::TO TO;
    static_assert(!C::FP8, "16-bit inputs only");
    static_assert(4 * 32 * C::OROW <= C::STAGE, "the four waves' output rows fit one stage");

    // This workgroup's share of the items: the block [lo, lo + cnt) of its
    // XCD (or all items without the XCD order), its first item `first`, the
    // number of workgroups sharing the block, and the block's claim counter.
    struct Sched {
        int lo, cnt, first, gx;
        int* ctr;
    };
    __device__ __forceinline__ static Sched sched(const AttnParams& p) {
        const int n = p.grid_x * p.grid_y * max(p.n_splits, 1);
        Sched s;
        if (p.xcds > 1) {
            const int X = p.xcds, xcd = (int)blockIdx.x % X;
            const int q = n / X, r = n % X;
            s.lo = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
            s.cnt = q + (xcd < r ? 1 : 0);
            s.first = (int)blockIdx.x / X;
            s.gx = ((int)gridDim.x - xcd + X - 1) / X;
            s.ctr = p.sched + xcd * 16;
        } else {
            s.lo = 0;
            s.cnt = n;
            s.first = blockIdx.x;
            s.gx = gridDim.x;
            s.ctr = p.sched;
        }
        return s;
    }

    // Item li -> (row-tile position bx, head group by, key slice bz), as the
    // one-shot kernel decomposes its (remapped) workgroup index.
    __device__ __forceinline__ static void decode(const AttnParams& p, int li, int& bx, int& by,
                                                  int& bz) {
        const int nx = p.grid_x, ny = p.grid_y, nz = max(p.n_splits, 1);
        bx = li % nx;
        if (p.xcds > 1) {
            bz = (li / nx) % nz;
            by = li / (nx * nz);
        } else {
            by = (li / nx) % ny;
            bz = li / (nx * ny);
        }
    }

    // A work item's workgroup-wide values, computed once by wave 0 into LDS
    // (ints; 64-bit values as two ints, low first).
    enum {
        D_MORE = 0,  // the item exists (the XCD block has it); else this workgroup is done
        D_VALID,     // the item has rows and keys for this workgroup
        D_B, D_QLEN, D_KVLEN, D_QSTART, D_DIAG, D_ROW0, D_T0, D_T1, D_NSL, D_BZ, D_BY,
        D_KBASE = 14, D_VBASE = 16, D_KBYTES = 18, D_VBYTES = 20, D_QBASE = 22, D_OBASE = 24,
        D_N = 28
    };

    // Per-item values besides the context.
    struct Item {
        int h, q_start, bz, nsl;
        const char* qsrc;  // this wave's first Q row
        uint32_t qbytes;   // bytes of its valid Q rows (a buffer window)
        const char* obase; // the workgroup's first output row (head 0)
    };

    __device__ __forceinline__ static int64_t ld64(const int* d, int i) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane(d[i]);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane(d[i + 1]);
        return (int64_t)(((uint64_t)hi << 32) | lo);
    }

    // Wave 0: the descriptor of block-local item k into d (lane 0 writes).
    // ord: the dispatch-ordered sequence table (idx, n, incl per lane),
    // seq: the sequences' (q_len, kv_len, q_start, kv_start).
    __device__ __forceinline__ static void describe(const AttnParams& p, const Sched& sd, int k,
                                                    const int (*ord)[4], const SeqInfo* seq,
                                                    int lane, int* d) {
        int v[D_N];
#pragma unroll
        for (int i = 0; i < D_N; ++i) v[i] = 0;
        v[D_MORE] = k < sd.cnt;
        if (k < sd.cnt) {
            int bx, by, bz;
            decode(p, sd.lo + k, bx, by, bz);
            const int idx = ord[lane][0], n = ord[lane][1], incl = ord[lane][2];
            const int ahead = incl - n;
            const uint64_t hit = __ballot(n > 0 && bx >= ahead && bx < incl);
            if (hit != 0) {
                const int src = (int)__builtin_ctzll(hit);
                const int b = __builtin_amdgcn_readlane(idx, src);
                const int t = __builtin_amdgcn_readlane(n - 1 - (bx - ahead), src);
                if (b < p.batch) {
                    const SeqInfo si = seq[b];
                    const int q_len = __builtin_amdgcn_readfirstlane(si.q_len);
                    const int kv_len = __builtin_amdgcn_readfirstlane(si.kv_len);
                    const int q_start = __builtin_amdgcn_readfirstlane(si.q_start);
                    const int kv_start = __builtin_amdgcn_readfirstlane(si.kv_start);
                    const int R = p.rows_per_wg;
                    const int row0 = t * R;
                    const int diag = p.causal == 1 ? 0 : kv_len - q_len;
                    const int wg_last = min(row0 + R, q_len) - 1;
                    int kv_end = kv_len;
                    if (p.causal) kv_end = min(kv_end, wg_last + diag + 1);
                    kv_end = max(kv_end, 0);
                    int t0 = 0, t1 = (kv_end + C::BN - 1) / C::BN, nsl = 1;
                    bool ok = true;
                    if (p.n_splits > 1) {
                        const int per = p.split_keys / C::BN;
                        nsl = (t1 + per - 1) / per;
                        ok = bz < max(nsl, 1);
                        t0 = min(bz * per, t1);
                        t1 = min(t0 + per, t1);
                    }
                    const int kvh = (by * p.heads_per_wg) / p.group;
                    const int64_t kro = p.kv_packed ? (int64_t)kv_start * p.k.sn : (int64_t)b * p.k.sb;
                    const int64_t vro = p.kv_packed ? (int64_t)kv_start * p.v.sn : (int64_t)b * p.v.sb;
                    const uint64_t kbase = (uint64_t)((const char*)p.k.ptr + (kro + (int64_t)kvh * p.k.sh) * C::ES);
                    const uint64_t vbase = (uint64_t)((const char*)p.v.ptr + (vro + (int64_t)kvh * p.v.sh) * C::ES);
                    const uint64_t kbytes = (uint64_t)rows_bytes64(kv_len, p.k.sn, D, C::ES);
                    const uint64_t vbytes = (uint64_t)rows_bytes64(kv_len, p.v.sn, D, C::ES);
                    const uint64_t qbase = (uint64_t)((const char*)p.q.ptr +
                        (p.q_packed ? (int64_t)q_start * p.q.sn : (int64_t)b * p.q.sb) * C::ES);
                    const uint64_t obase = (uint64_t)((const char*)p.out +
                        (p.q_packed ? (int64_t)q_start * p.o_sn : (int64_t)b * p.o_sb) * 2);
                    v[D_VALID] = ok;
                    v[D_B] = b;
                    v[D_QLEN] = q_len;
                    v[D_KVLEN] = kv_len;
                    v[D_QSTART] = q_start;
                    v[D_DIAG] = diag;
                    v[D_ROW0] = row0;
                    v[D_T0] = t0;
                    v[D_T1] = t1;
                    v[D_NSL] = nsl;
                    v[D_BZ] = bz;
                    v[D_BY] = by;
                    v[D_KBASE] = (int)(uint32_t)kbase;
                    v[D_KBASE + 1] = (int)(uint32_t)(kbase >> 32);
                    v[D_VBASE] = (int)(uint32_t)vbase;
                    v[D_VBASE + 1] = (int)(uint32_t)(vbase >> 32);
                    v[D_KBYTES] = (int)(uint32_t)kbytes;
                    v[D_KBYTES + 1] = (int)(uint32_t)(kbytes >> 32);
                    v[D_VBYTES] = (int)(uint32_t)vbytes;
                    v[D_VBYTES + 1] = (int)(uint32_t)(vbytes >> 32);
                    v[D_QBASE] = (int)(uint32_t)qbase;
                    v[D_QBASE + 1] = (int)(uint32_t)(qbase >> 32);
                    v[D_OBASE] = (int)(uint32_t)obase;
                    v[D_OBASE + 1] = (int)(uint32_t)(obase >> 32);
                }
            }
        }
        if (lane == 0) {
#pragma unroll
            for (int i = 0; i < D_N; ++i) d[i] = v[i];
        }
    }

    // This wave's context of the item described by d; false when the
    // workgroup has nothing to do for it.  koff / voff: this lane's copy
    // offsets (the same for every item).
    __device__ __forceinline__ static bool build(const AttnParams& p, const int* d,
                                                 const uint32_t (&koff)[C::KMAX],
                                                 const uint32_t (&voff)[C::VMAX], int wave,
                                                 int lane, Ctx& c, Item& im) {
        if (__builtin_amdgcn_readfirstlane(d[D_VALID]) == 0) return false;
        c.b = __builtin_amdgcn_readfirstlane(d[D_B]);
        c.q_len = __builtin_amdgcn_readfirstlane(d[D_QLEN]);
        c.kv_len = __builtin_amdgcn_readfirstlane(d[D_KVLEN]);
        im.q_start = __builtin_amdgcn_readfirstlane(d[D_QSTART]);
        c.diag = __builtin_amdgcn_readfirstlane(d[D_DIAG]);
        const int row0 = __builtin_amdgcn_readfirstlane(d[D_ROW0]);
        c.t0 = __builtin_amdgcn_readfirstlane(d[D_T0]);
        c.t1 = __builtin_amdgcn_readfirstlane(d[D_T1]);
        im.nsl = __builtin_amdgcn_readfirstlane(d[D_NSL]);
        im.bz = __builtin_amdgcn_readfirstlane(d[D_BZ]);
        const int by = __builtin_amdgcn_readfirstlane(d[D_BY]);
        c.causal = p.causal != 0;
        c.tree = false;
        c.tbase = 0;
        c.anc0 = c.anc1 = c.anc2 = c.anc3 = 0u;
        c.tree_over = false;
        const int hw = p.heads_per_wg;
        im.h = by * hw + (wave % hw);
        c.wr0 = row0 + (wave / hw) * 32;
        c.i = c.wr0 + (lane & 31);
        c.wave_rows = c.wr0 < c.q_len;
        const int wave_last = min(c.wr0 + 32, c.q_len) - 1;
        c.wave_kv_end = c.kv_len;
        if (p.causal) c.wave_kv_end = min(c.wave_kv_end, wave_last + c.diag + 1);
        c.kbase = (const char*)ld64(d, D_KBASE);
        c.vbase = (const char*)ld64(d, D_VBASE);
        c.kbytes = ld64(d, D_KBYTES);
        c.vbytes = ld64(d, D_VBYTES);
        c.ktile = (int64_t)C::BN * p.k.sn * C::ES;
        c.vtile = (int64_t)C::BN * p.v.sn * C::ES;
#pragma unroll
        for (int k = 0; k < C::KMAX; ++k) c.koff[k] = koff[k];
#pragma unroll
        for (int k = 0; k < C::VMAX; ++k) c.voff[k] = voff[k];
        c.mrow = nullptr;
        c.mtile = nullptr;
        c.mvalid = 0;
        c.moff = 0;
        c.mrow_l = -1;
        c.mchunk = 0;
        c.mbool = false;
        const int nrows = max(0, min(32, c.q_len - c.wr0));
        im.qsrc = (const char*)ld64(d, D_QBASE) + ((int64_t)im.h * p.q.sh + (int64_t)c.wr0 * p.q.sn) * C::ES;
        im.qbytes = rows_bytes(nrows, p.q.sn, D, C::ES);
        im.obase = (const char*)ld64(d, D_OBASE);
        return true;
    }

    // Q operand of an item straight into registers: lane (row lr, group lg)
    // reads the 16 bytes of k-step ks at (ks * 16 + lg * 8) elements into its
    // row; rows past the item's valid rows lie outside the window and read
    // as zero.  (A 32-row window spans < 2^32 bytes: host-checked.)
    __device__ __forceinline__ static void load_q(const AttnParams& p, const Item& im, int lane,
                                                  QRegs& q) {
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(im.qsrc, im.qbytes);
        __asm__ volatile("" : "+v"(lane));  // offsets computed here, not hoisted
        const uint32_t roff = (uint32_t)((int64_t)(lane & 31) * p.q.sn * C::ES);
        const int lg = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < C::QSTEPS; ++ks) {
            u32x4 v;
            buf_load(qr, roff + (uint32_t)((ks * 16 + lg * 8) * C::ES), v);
            q[ks] = __builtin_bit_cast(V8, v);
        }
    }

    // A negative scale moves onto Q (sign bits flipped), a zero scale zeroes
    // Q: the softmax folds a positive scale into its exp2 argument.
    __device__ __forceinline__ static void sign_q(float sc_raw, QRegs& q) {
        if (sc_raw <= 0.f) {
            const bool neg = sc_raw < 0.f;
#pragma unroll
            for (int ks = 0; ks < C::QSTEPS; ++ks) {
                u32x4 u = __builtin_bit_cast(u32x4, q[ks]);
#pragma unroll
                for (int w = 0; w < 4; ++w) u[w] = neg ? u[w] ^ 0x80008000u : 0u;
                q[ks] = __builtin_bit_cast(V8, u);
            }
        }
    }

    // One tile's online softmax and O += P V (the online pass of Prefill):
    // row max with lazy rescaling, exp2 of the scaled scores, P in the
    // 16-bit operand type, row sums of those rounded values, BMM2.
    __device__ __forceinline__ static void online_tile(f32x16 (&s)[2], float sc, float& m_run,
                                                       float& l_run, ORegs& o, const char* sV) {
        float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], s[kb][r]);
        float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])) * sc;
        mx = halves_max(mx);
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
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], sc, -m_use));
        V8 pb[4];
        P::p_operands(s, pb);
        float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) add_pairs(pb[ks], l4);
        l_run += (l4[0] + l4[1]) + (l4[2] + l4[3]);
        P::bmm2_ops(sV, pb, o);
    }

    // Key tiles [t0, t1) of the item, tile t0 + i in stage (i even ? sa :
    // sb), the first one already copied and published.  pf: the last tile's
    // body also starts the copy of the next item's first tile (into the
    // other stage) and loads its Q rows into qreg; that item's context is
    // rebuilt there from its descriptor nd rather than kept in registers
    // through the loop.
    __device__ __forceinline__ static void sweep(const AttnParams& p, const Ctx& c, char* sa,
                                                 char* sb, QRegs& qreg, float sc, float& m_run,
                                                 float& l_run, ORegs& o, bool pf, const int* nd,
                                                 const uint32_t (&koff)[C::KMAX],
                                                 const uint32_t (&voff)[C::VMAX], int wave,
                                                 int lane) {
        auto body = [&](int it, char* stage, char* nstage) {
            const bool more = it + 1 < c.t1;
            Ctx nc;
            Item ni;
            if (more) {
                P::dma_tile(p, c, it + 1, true, nstage, wave);
            } else if (pf) {
                build(p, nd, koff, voff, wave, lane, nc, ni);
                P::dma_tile(p, nc, nc.t0, true, nstage, wave);
            }
            if (c.wave_rows && it * C::BN < c.wave_kv_end) {
                f32x16 s[2];
                P::bmm1(stage, qreg, s);
                if (!more && pf) load_q(p, ni, lane, qreg);  // after its last use
                if (!P::cl_full(p, c, it)) P::predicate_raw(c, it, s);
                online_tile(s, sc, m_run, l_run, o, stage + C::KBYTES);
            } else if (!more && pf) {
                load_q(p, ni, lane, qreg);
            }
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's copies (and Q) landed
            __syncthreads();
        };
        int it = c.t0;
        for (; it + 1 < c.t1; it += 2) {
            body(it, sa, sb);
            body(it + 1, sb, sa);
        }
        if (it < c.t1) body(it, sa, sb);
    }

    __device__ __forceinline__ static void run(const AttnParams& p, char* __restrict__ st0,
                                               char* __restrict__ st1) {
        // descriptors of the current and the next item; the sequence table
        // in dispatch order (idx, row tiles, inclusive scan); the sequences'
        // (q_len, kv_len, q_start, kv_start)
        __shared__ int s_desc[2][D_N];
        __shared__ int s_ord[64][4];
        __shared__ SeqInfo s_seq[64];
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int R = p.rows_per_wg;
        const Sched sd = sched(p);
        if (wave == 0) {
            const SeqInfo si = map_lane_info(p);
            int idx, n, incl;
            dispatch_order(p, R, si, idx, n, incl);
            s_seq[lane] = si;
            s_ord[lane][0] = idx;
            s_ord[lane][1] = n;
            s_ord[lane][2] = incl;
        }

        // source offsets of this lane's copy positions (as Prefill::run)
        uint32_t koff[C::KMAX], voff[C::VMAX];
#pragma unroll
        for (int k = 0; k < C::KMAX; ++k) {
            const int pos = (wave + 4 * k) * 1024 + lane * 16;
            const int row = pos / C::KROW, byte = pos % C::KROW;
            koff[k] = pos < C::KBYTES && byte < D * C::ES
                          ? (uint32_t)((int64_t)row * p.k.sn * C::ES + byte)
                          : 0xFFFFFFF0u;
        }
#pragma unroll
        for (int k = 0; k < C::VMAX; ++k) {
            const int pos = (wave + 4 * k) * 1024 + lane * 16;
            const int row = pos / C::VROW, unit = (pos % C::VROW) / 16;
            voff[k] = pos < C::VBYTES
                          ? (uint32_t)((int64_t)row * p.v.sn * C::ES + ((unit ^ v_swz<C>(row)) << 4))
                          : 0xFFFFFFF0u;
        }
        const float sc_raw = p.scale * p.k_descale * kLog2e;
        const float sc = sc_raw < 0.f ? -sc_raw : sc_raw == 0.f ? 1.f : sc_raw;

        // wave 0 describes block-local item k into descriptor e, then a
        // workgroup barrier (that does not wait for earlier output stores)
        // publishes it; wave 0 reads only the tables its own lanes wrote
        auto resolve = [&](int k, int e) {
            if (wave == 0) describe(p, sd, k, s_ord, s_seq, lane, s_desc[e]);
            __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
            __asm__ volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            __asm__ volatile("" ::: "memory");
        };

        resolve(sd.first, 0);
        // the second item is fixed as well (first + gx); the claims number
        // the items from 2 gx on.  Lane 0 of wave 0 holds the last claim.
        // The claim is one atomic add by thread 0.  Its address is passed
        // through a vector register: with a uniform address the compiler
        // combines the atomic over the wave and reads its result right away,
        // waiting out the atomic's round trip; here the result is first
        // needed one item later.  (A global-memory pointer: a flat atomic
        // would make every later wait a full one.)
        __attribute__((address_space(1))) int* ctr = (__attribute__((address_space(1))) int*)sd.ctr;
        __asm__ volatile("" : "+v"(ctr));
        int claim = 0;
        int k_next = sd.first + sd.gx;
        int e = 0;
        bool primed = false;  // first tile copied and Q loaded by the previous item
        char* sa = st0;       // stage of the item's first tile
        char* sb = st1;
        QRegs qreg;
        while (__builtin_amdgcn_readfirstlane(s_desc[e][D_MORE]) != 0) {
            // the next item's map entry, then the claim for the one after it
            resolve(k_next, e ^ 1);
            if (tid == 0) claim = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            Ctx c;
            Item im;
            const bool has = build(p, s_desc[e], koff, voff, wave, lane, c, im);
            // prefetch when the next item has key tiles
            const bool pf = __builtin_amdgcn_readfirstlane(s_desc[e ^ 1][D_VALID]) != 0 &&
                            __builtin_amdgcn_readfirstlane(s_desc[e ^ 1][D_T0]) <
                                __builtin_amdgcn_readfirstlane(s_desc[e ^ 1][D_T1]);
            bool next_primed = false;
            if (has) {
                if (!primed) {
                    sa = st0;
                    sb = st1;
                    if (c.t0 < c.t1) P::dma_tile(p, c, c.t0, true, sa, wave);
                    load_q(p, im, lane, qreg);
                    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                    __syncthreads();
                }
                sign_q(sc_raw, qreg);
                ORegs o;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
                float m_run = -INFINITY, l_run = 0.f;
                sweep(p, c, sa, sb, qreg, sc, m_run, l_run, o, pf, s_desc[e ^ 1], koff, voff,
                      wave, lane);
                // the claim has long landed (the sweep ended with a full wait);
                // read before the output stores, after which the compiler
                // would wait for those too
                k_next = 2 * sd.gx + __builtin_amdgcn_readfirstlane(claim);
                const int ntiles = c.t1 - c.t0;
                next_primed = pf && ntiles > 0;
                // the last tile's stage (free after the sweep's last barrier);
                // the next item's first tile went into the other one
                char* last = (ntiles & 1) || ntiles == 0 ? sa : sb;
                char* other = (ntiles & 1) || ntiles == 0 ? sb : sa;
                epilogue(p, c, im, o, m_run, l_run, last, wave, lane);
                if (next_primed) {
                    sa = other;
                    sb = last;
                }
            }
            if (!has) k_next = 2 * sd.gx + __builtin_amdgcn_readfirstlane(claim);
            primed = next_primed;
            e ^= 1;
        }
    }

    // Output rows of the item: fp32 partials with (m, l) for the combine
    // kernel when the keys are split, else normalized rows through this
    // wave's slice of stage `os_stage` (whole-row 1 KiB stores).
    __device__ __forceinline__ static void epilogue(const AttnParams& p, const Ctx& c,
                                                    const Item& im, const ORegs& o, float m_run,
                                                    float l_run, char* os_stage, int wave, int lane) {
        // the lane index read again, opaque to the compiler: the epilogue's
        // addresses are then computed here, per item, rather than hoisted
        // out of the item loop and kept in registers through it
        __asm__ volatile("" : "+v"(lane));
        const int lr = lane & 31, lg = lane >> 5;
        const float l_tot = halves_sum(l_run);
        if (im.nsl > 1) {
            if (c.i < c.q_len) {
                const int64_t row = (p.q_packed ? (int64_t)im.q_start : (int64_t)c.b * p.n_q) + c.i;
                const int64_t slot = (row * p.hq + im.h) * p.n_splits + im.bz;
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
        const float factor = p.v_descale * (l_tot > 0.f ? 1.f / l_tot : 0.f);
        char* os = os_stage + wave * 32 * C::OROW;
        typedef TO TO4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                TO4 w;
#pragma unroll
                for (int u = 0; u < 4; ++u) w[u] = to_t(o[db][rq * 4 + u] * factor, (TO*)nullptr);
                const int ch = (db * 4 + rq) ^ P::o_swz(lr);
                *(TO4*)(os + lr * C::OROW + ch * 16 + lg * 8) = w;
            }
        // the wave's valid rows as a buffer window (32 rows span < 2^32
        // bytes: host-checked): stores of rows past them are dropped, so the
        // reads and the stores issue without branches
        const int nrows = max(0, min(32, c.q_len - c.wr0));
        const char* obase = im.obase + ((int64_t)im.h * p.o_sh + (int64_t)c.wr0 * p.o_sn) * 2;
        const __amdgpu_buffer_rsrc_t orr = make_rsrc(obase, rows_bytes(nrows, p.o_sn, D, 2));
        u32x4 w[C::OINS];
#pragma unroll
        for (int k = 0; k < C::OINS; ++k) {
            const int row = k * C::ORPI + lane / C::OCH;
            const int ch = lane % C::OCH;
            w[k] = *(const u32x4*)(os + row * C::OROW + ((ch ^ P::o_swz(row)) << 4));
        }
#pragma unroll
        for (int k = 0; k < C::OINS; ++k) {
            const int row = k * C::ORPI + lane / C::OCH;
            const int ch = lane % C::OCH;
            buf_store(orr, (uint32_t)((int64_t)row * p.o_sn * 2 + ch * 16), w[k]);
        }
    }
};

// Two workgroups per CU, as the one-shot kernel.
template <typename TI, int D>
__global__ __launch_bounds__(256, 2) void prefill_persist_kernel(AttnParams p) {
    typedef Persist<TI, D> K;
    __shared__ __attribute__((aligned(16))) char st0[K::P::SSTAGE];
    __shared__ __attribute__((aligned(16))) char st1[K::P::SSTAGE];
    K::run(p, st0, st1);
}

// Zeroes the claim counters before a launch (a kernel rather than a memset,
// so that the pair can be captured in a graph).
__global__ void prefill_sched_reset_kernel(int32_t* ctr, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) ctr[i] = 0;
}

}  // namespace gqa
