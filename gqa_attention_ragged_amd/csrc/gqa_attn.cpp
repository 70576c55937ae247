// gqa_attn.cpp -- host side of the C ABI declared in include/gqa_attn.h:
// argument validation, kernel selection, launch geometry, launches.
//
// The host never reads device memory: every geometry decision uses shapes
// only (T, B, N, H), and the kernels resolve the ragged lengths themselves.
#include "gqa_attn.h"
#include "gqa_kv_cache.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "launch.h"
#include "lengths.h"
#include "main_timer.h"

namespace {

thread_local char g_err[256];
thread_local int g_hip_err = 0;

// Main-kernel timing window (gqa_attn_timer_start / _stop): event pairs
// recorded around the main kernel of each call while the window is open.
// A call reserves its pair when it records the first event and closes it
// with the second (the reservation is per thread and per window, so calls
// on several threads never mix their pairs).
struct MainTimer {
    std::atomic<bool> on{false};
    std::mutex mu;
    std::vector<hipEvent_t> ev;  // pair i: ev[2i] before, ev[2i + 1] after
    std::vector<char> done;      // pair i has both events recorded
    int next = 0;                // pairs reserved
    unsigned gen = 0;            // window number
    hipError_t err = hipSuccess;
};
// this thread's open pair: (window number, pair index), index < 0: none
thread_local unsigned t_pair_gen = 0;
thread_local int t_pair = -1;
MainTimer& main_timer() {
    static MainTimer t;
    return t;
}
void destroy_events(MainTimer& t) {
    for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
    t.ev.clear();
}

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int elem_bytes(int dt) {
    switch (dt) {
    case GQA_DT_F16:
    case GQA_DT_BF16: return 2;
    case GQA_DT_FP8_E4M3: return 1;
    case GQA_DT_F32: return 4;
    case GQA_DT_BOOL: return 1;
    }
    return 0;
}

int elem_kind(int dt) {
    return dt == GQA_DT_F16 ? gqa::ELEM_F16 : dt == GQA_DT_BF16 ? gqa::ELEM_BF16 : gqa::ELEM_FP8;
}

int gcd(int a, int b) { return b ? gcd(b, a % b) : a; }

enum Kernel { K_NONE = 0, K_PREFILL = 1, K_DECODE = 2, K_PREFILL_PP = 3, K_PREFILL_PERSIST = 4 };

// Draft tokens per sequence the tree variants resolve.
constexpr int kMaxTreeDrafts = 128;
// Prefill grids of at least this many workgroups read their tile map from
// records written by the plan kernel (see plan_call).
constexpr int64_t kMinRecordWgs = 1024;
// Claim counters of the persistent prefill kernel at the head of its workspace.
constexpr size_t kSchedBytes = gqa::kSchedInts * sizeof(int32_t);

// Plan overrides for measurement, read from the environment once per
// process (the first call) rather than on every call.
struct EnvOverrides {
    int decode_split = 0;    // GQA_ATTN_DECODE_SPLIT: keys per decode split (0 = planner's)
    int prefill_splits = 0;  // GQA_ATTN_PREFILL_SPLITS: prefill key slices (0 = planner's)
    bool xcd_remap = true;   // GQA_ATTN_XCD_REMAP=0 turns the XCD-aware order off
    bool validate = false;   // GQA_ATTN_VALIDATE=1: device-side length checks before launching
    bool pingpong = false;   // GQA_ATTN_PINGPONG=1: the 8-wave ping-pong kernel where it applies
    bool persist = false;    // GQA_ATTN_PERSIST=1: the persistent prefill kernel where it applies
    bool records = true;     // GQA_ATTN_RECORDS=0: no tile-map records (every workgroup maps itself)
};

const EnvOverrides& env_overrides() {
    static const EnvOverrides env = [] {
        EnvOverrides e;
        if (const char* s = std::getenv("GQA_ATTN_DECODE_SPLIT")) {
            const int c = std::atoi(s);
            if (c >= 128 && c <= 8192 && (c & (c - 1)) == 0) e.decode_split = c;
        }
        if (const char* s = std::getenv("GQA_ATTN_PREFILL_SPLITS")) {
            const int v = std::atoi(s);
            if (v >= 1 && v <= 32) e.prefill_splits = v;
        }
        if (const char* s = std::getenv("GQA_ATTN_XCD_REMAP"))
            if (std::atoi(s) == 0) e.xcd_remap = false;
        if (const char* s = std::getenv("GQA_ATTN_VALIDATE")) e.validate = std::atoi(s) != 0;
        if (const char* s = std::getenv("GQA_ATTN_PINGPONG")) e.pingpong = std::atoi(s) != 0;
        if (const char* s = std::getenv("GQA_ATTN_PERSIST")) e.persist = std::atoi(s) != 0;
        if (const char* s = std::getenv("GQA_ATTN_RECORDS")) e.records = std::atoi(s) != 0;
        return e;
    }();
    return env;
}

struct Plan {
    Kernel kernel = K_NONE;
    gqa::AttnParams p{};
    int q_elem = 0, kv_elem = 0, head_dim = 0;
    int grid_x = 0, grid_y = 0;
    size_t workspace = 0;
    size_t part_bytes = 4;  // prefill split-KV: bytes per partial O element
    size_t rec_bytes = 0;   // prefill: per-workgroup records at the workspace's head
    gqa::LenCheck lc{};     // the call's device-side length preconditions
};

// Checks that a Q/K/V/Y tensor has the rank of its form and a contiguous,
// suitably aligned head_size dimension.
int check_tensor(const gqa_tensor_t& t, const char* name, int form) {
    if (!t.data) return fail(GQA_ERR_INVALID_ARG, "%s: null data pointer", name);
    const int want = form == GQA_FORM_PACKED_NHD ? 3 : 4;
    if (t.ndim != want)
        return fail(GQA_ERR_INVALID_ARG, "%s: rank %d, the %s form needs rank %d", name, t.ndim,
                    form == GQA_FORM_PACKED_NHD ? "packed_nhd" : "padded_bhnd", want);
    for (int d = 0; d < t.ndim; ++d)
        if (t.shape[d] < 0) return fail(GQA_ERR_INVALID_ARG, "%s: negative extent", name);
    if (t.stride[t.ndim - 1] != 1)
        return fail(GQA_ERR_INVALID_ARG, "%s: head_size dimension must be contiguous", name);
    const int es = elem_bytes(t.dtype);
    if (es == 0) return fail(GQA_ERR_INVALID_ARG, "%s: unknown dtype %d", name, t.dtype);
    const int64_t align_elems = 16 / es;
    if ((uintptr_t)t.data % 16)
        return fail(GQA_ERR_UNSUPPORTED, "%s: data pointer must be 16-byte aligned", name);
    for (int d = 0; d + 1 < t.ndim; ++d) {
        if (t.stride[d] < 0)
            return fail(GQA_ERR_UNSUPPORTED, "%s: negative stride %d", name, d);
        if (t.stride[d] % align_elems)
            return fail(GQA_ERR_UNSUPPORTED, "%s: stride %d (%lld) must be a multiple of 16 bytes",
                        name, d, (long long)t.stride[d]);
    }
    return GQA_OK;
}

// The kernels address one window of rows of a (sequence, head) through a
// buffer descriptor with a 32-bit range and 32-bit offsets: a query tile
// (32 rows), a key tile (64 rows) or a decode split.  The window's base is
// 64-bit, so a sequence may span any number of bytes, but `rows` consecutive
// rows of t (form's row stride) must lie within 2^32 bytes.
bool window_fits(const gqa_tensor_t& t, int form, int64_t rows) {
    const int64_t sn = form == GQA_FORM_PACKED_NHD ? t.stride[0] : t.stride[2];
    const int64_t es = elem_bytes(t.dtype), D = t.shape[t.ndim - 1];
    // (rows - 1) * sn * es + D * es < 2^32, without overflowing int64
    const double bytes = ((double)(rows - 1) * (double)sn + (double)D) * (double)es;
    return bytes < 4294967296.0 - 4096.0;
}

int plan_call(const gqa_attn_args_t* a, Plan* plan) {
    if (!a) return fail(GQA_ERR_INVALID_ARG, "args is null");
    const int qf = a->query_form;
    if ((qf != 0 && qf != 1) || (a->kv_form < 0 || a->kv_form > 2))
        return fail(GQA_ERR_INVALID_ARG, "query_form must be 0 or 1, kv_form 0, 1 or 2");
    // paged KV pools are rank-4 like the padded form; kf is the addressing
    // form used below (paged addressing is selected by `paged`)
    const bool paged = a->kv_form == GQA_FORM_PAGED;
    const int kf = paged ? GQA_FORM_PADDED_BHND : a->kv_form;
    if (a->causal_kind < 0 || a->causal_kind > 2)
        return fail(GQA_ERR_INVALID_ARG, "causal_kind must be 0, 1 or 2");
    if (a->norm != GQA_NORM_SOFTMAX && a->norm != GQA_NORM_NONE)
        return fail(GQA_ERR_INVALID_ARG, "norm must be softmax or none");
    if (a->qdq < 0 || a->qdq > 2) return fail(GQA_ERR_INVALID_ARG, "qdq must be 0, 1 or 2");

    int st;
    if ((st = check_tensor(a->q, "q", qf))) return st;
    if ((st = check_tensor(a->k, "k", kf))) return st;
    if ((st = check_tensor(a->v, "v", kf))) return st;
    if ((st = check_tensor(a->out, "out", qf))) return st;

    const int qdt = a->q.dtype, kdt = a->k.dtype;
    if (qdt != GQA_DT_F16 && qdt != GQA_DT_BF16 && qdt != GQA_DT_FP8_E4M3)
        return fail(GQA_ERR_INVALID_ARG, "q dtype must be f16, bf16 or fp8 e4m3");
    if (a->v.dtype != kdt) return fail(GQA_ERR_INVALID_ARG, "k and v dtypes differ");
    const bool kv_cache8 = kdt == GQA_DT_FP8_E4M3 && qdt != GQA_DT_FP8_E4M3;
    if (kdt != qdt && !kv_cache8)
        return fail(GQA_ERR_INVALID_ARG, "k/v dtype must equal q's, or be fp8 with 16-bit q");
    const int out_dt = qdt == GQA_DT_FP8_E4M3 ? GQA_DT_F16 : qdt;
    if (a->out.dtype != out_dt)
        return fail(GQA_ERR_INVALID_ARG, "out dtype must be %s",
                    out_dt == GQA_DT_F16 ? "f16" : "bf16");

    const int qn = a->q.ndim, kn = a->k.ndim;
    const int64_t D = a->q.shape[qn - 1];
    if (a->k.shape[kn - 1] != D || a->v.shape[kn - 1] != D)
        return fail(GQA_ERR_INVALID_ARG, "head_size of q, k and v differ");
    for (int d = 0; d < qn; ++d)
        if (a->out.shape[d] != a->q.shape[d])
            return fail(GQA_ERR_INVALID_ARG, "out shape must equal q's shape");
    const int64_t Hq = a->q.shape[1], Hkv = a->k.shape[1];
    if (a->num_heads != Hq) return fail(GQA_ERR_INVALID_ARG, "num_heads != q's head dimension");
    if (a->kv_num_heads != Hkv || a->v.shape[1] != Hkv)
        return fail(GQA_ERR_INVALID_ARG, "kv_num_heads != k/v head dimension");
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv)
        return fail(GQA_ERR_INVALID_ARG, "num_heads must be a positive multiple of kv_num_heads");
    for (int d = 0; d < kn; ++d)
        if (a->v.shape[d] != a->k.shape[d]) return fail(GQA_ERR_INVALID_ARG, "k and v shapes differ");

    const int64_t B = a->batch;
    if (B < 0) return fail(GQA_ERR_INVALID_ARG, "batch must be >= 0");
    if (qf == GQA_FORM_PADDED_BHND && a->q.shape[0] != B)
        return fail(GQA_ERR_INVALID_ARG, "batch != q.shape[0]");
    if (kf == GQA_FORM_PADDED_BHND && !paged && a->k.shape[0] != B)
        return fail(GQA_ERR_INVALID_ARG, "batch != k.shape[0]");
    int page_shift = 0;
    if (paged) {
        if (!a->kv_lengths) return fail(GQA_ERR_INVALID_ARG, "kv_lengths is required for paged KV");
        if (!a->kv_page_table || a->kv_max_pages < 1)
            return fail(GQA_ERR_INVALID_ARG, "paged KV needs kv_page_table and kv_max_pages >= 1");
        const int64_t ps = a->k.shape[2];
        while (page_shift < 30 && (int64_t{1} << page_shift) < ps) ++page_shift;
        if (ps < 32 || (int64_t{1} << page_shift) != ps)
            return fail(GQA_ERR_UNSUPPORTED, "page_size must be a power of two >= 32");
        if ((int64_t)a->kv_max_pages * ps > INT32_MAX)
            return fail(GQA_ERR_UNSUPPORTED, "kv_max_pages * page_size beyond int32");
    } else if (a->kv_page_table) {
        return fail(GQA_ERR_INVALID_ARG, "kv_page_table given without the paged KV form");
    }
    if (qf == GQA_FORM_PACKED_NHD && !a->query_lengths)
        return fail(GQA_ERR_INVALID_ARG, "query_lengths is required for packed_nhd Q");
    if (kf == GQA_FORM_PACKED_NHD && !a->kv_lengths)
        return fail(GQA_ERR_INVALID_ARG, "kv_lengths is required for packed_nhd KV");

    const int64_t Nq = qf == GQA_FORM_PADDED_BHND ? a->q.shape[2] : 0;
    // paged: the logical key extent of a sequence is kv_max_pages pages
    const int64_t Nkv = paged ? (int64_t)a->kv_max_pages * a->k.shape[2]
                              : (kf == GQA_FORM_PADDED_BHND ? a->k.shape[2] : 0);
    const int64_t Tq = qf == GQA_FORM_PACKED_NHD ? a->q.shape[0] : 0;
    const int64_t Tkv = kf == GQA_FORM_PACKED_NHD ? a->k.shape[0] : 0;
    const int64_t kv_max = kf == GQA_FORM_PADDED_BHND ? Nkv : Tkv;
    if (Nq > INT32_MAX || Nkv > INT32_MAX || Tq > INT32_MAX || Tkv > INT32_MAX || B > 65535)
        return fail(GQA_ERR_UNSUPPORTED, "extents beyond the int32 / grid limits of this build");
    if (!window_fits(a->q, qf, 32))
        return fail(GQA_ERR_UNSUPPORTED, "q: 32 rows span 4 GiB or more (row stride too large)");
    // key windows: a 64-key tile (prefill), a split of up to 8192 keys plus
    // the prefetch of up to two tiles of the 4 waves past its end (decode)
    const int64_t kv_window = 8192 + 512;
    if (!window_fits(a->k, kf, kv_window) || !window_fits(a->v, kf, kv_window))
        return fail(GQA_ERR_UNSUPPORTED, "k/v: %lld rows span 4 GiB or more (row stride too large)",
                    (long long)kv_window);

    if (a->qdq != GQA_QDQ_OFF && !(a->qscale > 0.f && std::isfinite(a->qscale)))
        return fail(GQA_ERR_INVALID_ARG, "qscale must be finite and > 0 when qdq is on");
    if (!std::isfinite(a->scale) || !std::isfinite(a->k_descale) || !std::isfinite(a->v_descale))
        return fail(GQA_ERR_INVALID_ARG, "scale / descales must be finite");

    // mask
    gqa::AttnParams& p = plan->p;
    p = gqa::AttnParams{};
    p.mask_kind = gqa::MASK_NONE;
    const gqa_tensor_t& m = a->attn_mask;
    int64_t mask_q = 0, mask_kv = 0;  // mask extents that must cover the lengths
    if (m.data) {
        if (m.ndim < 1 || m.ndim > 4) return fail(GQA_ERR_INVALID_ARG, "attn_mask rank must be 1..4");
        switch (m.dtype) {
        case GQA_DT_BOOL: p.mask_kind = gqa::MASK_BOOL; break;
        case GQA_DT_F16: p.mask_kind = gqa::MASK_F16; break;
        case GQA_DT_BF16: p.mask_kind = gqa::MASK_BF16; break;
        case GQA_DT_F32: p.mask_kind = gqa::MASK_F32; break;
        default: return fail(GQA_ERR_INVALID_ARG, "attn_mask dtype must be bool, f16, bf16 or f32");
        }
        int64_t ext[4] = {1, 1, 1, 1}, str[4] = {0, 0, 0, 0};
        for (int d = 0; d < m.ndim; ++d) {
            ext[4 - m.ndim + d] = m.shape[d];
            str[4 - m.ndim + d] = m.shape[d] == 1 ? 0 : m.stride[d];
            if (m.shape[d] < 1) return fail(GQA_ERR_INVALID_ARG, "attn_mask has an empty dimension");
            if (m.stride[d] < 0 && m.shape[d] != 1)
                return fail(GQA_ERR_UNSUPPORTED, "attn_mask: negative stride %d", d);
        }
        if (ext[0] != 1 && ext[0] != B) return fail(GQA_ERR_INVALID_ARG, "attn_mask batch extent");
        if (ext[1] != 1 && ext[1] != Hq) return fail(GQA_ERR_INVALID_ARG, "attn_mask head extent");
        if (qf == GQA_FORM_PADDED_BHND && !a->query_lengths && ext[2] != 1 && ext[2] < Nq)
            return fail(GQA_ERR_INVALID_ARG, "attn_mask query extent < N_q");
        if (kf == GQA_FORM_PADDED_BHND && !a->kv_lengths && ext[3] != 1 && ext[3] < Nkv)
            return fail(GQA_ERR_INVALID_ARG, "attn_mask key extent < N_kv");
        mask_q = ext[2] != 1 ? ext[2] : 0;
        mask_kv = ext[3] != 1 ? ext[3] : 0;
        p.mask = m.data;
        p.m_sb = str[0];
        p.m_sh = str[1];
        p.m_si = str[2];
        p.m_sj = str[3];
        const int mes = elem_bytes(m.dtype);
        p.mask_vec = str[3] == 1 && ((uintptr_t)m.data % (4 * mes)) == 0 && str[0] % 4 == 0 &&
                     str[1] % 4 == 0 && str[2] % 4 == 0;
    }

    // the device-side preconditions on the lengths (checked on the GPU when
    // GQA_ATTN_VALIDATE=1, or on host copies by gqa_attn_check_lengths)
    {
        gqa::LenCheck& lc = plan->lc;
        lc = gqa::LenCheck{};
        lc.batch = (int32_t)B;
        lc.ql = a->query_lengths;
        lc.kl = a->kv_lengths;
        lc.ptab = paged ? a->kv_page_table : nullptr;
        lc.q_packed = qf == GQA_FORM_PACKED_NHD;
        lc.kv_packed = kf == GQA_FORM_PACKED_NHD;
        lc.kv_paged = paged;
        lc.ptab_pages = paged ? a->kv_max_pages : 0;
        lc.page_size = paged ? (int32_t)a->k.shape[2] : 0;
        lc.t_q = Tq;
        lc.t_kv = Tkv;
        lc.n_q = Nq;
        lc.n_kv = Nkv;
        lc.k_pages = paged ? a->k.shape[0] : 0;
        lc.v_pages = paged ? a->v.shape[0] : 0;
        lc.mask_q = mask_q;
        lc.mask_kv = mask_kv;
        lc.max_drafts = a->tree_parents ? kMaxTreeDrafts : 0;
    }

    // supported combinations
    if (D != 64 && D != 128) return fail(GQA_ERR_UNSUPPORTED, "head_size must be 64 or 128");
    // tree decoding: each wave resolves the ancestor chains of up to 128
    // drafts per sequence (two per lane)
    if (a->tree_parents && qf == GQA_FORM_PADDED_BHND && Nq > kMaxTreeDrafts)
        return fail(GQA_ERR_UNSUPPORTED, "tree_parents with padded Q needs N_q <= %d",
                    kMaxTreeDrafts);
    if (qdt == GQA_DT_FP8_E4M3 && a->qdq != GQA_QDQ_FP8_E4M3)
        return fail(GQA_ERR_UNSUPPORTED, "fp8 Q/K/V needs fp8 Q/DQ of the scores");
    const int64_t G = Hq / Hkv;
    const bool decode = qf == GQA_FORM_PADDED_BHND && Nq == 1 && !m.data &&
                        a->norm == GQA_NORM_SOFTMAX && a->qdq == GQA_QDQ_OFF &&
                        a->causal_kind != GQA_CAUSAL_UPPER_LEFT && G <= 16 &&
                        qdt != GQA_DT_FP8_E4M3;
    // an fp8 KV cache with 16-bit Q: the decode kernels, or the prefill kernels
    // that convert each K / V tile to 16 bits in LDS (online softmax)
    const bool kv8 = kv_cache8 && !decode;
    if (kv8 && (a->norm != GQA_NORM_SOFTMAX || a->qdq != GQA_QDQ_OFF))
        return fail(GQA_ERR_UNSUPPORTED,
                    "an fp8 KV cache with 16-bit Q needs softmax without Q/DQ");
    if (paged && !decode &&
        (a->norm != GQA_NORM_SOFTMAX || a->qdq != GQA_QDQ_OFF || a->k.shape[2] < 64))
        return fail(GQA_ERR_UNSUPPORTED,
                    "paged KV beyond the decode step needs softmax without Q/DQ and pages of "
                    ">= 64 keys");

    // common parameters
    auto view = [](const gqa_tensor_t& t, int form) {
        gqa::TensorView v;
        v.ptr = t.data;
        if (form == GQA_FORM_PACKED_NHD) {
            v.sb = 0;
            v.sh = t.stride[1];
            v.sn = t.stride[0];
        } else {
            v.sb = t.stride[0];
            v.sh = t.stride[1];
            v.sn = t.stride[2];
        }
        return v;
    };
    p.q = view(a->q, qf);
    p.k = view(a->k, kf);
    p.v = view(a->v, kf);
    const gqa::TensorView ov = view(a->out, qf);
    p.out = a->out.data;
    p.o_sb = ov.sb;
    p.o_sh = ov.sh;
    p.o_sn = ov.sn;
    p.ql = a->query_lengths;
    p.kl = a->kv_lengths;
    // With one query row per sequence (the decode step) the row is its own
    // only draft and the tree rule allows every key: the tree has no effect.
    p.tree = a->tree_parents;
    p.kv_paged = paged;
    p.ptab = a->kv_page_table;
    p.ptab_pages = paged ? a->kv_max_pages : 0;
    p.page_shift = page_shift;
    p.q_packed = qf;
    p.kv_packed = kf;
    p.batch = (int)B;
    p.n_q = (int)Nq;
    p.n_kv = (int)Nkv;
    p.causal = a->causal_kind;
    p.norm_none = a->norm == GQA_NORM_NONE;
    p.qdq = a->qdq;
    p.scale = a->scale;
    p.qscale = a->qdq ? a->qscale : 1.f;
    // Softmax P <= 1, so x = P / qscale <= 1 / qscale (up to fp32 rounding):
    // when that stays below the rounding limit of the format (fp8 E4M3FN: 464,
    // int8: 127.5) the saturation of the quantizer can never act.
    p.qdq_nosat = a->norm == GQA_NORM_SOFTMAX && a->qdq != GQA_QDQ_OFF && a->qscale > 0.f &&
                  1.0 / (double)a->qscale <= (a->qdq == GQA_QDQ_FP8_E4M3 ? 460.0 : 127.0);
    p.k_descale = a->k_descale;
    p.v_descale = a->v_descale;
    p.hq = (int)Hq;
    p.hkv = (int)Hkv;
    p.group = (int)G;
    plan->q_elem = elem_kind(qdt);
    plan->kv_elem = elem_kind(kdt);
    plan->head_dim = (int)D;

    // nothing to compute
    if (B == 0 || (qf == GQA_FORM_PADDED_BHND && Nq == 0) ||
        (qf == GQA_FORM_PACKED_NHD && Tq == 0)) {
        plan->kernel = K_NONE;
        plan->workspace = 0;
        return GQA_OK;
    }

    if (decode) {
        // Keys per split: 4096 (measured best at 128 x 8 heads x 32k keys, for
        // fp16 and fp8 KV, against 512 .. 8192), halved while the grid has
        // fewer than 4096 workgroups; GQA_ATTN_DECODE_SPLIT (a power of two,
        // 128..8192) overrides the start value for tuning.
        int C = env_overrides().decode_split ? env_overrides().decode_split : 4096;
        auto nsplit = [&](int c) { return (kv_max + c - 1) / c; };
        while (C > 128 && B * Hkv * nsplit(C) < 4096) C /= 2;
        const int64_t S = kv_max > 0 ? nsplit(C) : 1;
        if (S > 65535) return fail(GQA_ERR_UNSUPPORTED, "too many KV splits");
        if (B > 65535) return fail(GQA_ERR_UNSUPPORTED, "decode batch above 65535");
        p.split_keys = C;
        p.n_splits = (int)S;
        plan->kernel = K_DECODE;
        plan->workspace = (size_t)B * Hq * S * (D + 2) * sizeof(float) + 256;
        return GQA_OK;
    }

    // The 8-wave ping-pong kernel (one workgroup per CU) takes 16-bit Q/K/V of
    // one type with online softmax and no mask, tree or paging; the 4-wave
    // kernel (two workgroups per CU) everything else.
    const bool plain16 = qdt != GQA_DT_FP8_E4M3 && kdt == qdt && a->norm == GQA_NORM_SOFTMAX &&
                         a->qdq == GQA_QDQ_OFF && !m.data && !a->tree_parents && !paged;
    const bool pp = env_overrides().pingpong && plain16;
    // The same plain case can run as a persistent kernel (two workgroups per
    // CU working through the row tiles, each prefetching its next item's
    // first K / V tile and Q rows during the current item's last tile):
    // faster on short sequences, slower on long ones, so opt-in.
    const bool persist = !pp && env_overrides().persist && plain16 && B <= 64 &&
                         window_fits(a->out, qf, 32);
    const int hw = gcd((int)G, 4);
    const int R = 32 * ((pp ? 8 : 4) / hw);
    p.heads_per_wg = hw;
    p.rows_per_wg = R;
    // Mask tiles shared by a workgroup's heads are staged through LDS when the
    // mask broadcasts over heads, is 1 or 2 bytes wide with contiguous keys
    // and 16-byte aligned rows whose key extent is a whole number of 16-byte
    // chunks (tiles are loaded in 16-byte chunks), and the workgroup covers
    // 32 rows; with tree decoding a mask is read per lane (the generic
    // variant carries the tree rule).
    p.mask_lds = 0;
    if (m.data && !a->tree_parents && !paged && !kv8 && R == 32 && p.m_sh == 0 && p.m_sj == 1 &&
        (p.mask_kind == gqa::MASK_BOOL || p.mask_kind == gqa::MASK_F16 ||
         p.mask_kind == gqa::MASK_BF16)) {
        const int64_t es = p.mask_kind == gqa::MASK_BOOL ? 1 : 2;
        // a staged tile's 32 rows are read through one 32-bit window
        const double span = (31.0 * (double)p.m_si + (double)m.shape[m.ndim - 1]) * (double)es;
        p.mask_lds = (uintptr_t)m.data % 16 == 0 && (p.m_si * es) % 16 == 0 &&
                     (p.m_sb * es) % 16 == 0 && (m.shape[m.ndim - 1] * es) % 16 == 0 &&
                     span < 4294967296.0 - 4096.0;
    }
    int64_t gx = qf == GQA_FORM_PADDED_BHND ? B * ((Nq + R - 1) / R) : (Tq + R - 1) / R + B;
    if (gx > INT32_MAX) return fail(GQA_ERR_UNSUPPORTED, "too many query tiles");
    plan->grid_x = (int)gx;
    plan->grid_y = (int)(Hq / hw);
    if (plan->grid_y > 65535) return fail(GQA_ERR_UNSUPPORTED, "too many heads");
    // MI355X has 8 XCDs (each with its own L2) that receive workgroup ids in
    // turn; the prefill kernel remaps ids so that an XCD works through whole
    // head groups when they divide evenly (GQA_ATTN_XCD_REMAP=0 turns it off).
    p.xcds = plan->grid_y % 8 == 0 && env_overrides().xcd_remap ? 8 : 0;
    plan->kernel = pp ? K_PREFILL_PP : persist ? K_PREFILL_PERSIST : K_PREFILL;
    plan->workspace = 0;
    p.n_splits = 1;
    p.split_keys = 0;
    // Split-KV for prefill: with too few query tiles to fill the GPU and long
    // key ranges (chunked context), the keys of each tile are divided among
    // several workgroups whose fp32 partials a combine kernel merges.  Only
    // for online softmax (Q/DQ needs the full row before quantizing).
    const int64_t wgs = (int64_t)plan->grid_x * plan->grid_y;
    const int64_t kv_tiles = (kv_max + 63) / 64;
    // Concurrent workgroups: two 4-wave workgroups per CU (256 CUs), or one
    // 8-wave ping-pong workgroup.
    const int64_t slots = pp ? 256 : 512;
    // Splitting pays while the workgroups fill the GPU about once (the
    // longest row tile then sets the time); the fp32 partials cost
    // rows * H_q * S * (D + 2) * 4 bytes written and read again.  Measured
    // on the chunked-context workload (576 workgroups at most, 496 with
    // work): no split 510 TFLOP/s, 2 slices 570, 3 slices 591, 4 slices 549;
    // tree decoding (512 workgroups): no split 662, 2 slices 650, 3 slices
    // 669.  At most 1.25 rounds of workgroups: slices for about 3 rounds.
    const bool can_split = a->norm == GQA_NORM_SOFTMAX && a->qdq == GQA_QDQ_OFF &&
                           qdt != GQA_DT_FP8_E4M3 && kv_tiles >= 8;
    // With padded Q the grid is exact (no ragged slack): when it fills most
    // of one round of workgroups, slices add partials and the merge but no
    // balance (tree decoding, 512 workgroups: one slice 731 TFLOP/s, three
    // 675); a packed grid is an upper bound and keeps the rule above.
    const bool full_round = qf == GQA_FORM_PADDED_BHND && wgs >= slots * 3 / 4 && wgs <= slots;
    if (can_split) {
        int64_t S = 1;
        if (wgs < slots * 5 / 4 && !full_round) {
            S = (3 * slots + wgs - 1) / wgs;
            S = std::min<int64_t>(S, std::min<int64_t>(kv_tiles / 4, 32));  // <= 64: combine kernel
        }
        // GQA_ATTN_PREFILL_SPLITS (1..32) overrides the slice count for tuning
        if (const int v = env_overrides().prefill_splits)
            S = std::min<int64_t>(v, std::max<int64_t>(kv_tiles, 1));
        if (S > 1) {
            const int64_t per_tiles = (kv_tiles + S - 1) / S;
            S = (kv_tiles + per_tiles - 1) / per_tiles;
            const int64_t rows = qf == GQA_FORM_PACKED_NHD ? Tq : B * Nq;
            p.n_splits = (int)S;
            p.split_keys = (int)(per_tiles * 64);
            // partial O and (m, l) in fp32: the output is rounded once, in
            // the merge
            plan->part_bytes = 4;
            plan->workspace = (size_t)rows * Hq * S * (D * plan->part_bytes + 2 * sizeof(float)) + 256;
        }
    }
    // the remap linearizes the grid in 32-bit arithmetic
    if ((int64_t)plan->grid_x * plan->grid_y * p.n_splits > INT32_MAX) p.xcds = 0;
    p.grid_x = plan->grid_x;
    p.grid_y = plan->grid_y;
    p.kv8 = kv8;
    // The 4-wave kernel with at most 64 sequences reads its tile map from
    // per-workgroup records that a plan kernel writes once per call (the
    // sort and remap that every workgroup would otherwise repeat: about 1.9
    // of a workgroup's 5.3 us outside the key loop); they lead the
    // workspace.  Worth the extra launch (about 5 us) from two rounds of
    // workgroups on, without split-KV: measured 64 x 128 tokens +16%, 64 x
    // 256 +7%, 64 x 512 +4%, quantized with mask +1.4%, the ragged causal
    // prefill within noise; a 6-workgroup call -18%, and split-KV grids
    // (one to three rounds of workgroups plus the merge) -0.6%.
    const int64_t n_wg = (int64_t)plan->grid_x * plan->grid_y * std::max(p.n_splits, 1);
    if (plan->kernel == K_PREFILL && B <= 64 && p.n_splits <= 1 && n_wg >= kMinRecordWgs &&
        env_overrides().records) {
        plan->rec_bytes =
            ((size_t)n_wg * gqa::kWorkRecInts * sizeof(int32_t) + 255) & ~(size_t)255;
        plan->workspace = plan->rec_bytes + (plan->workspace ? plan->workspace : 256);
    }
    if (plan->kernel == K_PREFILL_PERSIST) {
        // the claim counters lead the workspace (the split partials, if
        // any, follow them)
        if ((int64_t)plan->grid_x * plan->grid_y * std::max(p.n_splits, 1) > INT32_MAX)
            return fail(GQA_ERR_UNSUPPORTED, "too many work items");
        plan->workspace = kSchedBytes + (plan->workspace ? plan->workspace : 256);
    }
    return GQA_OK;
}

}  // namespace

namespace gqa {
void main_kernel_begin(hipStream_t stream) {
    t_pair = -1;
    MainTimer& t = main_timer();
    if (!t.on.load(std::memory_order_acquire)) return;
    std::lock_guard<std::mutex> g(t.mu);
    if (!t.on.load(std::memory_order_relaxed) || 2 * t.next >= (int)t.ev.size()) return;
    const hipError_t e = hipEventRecord(t.ev[2 * t.next], stream);
    if (e != hipSuccess) {
        t.err = e;
        return;
    }
    t_pair = t.next++;
    t_pair_gen = t.gen;
}
void main_kernel_end(hipStream_t stream) {
    const int i = t_pair;
    t_pair = -1;
    if (i < 0) return;
    MainTimer& t = main_timer();
    std::lock_guard<std::mutex> g(t.mu);
    if (!t.on.load(std::memory_order_relaxed) || t_pair_gen != t.gen) return;  // window closed
    const hipError_t e = hipEventRecord(t.ev[2 * i + 1], stream);
    if (e != hipSuccess) t.err = e;
    else t.done[i] = 1;
}
}  // namespace gqa

extern "C" {

int gqa_attn_validate(const gqa_attn_args_t* args) {
    Plan plan;
    return plan_call(args, &plan);
}

int gqa_attn_workspace_size(const gqa_attn_args_t* args, size_t* bytes) {
    Plan plan;
    const int st = plan_call(args, &plan);
    if (st == GQA_OK && bytes) *bytes = plan.workspace;
    return st;
}

int gqa_attn_check_lengths(const gqa_attn_args_t* args, const int32_t* query_lengths_host,
                           const int32_t* kv_lengths_host, const int32_t* kv_page_table_host) {
    Plan plan;
    const int st = plan_call(args, &plan);
    if (st != GQA_OK) return st;
    gqa::LenCheck lc = plan.lc;
    if ((lc.ql && !query_lengths_host) || (lc.kl && !kv_lengths_host) ||
        (lc.ptab && !kv_page_table_host))
        return fail(GQA_ERR_INVALID_ARG, "a host copy of every length array the call uses is needed");
    lc.ql = lc.ql ? query_lengths_host : nullptr;
    lc.kl = lc.kl ? kv_lengths_host : nullptr;
    lc.ptab = lc.ptab ? kv_page_table_host : nullptr;
    uint32_t e = 0;
    for (int b = 0; b < lc.batch; ++b) e |= gqa::check_sequence(lc, b);
    if (e) return fail(GQA_ERR_INVALID_ARG, "lengths: %s", gqa::len_error_text(e));
    return GQA_OK;
}

namespace {

// Launch a planned call with the given workspace (the caller's, or the
// library's static one).
// Compute units of the current device (the persistent prefill grid is two
// workgroups per CU); 256, MI355X's count, if the query fails.
int device_cus() {
    static std::atomic<int> cache[256];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return 256;
    int v = cache[dev].load();
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
        v = 256;
    cache[dev].store(v);
    return v;
}

int forward_planned(const gqa_attn_args_t* args, Plan& plan, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (plan.kernel == K_NONE) return GQA_OK;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (env_overrides().validate && plan.lc.batch > 0) {
        // debug mode: check the lengths on the device, wait for the verdict,
        // and launch nothing if they break a precondition
        uint32_t* status = nullptr;
        uint32_t bits = 0;
        e = gqa::length_status_ptr(&status);
        if (e == hipSuccess) e = gqa::launch_length_check(plan.lc, status, s);
        if (e == hipSuccess) e = hipMemcpyAsync(&bits, status, sizeof bits, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) {
            g_hip_err = (int)e;
            return fail(GQA_ERR_HIP, "length check failed: %s", hipGetErrorString(e));
        }
        if (bits) return fail(GQA_ERR_INVALID_ARG, "lengths (device check): %s",
                              gqa::len_error_text(bits));
    }
    if (plan.kernel == K_DECODE) {
        if (!workspace || workspace_bytes < plan.workspace)
            return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes needed", plan.workspace);
        uintptr_t w = ((uintptr_t)workspace + 255) & ~(uintptr_t)255;
        const int64_t slots = (int64_t)plan.p.batch * plan.p.hq * plan.p.n_splits;
        plan.p.part_o = (float*)w;
        plan.p.part_ml = (float*)(w + (size_t)slots * plan.head_dim * sizeof(float));
        e = gqa::launch_decode(plan.p, plan.q_elem, plan.kv_elem, plan.head_dim, s);
    } else {
        const bool persist = plan.kernel == K_PREFILL_PERSIST;
        if (persist || plan.p.n_splits > 1) {
            if (!workspace || workspace_bytes < plan.workspace)
                return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes needed", plan.workspace);
        }
        uintptr_t w = ((uintptr_t)workspace + 255) & ~(uintptr_t)255;
        // the per-workgroup records need the whole workspace; without one a
        // call without split-KV runs with the map built in every workgroup
        const bool recs = plan.rec_bytes && workspace && workspace_bytes >= plan.workspace;
        plan.p.wrec = nullptr;
        if (recs) {
            plan.p.wrec = (const int32_t*)w;
            w += plan.rec_bytes;
        }
        if (persist) {
            plan.p.sched = (int32_t*)w;
            w += kSchedBytes;
        }
        if (plan.p.n_splits > 1) {
            const int64_t rows = plan.p.q_packed ? args->q.shape[0]
                                                 : (int64_t)plan.p.batch * plan.p.n_q;
            const int64_t slots = rows * plan.p.hq * plan.p.n_splits;
            plan.p.part_o = (float*)w;
            plan.p.part_ml = (float*)(w + (size_t)slots * plan.head_dim * plan.part_bytes);
        }
        if (plan.kernel == K_PREFILL_PERSIST) {
            // two workgroups per CU (at most one per work item); the XCD
            // order needs a workgroup on every XCD
            const int64_t items = (int64_t)plan.grid_x * plan.grid_y * std::max(plan.p.n_splits, 1);
            const int wgs = (int)std::min<int64_t>(items, 2 * (int64_t)device_cus());
            if (wgs < 8) plan.p.xcds = 0;
            e = gqa::launch_prefill_persist(plan.p, plan.q_elem, plan.head_dim, wgs, s);
        } else if (plan.kernel == K_PREFILL_PP)
            e = gqa::launch_prefill_pp(plan.p, plan.q_elem, plan.head_dim, plan.grid_x, plan.grid_y, s);
        else {
            if (recs) {
                const int n_wg = plan.grid_x * plan.grid_y * std::max(plan.p.n_splits, 1);
                e = gqa::launch_prefill_plan(plan.p, (int32_t*)plan.p.wrec, n_wg, s);
            }
            // one round of workgroups (two per CU): heavy and light work
            // items share the CUs (the kernel's in-grid map)
            const int64_t n_wg = (int64_t)plan.grid_x * plan.grid_y * std::max(plan.p.n_splits, 1);
            plan.p.mirror = !recs && n_wg <= 2 * (int64_t)device_cus();
            if (e == hipSuccess)
                e = gqa::launch_prefill(plan.p, plan.q_elem, plan.head_dim, plan.grid_x,
                                        plan.grid_y, s);
        }
    }
    if (e != hipSuccess) {
        g_hip_err = (int)e;
        return fail(GQA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return GQA_OK;
}

}  // namespace

int gqa_attn_forward(const gqa_attn_args_t* args, void* workspace, size_t workspace_bytes,
                     void* stream) {
    Plan plan;
    const int st = plan_call(args, &plan);
    if (st != GQA_OK) return st;
    return forward_planned(args, plan, workspace, workspace_bytes, stream);
}

int gqa_attn_forward_noalloc(const gqa_attn_args_t* args, void* stream) {
    Plan plan;
    const int st = plan_call(args, &plan);
    if (st != GQA_OK) return st;
    if (plan.workspace == 0) return forward_planned(args, plan, nullptr, 0, stream);
    if (plan.workspace > gqa::kStaticScratchBytes)
        return fail(GQA_ERR_WORKSPACE,
                    "the call needs %zu bytes of workspace; the static scratch buffer holds %zu "
                    "(use gqa_attn_forward with a caller workspace)",
                    plan.workspace, gqa::kStaticScratchBytes);
    void* scratch = nullptr;
    const hipError_t e = gqa::static_scratch_ptr(&scratch);
    if (e != hipSuccess) {
        g_hip_err = (int)e;
        return fail(GQA_ERR_HIP, "static scratch address: %s", hipGetErrorString(e));
    }
    return forward_planned(args, plan, scratch, gqa::kStaticScratchBytes, stream);
}

const char* gqa_attn_status_str(int status) {
    switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_INVALID_ARG: return "invalid argument";
    case GQA_ERR_UNSUPPORTED: return "unsupported combination";
    case GQA_ERR_WORKSPACE: return "workspace too small";
    case GQA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

// ------------------------------------------------------------ KV-cache update
namespace {

int plan_kv_update(const gqa_kv_update_args_t* a, gqa::KvUpdateParams* p) {
    if (!a) return fail(GQA_ERR_INVALID_ARG, "args is null");
    if (a->update_form != GQA_FORM_PADDED_BHND && a->update_form != GQA_FORM_PACKED_NHD)
        return fail(GQA_ERR_INVALID_ARG, "update_form must be 0 or 1");
    int st;
    if ((st = check_tensor(a->past_cache, "past_cache", GQA_FORM_PADDED_BHND))) return st;
    if ((st = check_tensor(a->update, "update", a->update_form))) return st;
    if ((st = check_tensor(a->out, "out", GQA_FORM_PADDED_BHND))) return st;
    const gqa_tensor_t &c = a->past_cache, &u = a->update, &y = a->out;
    const int dt = c.dtype;
    if (dt != GQA_DT_F16 && dt != GQA_DT_BF16 && dt != GQA_DT_FP8_E4M3)
        return fail(GQA_ERR_INVALID_ARG, "past_cache dtype must be f16, bf16 or fp8 e4m3");
    if (u.dtype != dt || y.dtype != dt)
        return fail(GQA_ERR_INVALID_ARG, "update and out must have past_cache's dtype");
    const int64_t B = c.shape[0], H = c.shape[1], N = c.shape[2], D = c.shape[3];
    for (int d = 0; d < 4; ++d)
        if (y.shape[d] != c.shape[d]) return fail(GQA_ERR_INVALID_ARG, "out must have past_cache's shape");
    const bool packed = a->update_form == GQA_FORM_PACKED_NHD;
    if (packed) {
        if (u.shape[1] != H || u.shape[2] != D)
            return fail(GQA_ERR_INVALID_ARG, "packed update must be [T, H, D] with the cache's H and D");
        if (!a->update_lengths)
            return fail(GQA_ERR_INVALID_ARG, "a packed update needs update_lengths");
    } else {
        if (u.shape[0] != B || u.shape[1] != H || u.shape[3] != D)
            return fail(GQA_ERR_INVALID_ARG, "padded update must be [B, H, N_u, D] with the cache's B, H, D");
    }
    const int es = elem_bytes(dt);
    if ((D * es) % 16) return fail(GQA_ERR_UNSUPPORTED, "D * element size must be a multiple of 16 bytes");
    if (B > INT32_MAX || H > INT32_MAX || N > INT32_MAX || (!packed && u.shape[2] > INT32_MAX))
        return fail(GQA_ERR_UNSUPPORTED, "extent above 2^31");
    const bool same = y.data == c.data;
    if (same)
        for (int d = 0; d < 4; ++d)
            if (y.stride[d] != c.stride[d])
                return fail(GQA_ERR_INVALID_ARG, "out aliases past_cache with different strides");
    *p = gqa::KvUpdateParams{};
    p->upd = (const char*)u.data;
    if (packed) {
        p->u_sb = 0;
        p->u_sh = u.stride[1];
        p->u_sn = u.stride[0];
        p->T = u.shape[0];
    } else {
        p->u_sb = u.stride[0];
        p->u_sh = u.stride[1];
        p->u_sn = u.stride[2];
        p->n_u = (int32_t)u.shape[2];
    }
    p->cache = (const char*)c.data;
    p->c_sb = c.stride[0];
    p->c_sh = c.stride[1];
    p->c_sn = c.stride[2];
    p->out = (char*)y.data;
    p->o_sb = y.stride[0];
    p->o_sh = y.stride[1];
    p->o_sn = y.stride[2];
    p->wi = a->write_indices;
    p->ul = a->update_lengths;
    p->packed = packed;
    p->B = (int32_t)B;
    p->H = (int32_t)H;
    p->N = (int32_t)N;
    p->es = es;
    p->row_bytes = (int32_t)(D * es);
    p->in_place = same;
    return GQA_OK;
}

}  // namespace

int gqa_kv_cache_update_validate(const gqa_kv_update_args_t* args) {
    gqa::KvUpdateParams p;
    return plan_kv_update(args, &p);
}

int gqa_kv_cache_update(const gqa_kv_update_args_t* args, void* stream) {
    gqa::KvUpdateParams p;
    const int st = plan_kv_update(args, &p);
    if (st != GQA_OK) return st;
    const hipError_t e = gqa::launch_kv_update(p, (hipStream_t)stream);
    if (e != hipSuccess) {
        g_hip_err = (int)e;
        return fail(GQA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return GQA_OK;
}

int gqa_attn_timer_start(int max_launches) {
    if (max_launches <= 0) return fail(GQA_ERR_INVALID_ARG, "max_launches must be > 0");
    MainTimer& t = main_timer();
    std::lock_guard<std::mutex> g(t.mu);
    if (t.on.load()) return fail(GQA_ERR_INVALID_ARG, "a timing window is already open");
    t.ev.assign(2 * (size_t)max_launches, nullptr);
    for (size_t i = 0; i < t.ev.size(); ++i) {
        // timing-only events: no system-scope fence when they complete (its
        // cache writeback would be timed with the kernel and slow the next one)
        const hipError_t e = hipEventCreateWithFlags(&t.ev[i], hipEventDisableSystemFence);
        if (e != hipSuccess) {
            t.ev.resize(i);
            destroy_events(t);
            g_hip_err = (int)e;
            return fail(GQA_ERR_HIP, "hipEventCreateWithFlags: %s", hipGetErrorString(e));
        }
    }
    t.done.assign((size_t)max_launches, 0);
    t.next = 0;
    ++t.gen;
    t.err = hipSuccess;
    t.on.store(true, std::memory_order_release);
    return GQA_OK;
}

int gqa_attn_timer_stop(double* total_ms, int* launches) {
    if (!total_ms || !launches) return fail(GQA_ERR_INVALID_ARG, "null output pointer");
    MainTimer& t = main_timer();
    std::lock_guard<std::mutex> g(t.mu);
    if (!t.on.load()) return fail(GQA_ERR_INVALID_ARG, "no timing window is open");
    t.on.store(false, std::memory_order_release);
    hipError_t e = t.err;
    double sum = 0.0;
    int n = 0;
    for (int i = 0; i < t.next && e == hipSuccess; ++i) {
        if (!t.done[i]) continue;  // a call still between its two records
        e = hipEventSynchronize(t.ev[2 * i + 1]);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]);
        sum += ms;
        ++n;
    }
    destroy_events(t);
    t.done.clear();
    t.next = 0;
    if (e != hipSuccess) {
        g_hip_err = (int)e;
        return fail(GQA_ERR_HIP, "main-kernel timing: %s", hipGetErrorString(e));
    }
    *total_ms = sum;
    *launches = n;
    return GQA_OK;
}

const char* gqa_attn_last_error(void) { return g_err; }

int gqa_attn_last_hip_error(void) { return g_hip_err; }

int gqa_attn_abi_version(void) { return 6; }

}  // extern "C"
