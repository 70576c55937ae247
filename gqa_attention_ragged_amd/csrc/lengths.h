// lengths.h -- the device-side preconditions of a forward call on its ragged
// lengths, as one predicate per sequence that runs on the host (over host
// copies of the length arrays) and on the GPU (over the device arrays, in
// the length-check kernel that GQA_ATTN_VALIDATE=1 adds before a launch).
//
// The lengths follow the onnx-tensorrt "TensorRT Custom Operator Schemas"
// page (TRT_Attention inputs query_lengths / kv_lengths: cumulative INT32
// lengths starting at 0 for a packed form, per-sequence lengths for padded
// KV), the mask extents its attn_mask input (broadcast to the attention
// shape), and the page table the TensorRT Edge-LLM "TensorRT Plugins Guide"
// (AttentionPlugin decoder tensor contract, kv_page_table).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// Violations, one bit each.
enum LenError : uint32_t {
    LEN_QL_START = 1u << 0,   // query_lengths[0] != 0
    LEN_QL_ORDER = 1u << 1,   // query_lengths decreasing
    LEN_QL_RANGE = 1u << 2,   // query_lengths[B] > T_q, or q_len_b > N_q (padded Q)
    LEN_KL_START = 1u << 3,   // packed KV: kv_lengths[0] != 0
    LEN_KL_ORDER = 1u << 4,   // packed KV: kv_lengths decreasing; padded: a negative length
    LEN_KL_RANGE = 1u << 5,   // kv_lengths[B] > T_kv, or kv_len_b > N_kv (padded / paged)
    LEN_MASK = 1u << 6,       // the mask's query / key extent does not cover q_len_b / kv_len_b
    LEN_PAGE = 1u << 7,       // a page-table entry a sequence uses is outside its pool
    LEN_TREE = 1u << 8,       // tree decoding with more drafts than the kernels resolve
};

// What the checks read: device pointers for the kernel, host copies for the
// host check.  Extents are those of the call's tensors.
struct LenCheck {
    int32_t batch;
    const int32_t* ql;   // cumulative [B+1], or null (padded Q: every row valid)
    const int32_t* kl;   // cumulative [B+1] (packed KV), [B] (padded / paged), or null
    const int32_t* ptab; // paged KV: [B, 2, ptab_pages]; else null
    int32_t q_packed, kv_packed, kv_paged;
    int32_t ptab_pages, page_size;
    int64_t t_q, t_kv;   // packed row counts
    int64_t n_q, n_kv;   // padded extents (paged: ptab_pages * page_size)
    int64_t k_pages, v_pages;  // paged: pages in the K / V pools
    int64_t mask_q, mask_kv;   // mask extents (0: no mask, or a broadcast dimension)
    int32_t max_drafts;        // tree decoding: drafts per sequence the kernels resolve; 0 = no tree
};

__host__ __device__ inline uint32_t check_sequence(const LenCheck& c, int b) {
    uint32_t e = 0;
    int64_t q_len = c.n_q, kv_len = c.n_kv;
    if (c.ql) {
        if (b == 0 && c.ql[0] != 0) e |= LEN_QL_START;
        q_len = (int64_t)c.ql[b + 1] - c.ql[b];
        if (q_len < 0) e |= LEN_QL_ORDER;
        if (c.q_packed) {
            if (b == c.batch - 1 && (int64_t)c.ql[c.batch] > c.t_q) e |= LEN_QL_RANGE;
        } else if (q_len > c.n_q) {
            e |= LEN_QL_RANGE;
        }
    }
    if (c.kv_packed) {
        if (b == 0 && c.kl[0] != 0) e |= LEN_KL_START;
        kv_len = (int64_t)c.kl[b + 1] - c.kl[b];
        if (kv_len < 0) e |= LEN_KL_ORDER;
        if (b == c.batch - 1 && (int64_t)c.kl[c.batch] > c.t_kv) e |= LEN_KL_RANGE;
    } else if (c.kl) {
        kv_len = c.kl[b];
        if (kv_len < 0) e |= LEN_KL_ORDER;
        if (kv_len > c.n_kv) e |= LEN_KL_RANGE;
    }
    if (c.mask_q > 0 && q_len > c.mask_q) e |= LEN_MASK;
    if (c.mask_kv > 0 && kv_len > c.mask_kv) e |= LEN_MASK;
    if (c.kv_paged && c.ptab && kv_len > 0 && kv_len <= c.n_kv) {
        const int64_t pages = (kv_len + c.page_size - 1) / c.page_size;
        const int32_t* row = c.ptab + (int64_t)b * 2 * c.ptab_pages;
        for (int64_t pg = 0; pg < pages; ++pg) {
            const int32_t pk = row[pg], pv = row[c.ptab_pages + pg];
            if (pk < 0 || pk >= c.k_pages || pv < 0 || pv >= c.v_pages) e |= LEN_PAGE;
        }
    }
    if (c.max_drafts > 0 && q_len > c.max_drafts) e |= LEN_TREE;
    return e;
}

// Text of the lowest violation bit.
inline const char* len_error_text(uint32_t e) {
    if (e & LEN_QL_START) return "query_lengths[0] must be 0";
    if (e & LEN_QL_ORDER) return "query_lengths must be non-decreasing";
    if (e & LEN_QL_RANGE) return "query lengths exceed q's rows (T_q or N_q)";
    if (e & LEN_KL_START) return "kv_lengths[0] must be 0 (packed KV)";
    if (e & LEN_KL_ORDER) return "kv_lengths must be non-decreasing (packed) / non-negative";
    if (e & LEN_KL_RANGE) return "kv lengths exceed k/v's rows (T_kv, N_kv or the pages)";
    if (e & LEN_MASK) return "attn_mask extents do not cover the query / key lengths";
    if (e & LEN_PAGE) return "kv_page_table entry outside the page pool";
    if (e & LEN_TREE) return "tree decoding: more drafts in a sequence than this build resolves";
    return "ok";
}

}  // namespace gqa
