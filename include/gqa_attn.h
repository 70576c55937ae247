/*
 * gqa_attn.h -- C ABI of the fused ragged GQA attention library (gfx950).
 *
 * The operator is the one defined on the onnx-tensorrt "TensorRT Custom
 * Operator Schemas" page:
 *   - TRT_Attention: BMM1 -> mask -> normalization -> BMM2, with Q and KV
 *     each in "padded_bhnd" [B,H,N,D] or "packed_nhd" [T,H,D] form
 *     (tensor format notation; attributes query_form / kv_form /
 *     causal_kind / TRT_normalization_op; inputs attn_mask, query_lengths,
 *     kv_lengths; output Y with Q's shape, form and dtype);
 *   - TRT_QuantizedAttention: the same plus a quantize-dequantize of the
 *     normalized scores between normalization and BMM2
 *     (normalization_quantize_to_type, normalization_quantize_scale), with
 *     grouped-query heads (q_num_heads / kv_num_heads).
 * The KV-cache data type option (FP16 or FP8) follows the TensorRT
 * Edge-LLM "TensorRT Plugins Guide" page, AttentionPlugin section; an FP8
 * cache carries one fp32 dequantization scale per tensor here.
 *
 * Conventions that the page leaves open (fixed here):
 *   - Y = softmax(scale * Q K^T * k_descale + additive_mask) (V * v_descale)
 *     with the grouped-query map  kv_head = q_head / (H_q / H_kv);
 *   - scale is always explicit: pass 1.0f for TRT_Attention's "no implicit
 *     scaling", 1/sqrt(D) for the ONNX default of the quantized op;
 *   - causal upper_left allows key j <= i, lower_right allows
 *     j <= i + kv_len_b - q_len_b (per-sequence valid lengths); both may be
 *     combined with a mask (bool: AND; additive: added after scaling; an
 *     additive -inf removes the key);
 *   - a mask of rank <= 4 is right-aligned to [B, H_q, Nq, Nkv]; size-1
 *     dimensions broadcast; (i, j) index the row / key within sequence b;
 *   - a query row with no allowed key produces zeros;
 *   - Q/DQ: x = P / qscale, round half to even, saturate (fp8 E4M3FN to
 *     +-448, int8 to [-128,127]), P' = code * qscale; applied to the
 *     normalized P, no renormalization;
 *   - output rows that are not valid (padded rows i >= q_len_b, packed rows
 *     beyond query_lengths[B]) are never written, and padding of Q/K/V is
 *     never read.
 *
 * Tree decoding (TensorRT Edge-LLM "TensorRT Plugins Guide", AttentionPlugin:
 * tree decoding attention, used by speculative decoding; tree parent data
 * follows the query rows).  With tree_parents given, the q_len_b query rows
 * of sequence b are draft tokens whose keys and values are the last q_len_b
 * valid KV rows (draft t at key kv_len_b - q_len_b + t).  tree_parents
 * holds, token-aligned with Q's rows, the parent draft of each token:
 * parent[t] in [0, t-1], any other value attaches the token to the
 * committed context.  Row i may attend every key j < kv_len_b - q_len_b and
 * the drafts on its own ancestor chain, itself included; the rule is ANDed
 * with causal_kind and the mask.
 *
 * Paged KV (TensorRT Edge-LLM "TensorRT Plugins Guide", AttentionPlugin
 * decoder tensor contract: kv_page_table [N, 2, max_pages_per_sequence], a
 * page-table view into resident paged KV pools).  With kv_form
 * GQA_FORM_PAGED, k and v are pools of pages [P, H_kv, page_size, D] (the
 * same shape; they may be one tensor), kv_page_table is [B, 2, kv_max_pages]
 * int32 and key j of sequence b is row j % page_size of page
 * kv_page_table[b][0][j / page_size] of k, and of page
 * kv_page_table[b][1][j / page_size] of v.  kv_lengths [B] is required.
 *
 * Ownership: the caller owns every buffer (all device pointers unless noted);
 * the library never allocates or frees device memory on the forward path and
 * launches asynchronously on the caller's stream (it synchronizes only in the
 * GQA_ATTN_VALIDATE=1 debug mode described at gqa_attn_forward).
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of tensors. */
typedef enum {
    GQA_DT_F16 = 0,      /* IEEE binary16 */
    GQA_DT_BF16 = 1,     /* bfloat16 */
    GQA_DT_FP8_E4M3 = 2, /* OCP FP8 E4M3FN (max 448, no inf) */
    GQA_DT_F32 = 3,      /* additive masks only */
    GQA_DT_BOOL = 4      /* one byte, nonzero = may attend; masks only */
} gqa_dtype_t;

/* GQA_FORM_PAGED is a KV form only: see "Paged KV" above. */
typedef enum { GQA_FORM_PADDED_BHND = 0, GQA_FORM_PACKED_NHD = 1, GQA_FORM_PAGED = 2 } gqa_form_t;
typedef enum {
    GQA_CAUSAL_NONE = 0,
    GQA_CAUSAL_UPPER_LEFT = 1,
    GQA_CAUSAL_LOWER_RIGHT = 2
} gqa_causal_t;
typedef enum { GQA_NORM_SOFTMAX = 0, GQA_NORM_NONE = 1 } gqa_norm_t;
typedef enum { GQA_QDQ_OFF = 0, GQA_QDQ_FP8_E4M3 = 1, GQA_QDQ_INT8 = 2 } gqa_qdq_t;

/* Status codes. Host-detectable errors are returned before any launch. */
typedef enum {
    GQA_OK = 0,
    GQA_ERR_INVALID_ARG = 1, /* shapes, ranks, forms, missing lengths, heads ... */
    GQA_ERR_UNSUPPORTED = 2, /* a valid combination this build has no kernel for */
    GQA_ERR_WORKSPACE = 3,   /* workspace missing or too small */
    GQA_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} gqa_status_t;

/* A strided tensor view.  Strides are in elements; the last (head_size)
 * dimension must have stride 1.  data == NULL marks an absent optional
 * tensor (attn_mask). */
typedef struct {
    void* data;
    int32_t dtype; /* gqa_dtype_t */
    int32_t ndim;
    int64_t shape[4];
    int64_t stride[4];
} gqa_tensor_t;

/* Everything one forward call needs except the workspace and stream.
 *
 * q:   padded [B, H_q, N_q, D] or packed [T_q, H_q, D]; f16, bf16 or fp8.
 * k,v: padded [B, H_kv, N_kv, D] or packed [T_kv, H_kv, D]; same dtype as
 *      q, or fp8 with f16/bf16 q (an FP8 KV cache, dequantized with
 *      k_descale / v_descale).
 * attn_mask: optional, rank 1..4, bool or f16/bf16/f32 additive.
 * query_lengths: device int32 [B+1], cumulative, starting at 0.  Required
 *      when q is packed; optional when padded (then rows i >= q_len_b are
 *      padding).
 * kv_lengths: device int32.  KV packed: cumulative [B+1], required.  KV
 *      padded: per-sequence lengths [B], optional (NULL = N_kv).
 * batch: B.  Must equal q.shape[0] / k.shape[0] for padded forms; when both
 *      forms are packed it is the only source of B on the host.
 * out: Y in q's form and shape; dtype of q, except f16 when q is fp8.
 * kv_page_table, kv_max_pages: paged KV only (device int32 [B, 2,
 *      kv_max_pages], contiguous).  page_size must be a power of two, >= 32
 *      for the decode step and >= 64 otherwise; paged KV supports softmax
 *      without Q/DQ.  Device-side preconditions: kv_len_b <= kv_max_pages *
 *      page_size and every page index a sequence uses lies in [0, P).
 * tree_parents: optional device int32, token-aligned with q's rows ([T_q]
 *      packed, [B, N_q] contiguous padded); see "Tree decoding" above.
 *      The kernels resolve the ancestor chains of up to 128 drafts per
 *      sequence: padded q needs N_q <= 128 (GQA_ERR_UNSUPPORTED otherwise);
 *      with packed q, the rows of a sequence past its 128th draft come out
 *      as NaN (a device-side precondition: see below).
 *
 * Strides: non-negative element strides.  The kernels read a query tile
 * (32 rows) and a key tile or decode split (up to 8704 rows) through 32-bit
 * buffer windows whose bases are 64-bit: a sequence may span any number of
 * bytes, but that many consecutive rows (row stride x element size) must
 * span less than 4 GiB (GQA_ERR_UNSUPPORTED otherwise).
 *
 * Device-side length preconditions (the host never reads device memory, so
 * gqa_attn_forward does not check them unless GQA_ATTN_VALIDATE=1 is set,
 * see below): lengths non-negative and monotone, query_lengths[0] =
 * kv_lengths[0] = 0 when cumulative, query_lengths[B] <= T_q, kv_lengths[B]
 * <= T_kv, q_len_b <= N_q and kv_len_b <= N_kv for padded forms (paged:
 * kv_max_pages * page_size), every page-table entry a sequence uses inside
 * its pool, the mask's query / key extents covering q_len_b / kv_len_b, and
 * with tree_parents q_len_b <= 128. */
typedef struct {
    gqa_tensor_t q, k, v;
    gqa_tensor_t attn_mask;
    gqa_tensor_t out;
    const int32_t* query_lengths;
    const int32_t* kv_lengths;
    int32_t batch;
    int32_t query_form;  /* gqa_form_t */
    int32_t kv_form;     /* gqa_form_t */
    int32_t causal_kind; /* gqa_causal_t */
    int32_t norm;        /* gqa_norm_t */
    int32_t qdq;         /* gqa_qdq_t */
    float scale;         /* multiplies Q K^T */
    float qscale;        /* normalization_quantize_scale; used iff qdq != OFF */
    float k_descale;     /* 1.0f unless K is an fp8 cache */
    float v_descale;     /* 1.0f unless V is an fp8 cache */
    int32_t num_heads;    /* H_q */
    int32_t kv_num_heads; /* H_kv; H_q % H_kv == 0 */
    const int32_t* tree_parents; /* NULL: no tree (ordinary attention) */
    const int32_t* kv_page_table; /* paged KV: [B, 2, kv_max_pages]; else NULL */
    int32_t kv_max_pages;
} gqa_attn_args_t;

/* Check every host-visible property of args; launches nothing, touches no
 * device memory.  Returns a gqa_status_t. */
int gqa_attn_validate(const gqa_attn_args_t* args);

/* Bytes of device workspace gqa_attn_forward needs for args (0 when the
 * selected kernels need none).  Returns a gqa_status_t; *bytes is written
 * on success.
 *
 * What it holds: the decode step's split-KV partials, or the prefill
 * split-KV partials; for prefill without split-KV, with at most 64
 * sequences and a grid of at least 1024 workgroups, 32 bytes per workgroup
 * (the tile map, computed once per call by a small plan kernel rather than
 * in every workgroup).  Such a call also runs when given no (or too little)
 * workspace: each workgroup then builds the map itself (the same map, so
 * the same results; slower on short sequences).
 *
 * The kernel plan (and with it the workspace size) is chosen per call from
 * the shapes.  Environment variables, read once per process (at the first
 * call), override it for measurement: GQA_ATTN_DECODE_SPLIT (keys per
 * decode split, a power of two in 128..8192), GQA_ATTN_PREFILL_SPLITS (key
 * slices of the prefill split-KV path, 1..32), GQA_ATTN_XCD_REMAP=0 (no
 * XCD-aware workgroup order) and GQA_ATTN_PINGPONG=1 (an experimental
 * 8-wave ping-pong prefill kernel for plain 16-bit softmax prefill without
 * mask, tree, paging or Q/DQ; slower than the default 4-wave kernel on
 * gfx950 today, kept for measurement) and GQA_ATTN_PERSIST=1 (a persistent
 * form of the 4-wave kernel for the same plain case with at most 64
 * sequences: two workgroups per CU claim row tiles in turn and prefetch the
 * next one's first K / V tile and Q rows; faster on short sequences, slower
 * on long ones; needs a workspace of its 512-byte claim counters) and
 * GQA_ATTN_RECORDS=0 (no tile-map records: every prefill workgroup builds
 * the map itself). */
int gqa_attn_workspace_size(const gqa_attn_args_t* args, size_t* bytes);

/* Compute Y = attention(args) on `stream` (a hipStream_t; NULL = the null
 * stream).  workspace: device memory of at least gqa_attn_workspace_size
 * bytes (may be NULL when that is 0), owned by the caller and not used by
 * any other in-flight call.  Returns GQA_OK once the kernels are enqueued;
 * a HIP launch error returns GQA_ERR_HIP (see gqa_attn_last_hip_error).
 *
 * Debug mode: with GQA_ATTN_VALIDATE=1 in the environment (read once per
 * process), each call first runs a one-workgroup kernel that checks the
 * device-side length preconditions above on the device arrays, waits for it
 * (the call then synchronizes `stream`, so it cannot be captured into a
 * graph) and returns GQA_ERR_INVALID_ARG, naming the violated condition in
 * gqa_attn_last_error, without launching any attention kernel.  The check
 * writes its result to one word of device memory per device held by the
 * library: calls that overlap on one device race on it. */
int gqa_attn_forward(const gqa_attn_args_t* args, void* workspace, size_t workspace_bytes,
                     void* stream);

/* gqa_attn_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the workspace (tile-map records and
 * split-KV partials) lives in a static
 * device buffer of the library, 128 MiB per device (allocated when the
 * library's code object is loaded on a device and held until the process
 * ends).  Calls whose plan needs more workspace than that (see
 * gqa_attn_workspace_size) return GQA_ERR_WORKSPACE before launching
 * anything.  The call allocates and frees nothing.  Every call on one device
 * shares that device's buffer: calls that overlap on one device (other
 * streams, other threads) race on it and must be serialized by the caller.
 * Same arguments, results and error codes as gqa_attn_forward otherwise. */
int gqa_attn_forward_noalloc(const gqa_attn_args_t* args, void* stream);

/* The device-side length preconditions above, checked on the host over host
 * copies of the call's length arrays (query_lengths_host, kv_lengths_host,
 * kv_page_table_host: the same contents as args->query_lengths,
 * args->kv_lengths and args->kv_page_table; each needed when that argument
 * is non-NULL).  For callers that hold the lengths on the host anyway; the
 * device check of GQA_ATTN_VALIDATE=1 evaluates the same predicate.  Also
 * runs every host check of gqa_attn_validate.  Returns GQA_OK or
 * GQA_ERR_INVALID_ARG (detail in gqa_attn_last_error); launches nothing. */
int gqa_attn_check_lengths(const gqa_attn_args_t* args, const int32_t* query_lengths_host,
                           const int32_t* kv_lengths_host, const int32_t* kv_page_table_host);

/* Timing of the main kernel, for measurement.  gqa_attn_timer_start opens a
 * window of at most max_launches (> 0) timed calls on the current device:
 * it creates 2 x max_launches HIP events, and every later gqa_attn_forward
 * or gqa_attn_forward_noalloc call records one pair of them on its stream,
 * right before and right after its main kernel (the prefill attention
 * kernel, or the decode split kernel; the tile-map plan kernel, the split-KV
 * merge, the decode combine and the length check fall outside), until the
 * pairs run out: later calls are not timed.  gqa_attn_timer_stop waits for
 * the recorded events, writes the summed main-kernel time in milliseconds
 * to *total_ms and the number of timed calls to *launches, destroys the
 * events and closes the window.  Errors: GQA_ERR_INVALID_ARG (max_launches
 * <= 0, a window already open or none open, a null output pointer),
 * GQA_ERR_HIP (creating, recording or timing the events failed; the window
 * is closed).  One window per process, shared by all threads: each call's
 * pair belongs to the calling thread, and a call still between its two
 * records when the window closes is not counted.  Not for calls under graph
 * capture (the event records would be captured with them). */
int gqa_attn_timer_start(int max_launches);
int gqa_attn_timer_stop(double* total_ms, int* launches);

/* Human-readable text of a status code (static storage). */
const char* gqa_attn_status_str(int status);

/* Detail of the last failing call on this thread (static per-thread
 * storage): which argument was rejected, or the HIP error string. */
const char* gqa_attn_last_error(void);

/* The hipError_t of the last GQA_ERR_HIP on this thread (0 if none). */
int gqa_attn_last_hip_error(void);

/* Library ABI version (bumped on any change of these declarations or of
 * those in gqa_kv_cache.h; 2 adds the KV-cache update, 3 tree_parents, 4 paged
 * KV, 5 gqa_attn_check_lengths and 128-draft trees, 6 the main-kernel timer). */
int gqa_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
