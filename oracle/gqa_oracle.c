/*
 * gqa_oracle.c -- CPU oracle for the fused ragged GQA attention operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file; only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the GPU library.
 *
 * What it computes (plain fp64, one query row at a time, no blocking, no
 * online rescaling, no fusion):
 *
 *   Source: onnx-tensorrt "TensorRT Custom Operator Schemas" page,
 *   sections TRT_Attention (tensor format notation, attributes, inputs,
 *   outputs, restrictions) and TRT_QuantizedAttention (attributes
 *   normalization_quantize_to_type / TRT_normalization_op, input
 *   normalization_quantize_scale).
 *
 *   For every batch entry b, query head h and valid query row i:
 *     g      = h / (H_q / H_kv)                      (grouped-query head map)
 *     s_j    = scale * sum_d q_d * (k_jd * k_descale) + additive_mask(b,h,i,j)
 *     allow_j= j < kv_len_b  and causal_ok(i,j)  and bool_mask(b,h,i,j)
 *     softmax: P_j = exp(s_j - m) / sum_allowed exp(s_j - m), m = max allowed s
 *     none   : P_j = s_j
 *     Q/DQ   : x_j = P_j / qscale ; c_j = encode(x_j) ; P_j <- c_j * qscale
 *     O_d    = sum_allowed P_j * (v_jd * v_descale)
 *
 * Readings taken where the page is silent (each is listed in the design
 * notes with its justification):
 *   - scale multiplies the whole BMM1 output and the additive mask is added
 *     after it; TRT_Attention callers that want "no scaling" pass 1.0;
 *   - head map is contiguous groups, H_q % H_kv == 0;
 *   - upper_left: j <= i; lower_right: j <= i + kv_len_b - q_len_b, with the
 *     per-sequence valid lengths;
 *   - a mask of rank <= 4 is right-aligned to [B, H_q, Nq, Nkv]; a size-1
 *     dimension broadcasts; (i, j) are the row and key within sequence b;
 *   - mask and causal compose (AND for bool, causal exclusion then add for
 *     additive); an additive -inf entry removes the key;
 *   - a row with no allowed key outputs zeros;
 *   - Q/DQ divides by the scale, rounds half to even, saturates (fp8 E4M3FN
 *     to +-448, int8 to [-128, 127]), dequantizes by multiplying back, and
 *     is applied to the normalized P (final max and sum); no renormalization.
 *
 * Tree decoding (TensorRT Edge-LLM "TensorRT Plugins Guide", AttentionPlugin:
 * tree decoding attention for speculative decoding, with tree parent data
 * carried row by row alongside the query rows).  When tree parents are
 * given, the q_len_b query rows of sequence b are draft tokens whose keys
 * are the last q_len_b valid keys (draft t at key kv_len_b - q_len_b + t);
 * parent[t] in [0, t-1] names the draft it extends, any other value hangs
 * it off the committed context.  Row i may attend every context key
 * (j < kv_len_b - q_len_b) and the drafts on its own ancestor chain, itself
 * included; this rule is ANDed with the causal kind and the mask.
 *
 * Paged KV (TensorRT Edge-LLM "TensorRT Plugins Guide", AttentionPlugin
 * decoder tensor contract: kv_page_table [N, 2, max_pages_per_sequence], a
 * page-table view into resident paged KV pools).  K and V are pools of
 * pages [P, H_kv, page_size, D]; key j of sequence b is row j % page_size
 * of page kv_page_table[b][0][j / page_size] of the K pool, and of page
 * kv_page_table[b][1][j / page_size] of the V pool; kv_lengths [B] gives
 * the sequence lengths.
 *
 * Alongside O the oracle returns, per output element, the largest change a
 * different rounding of "ambiguous" quantization inputs could make
 * (|x - nearest rounding midpoint| <= amb_rel * |x|), so that a GPU result
 * that computes P in fp32 can be judged fairly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- dtype codes private to the oracle ------------------------------- */
enum { OR_F16 = 0, OR_BF16 = 1, OR_E4M3 = 2, OR_F32 = 3, OR_BOOL = 4, OR_F64 = 5 };
enum { OR_PADDED = 0, OR_PACKED = 1, OR_PAGED = 2 };
enum { OR_CAUSAL_NONE = 0, OR_CAUSAL_UPPER_LEFT = 1, OR_CAUSAL_LOWER_RIGHT = 2 };
enum { OR_NORM_SOFTMAX = 0, OR_NORM_NONE = 1 };
enum { OR_QDQ_OFF = 0, OR_QDQ_FP8 = 1, OR_QDQ_INT8 = 2 };

typedef struct {
    const void* data; /* host memory; NULL = absent */
    int32_t dtype;
    int32_t ndim;
    int64_t shape[4];
    int64_t stride[4]; /* in elements */
} or_tensor;

typedef struct {
    or_tensor q, k, v, mask;
    int32_t query_form, kv_form;
    const int32_t* query_lengths; /* cumulative [B+1] or NULL */
    const int32_t* kv_lengths;    /* packed KV: cumulative [B+1]; padded: [B] or NULL */
    int32_t batch;                /* B */
    int32_t causal_kind, norm, qdq;
    float scale, qscale, k_descale, v_descale;
    int32_t num_heads, kv_num_heads;
    double amb_rel;
    const int32_t* tree_parents; /* [T_q] (packed Q) or [B, N_q] (padded Q), or NULL */
    const int32_t* kv_page_table; /* paged KV: [B, 2, kv_max_pages] */
    int32_t kv_max_pages;
} or_args;

/* ---- exact decoding of the storage formats -------------------------- */
/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double dec_f16(uint16_t b) {
    int s = b >> 15, e = (b >> 10) & 31, m = b & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}
/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
static double dec_bf16(uint16_t b) {
    int s = b >> 15, e = (b >> 7) & 255, m = b & 127;
    double v;
    if (e == 0) v = ldexp((double)m, -133);
    else if (e == 255) v = m ? NAN : INFINITY;
    else v = ldexp((double)(128 + m), e - 134);
    return s ? -v : v;
}
/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 fraction bits; no
 * infinities; S.1111.111 is NaN; largest finite 448. */
static double dec_e4m3(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

static double load_elem(const or_tensor* t, int64_t off) {
    switch (t->dtype) {
    case OR_F16: return dec_f16(((const uint16_t*)t->data)[off]);
    case OR_BF16: return dec_bf16(((const uint16_t*)t->data)[off]);
    case OR_E4M3: return dec_e4m3(((const uint8_t*)t->data)[off]);
    case OR_F32: return (double)((const float*)t->data)[off];
    case OR_F64: return ((const double*)t->data)[off];
    case OR_BOOL: return ((const uint8_t*)t->data)[off] ? 1.0 : 0.0;
    }
    return NAN;
}

/* ---- quantization of the normalized scores ------------------------- */
/* The 127 non-negative finite E4M3FN values, ascending (codes 0x00..0x7E). */
static double e4m3_pos[127];
static int e4m3_ready = 0;
static void init_e4m3_table(void) {
    if (e4m3_ready) return;
    for (int c = 0; c < 127; ++c) e4m3_pos[c] = dec_e4m3((uint8_t)c);
    e4m3_ready = 1;
}

/* Round x to the nearest E4M3FN value, ties to the even code, saturating
 * at +-448.  Returns the value; *delta receives the gap to the other
 * neighbour when x lies within amb_rel*|x| of a rounding midpoint, else 0. */
static double q_fp8(double x, double amb_rel, double* delta) {
    *delta = 0.0;
    if (isnan(x)) return NAN;
    double a = fabs(x);
    double r;
    if (a >= e4m3_pos[126]) {
        r = e4m3_pos[126];
    } else {
        int lo = 0, hi = 126; /* invariant: pos[lo] <= a < pos[hi] */
        while (hi - lo > 1) {
            int mid = (lo + hi) / 2;
            if (e4m3_pos[mid] <= a) lo = mid; else hi = mid;
        }
        double vlo = e4m3_pos[lo], vhi = e4m3_pos[hi];
        double dlo = a - vlo, dhi = vhi - a;
        if (dlo < dhi) r = vlo;
        else if (dhi < dlo) r = vhi;
        else r = (lo % 2 == 0) ? vlo : vhi; /* tie: even mantissa */
        double midpt = 0.5 * (vlo + vhi);
        if (fabs(a - midpt) <= amb_rel * a) *delta = vhi - vlo;
    }
    return x < 0 ? -r : r;
}

/* Round half to even, then clamp to [-128, 127]. */
static double q_int8(double x, double amb_rel, double* delta) {
    *delta = 0.0;
    if (isnan(x)) return NAN;
    double f = floor(x);
    double frac = x - f;
    double r;
    if (frac < 0.5) r = f;
    else if (frac > 0.5) r = f + 1.0;
    else r = (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
    if (fabs(frac - 0.5) <= amb_rel * fabs(x) && f >= -128.0 && f + 1.0 <= 127.0) *delta = 1.0;
    if (r < -128.0) r = -128.0;
    if (r > 127.0) r = 127.0;
    return r;
}

/* ---- lengths and addressing ----------------------------------------- */
static int64_t q_len_of(const or_args* a, int b) {
    if (a->query_lengths) return (int64_t)a->query_lengths[b + 1] - a->query_lengths[b];
    return a->q.shape[2]; /* padded Q without lengths: the full N_q */
}
static int64_t kv_len_of(const or_args* a, int b) {
    if (a->kv_form == OR_PACKED) return (int64_t)a->kv_lengths[b + 1] - a->kv_lengths[b];
    if (a->kv_form == OR_PAGED) return a->kv_lengths[b];
    if (a->kv_lengths) return a->kv_lengths[b];
    return a->k.shape[2];
}
/* Offset (elements) of row (b, head, i) in a tensor of the given form. */
static int64_t row_off(const or_tensor* t, int form, const int32_t* cum, int b, int head, int64_t i) {
    if (form == OR_PACKED)
        return ((int64_t)cum[b] + i) * t->stride[0] + (int64_t)head * t->stride[1];
    return (int64_t)b * t->stride[0] + (int64_t)head * t->stride[1] + i * t->stride[2];
}
/* Offset (elements) of key row (b, kv head, j) of K (which = 0) or V (1);
 * paged KV looks the page up in the page table. */
static int64_t kv_row_off(const or_args* a, int which, int b, int head, int64_t j) {
    const or_tensor* t = which ? &a->v : &a->k;
    if (a->kv_form != OR_PAGED) return row_off(t, a->kv_form, a->kv_lengths, b, head, j);
    const int64_t ps = t->shape[2];
    const int32_t page = a->kv_page_table[((int64_t)b * 2 + which) * a->kv_max_pages + j / ps];
    return (int64_t)page * t->stride[0] + (int64_t)head * t->stride[1] + (j % ps) * t->stride[2];
}
/* Mask element (b, h, i, j): right-aligned broadcast, size-1 dims stride 0. */
static int64_t mask_off(const or_tensor* m, int b, int h, int64_t i, int64_t j) {
    int64_t idx[4] = {b, h, i, j};
    int64_t off = 0;
    int lead = 4 - m->ndim;
    for (int d = 0; d < m->ndim; ++d) {
        int64_t n = m->shape[d];
        if (n != 1) off += idx[lead + d] * m->stride[d];
    }
    return off;
}

/* Tree rule: may row i of sequence b attend key j?  Walks the parent chain
 * from draft i to the context; a parent outside [0, u-1] ends the chain. */
static int tree_allows(const or_args* a, int b, int64_t i, int64_t j, int64_t ql, int64_t kl) {
    const int64_t base = kl - ql;
    if (j < base) return 1;
    const int64_t t = j - base;
    const int64_t row0 = a->query_form == OR_PACKED ? (int64_t)a->query_lengths[b]
                                                     : (int64_t)b * a->q.shape[2];
    for (int64_t u = i; u >= 0;) {
        if (u == t) return 1;
        const int32_t par = a->tree_parents[row0 + u];
        u = (par >= 0 && par < u) ? (int64_t)par : -1;
    }
    return 0;
}

/* Host-side guard: every row the definition reads lies inside its tensor. */
static int rows_in_bounds(const or_args* a, int b, int64_t ql, int64_t kl) {
    if (ql < 0 || kl < 0) return 0;
    if (a->query_form == OR_PACKED) {
        if ((int64_t)a->query_lengths[b] + ql > a->q.shape[0]) return 0;
    } else if (ql > a->q.shape[2] || b >= a->q.shape[0]) return 0;
    if (a->kv_form == OR_PACKED) {
        if ((int64_t)a->kv_lengths[b] + kl > a->k.shape[0]) return 0;
    } else if (a->kv_form == OR_PAGED) {
        const int64_t ps = a->k.shape[2];
        if (!a->kv_page_table || ps != a->v.shape[2] || kl > (int64_t)a->kv_max_pages * ps) return 0;
        for (int64_t p = 0; p * ps < kl; ++p)
            for (int w = 0; w < 2; ++w) {
                const int32_t pg = a->kv_page_table[((int64_t)b * 2 + w) * a->kv_max_pages + p];
                if (pg < 0 || pg >= (w ? a->v.shape[0] : a->k.shape[0])) return 0;
            }
    } else if (kl > a->k.shape[2] || b >= a->k.shape[0]) return 0;
    if (a->mask.data) {
        int64_t need[4] = {b + 1, a->num_heads, ql, kl};
        int lead = 4 - a->mask.ndim;
        for (int d = 0; d < a->mask.ndim; ++d) {
            int64_t n = a->mask.shape[d];
            if (n != 1 && n < need[lead + d]) return 0;
        }
    }
    return 1;
}

/* ---- public entry points --------------------------------------------- */

/* Number of valid output rows (b, h, i) with i < q_len_b. */
int64_t oracle_count_rows(const or_args* a) {
    int64_t n = 0;
    for (int b = 0; b < a->batch; ++b) {
        int64_t ql = q_len_of(a, b);
        if (ql > 0) n += ql * a->num_heads;
    }
    return n;
}

/* Write the (b, h, i) triples of every valid output row, b-major then h then i. */
int64_t oracle_list_rows(const or_args* a, int32_t* rows, int64_t cap) {
    int64_t n = 0;
    for (int b = 0; b < a->batch; ++b) {
        int64_t ql = q_len_of(a, b);
        for (int h = 0; h < a->num_heads; ++h)
            for (int64_t i = 0; i < ql; ++i) {
                if (n < cap) {
                    rows[3 * n] = b; rows[3 * n + 1] = h; rows[3 * n + 2] = (int32_t)i;
                }
                ++n;
            }
    }
    return n;
}

/* Compute the output rows listed in rows[3*r .. 3*r+2] = (b, h, i).
 * out[r*D + d] = O (fp64), amb[r*D + d] = ambiguity bound, nallowed[r] =
 * number of allowed keys.  Returns 0, or a negative code on bad arguments. */
int oracle_rows(const or_args* a, const int32_t* rows, int64_t nrows, double* out, double* amb,
                int64_t* nallowed) {
    init_e4m3_table();
    if (a->num_heads <= 0 || a->kv_num_heads <= 0 || a->num_heads % a->kv_num_heads) return -1;
    const int64_t D = (a->query_form == OR_PACKED) ? a->q.shape[2] : a->q.shape[3];
    const int group = a->num_heads / a->kv_num_heads;
    const double scale = (double)a->scale, kd = (double)a->k_descale, vd = (double)a->v_descale;
    const double qs = (double)a->qscale;
    const int has_mask = a->mask.data != NULL;
    const int bool_mask = has_mask && a->mask.dtype == OR_BOOL;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 8) reduction(| : bad)
    for (int64_t r = 0; r < nrows; ++r) {
        const int b = rows[3 * r], h = rows[3 * r + 1];
        const int64_t i = rows[3 * r + 2];
        double* o = out + r * D;
        double* ab = amb + r * D;
        for (int64_t d = 0; d < D; ++d) { o[d] = 0.0; ab[d] = 0.0; }
        const int64_t ql = q_len_of(a, b), kl = kv_len_of(a, b);
        if (b < 0 || b >= a->batch || h < 0 || h >= a->num_heads || i < 0 || i >= ql ||
            !rows_in_bounds(a, b, ql, kl)) { bad = 1; continue; }
        const int g = h / group;
        const int64_t qo = row_off(&a->q, a->query_form, a->query_lengths, b, h, i);
        const int64_t n = kl > 0 ? kl : 0;
        double* s = (double*)malloc(sizeof(double) * (size_t)(n + 1));
        char* ok = (char*)malloc((size_t)(n + 1));

        /* BMM1, causal/length predicate, mask */
        for (int64_t j = 0; j < n; ++j) {
            int allowed = 1;
            if (a->causal_kind == OR_CAUSAL_UPPER_LEFT) allowed = (j <= i);
            else if (a->causal_kind == OR_CAUSAL_LOWER_RIGHT) allowed = (j <= i + (kl - ql));
            if (a->tree_parents) allowed = allowed && tree_allows(a, b, i, j, ql, kl);
            double add = 0.0;
            if (has_mask) {
                double mv = load_elem(&a->mask, mask_off(&a->mask, b, h, i, j));
                if (bool_mask) allowed = allowed && (mv != 0.0);
                else {
                    add = mv;
                    if (isinf(mv) && mv < 0) allowed = 0;
                }
            }
            ok[j] = (char)allowed;
            if (!allowed) { s[j] = 0.0; continue; }
            const int64_t ko = kv_row_off(a, 0, b, g, j);
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d)
                dot += load_elem(&a->q, qo + d * a->q.stride[a->query_form == OR_PACKED ? 2 : 3]) *
                       (load_elem(&a->k, ko + d * a->k.stride[a->kv_form == OR_PACKED ? 2 : 3]) * kd);
            s[j] = scale * dot + add;
        }

        /* normalization */
        int64_t cnt = 0;
        double mx = -INFINITY;
        for (int64_t j = 0; j < n; ++j)
            if (ok[j]) { ++cnt; if (s[j] > mx) mx = s[j]; }
        nallowed[r] = cnt;
        if (cnt == 0) { free(s); free(ok); continue; } /* no allowed key: zeros */
        if (a->norm == OR_NORM_SOFTMAX) {
            double l = 0.0;
            for (int64_t j = 0; j < n; ++j)
                if (ok[j]) { s[j] = exp(s[j] - mx); l += s[j]; }
            for (int64_t j = 0; j < n; ++j)
                if (ok[j]) s[j] /= l;
        }

        /* Q/DQ of the normalized scores, then BMM2 */
        for (int64_t j = 0; j < n; ++j) {
            if (!ok[j]) continue;
            double p = s[j], delta = 0.0;
            if (a->qdq == OR_QDQ_FP8) p = q_fp8(p / qs, a->amb_rel, &delta) * qs;
            else if (a->qdq == OR_QDQ_INT8) p = q_int8(p / qs, a->amb_rel, &delta) * qs;
            const int64_t vo = kv_row_off(a, 1, b, g, j);
            const int64_t vs = a->v.stride[a->kv_form == OR_PACKED ? 2 : 3];
            for (int64_t d = 0; d < D; ++d) {
                double vv = load_elem(&a->v, vo + d * vs) * vd;
                o[d] += p * vv;
                if (delta != 0.0) ab[d] += delta * qs * fabs(vv);
            }
        }
        free(s);
        free(ok);
    }
    return bad ? -2 : 0;
}

/* Exposed for the format pins: decode one code, encode one value. */
double oracle_decode(int32_t dtype, uint32_t bits) {
    switch (dtype) {
    case OR_F16: return dec_f16((uint16_t)bits);
    case OR_BF16: return dec_bf16((uint16_t)bits);
    case OR_E4M3: return dec_e4m3((uint8_t)bits);
    }
    return NAN;
}
double oracle_quantize(int32_t kind, double x, double amb_rel, double* delta) {
    init_e4m3_table();
    if (kind == OR_QDQ_FP8) return q_fp8(x, amb_rel, delta);
    if (kind == OR_QDQ_INT8) return q_int8(x, amb_rel, delta);
    *delta = 0.0;
    return x;
}
