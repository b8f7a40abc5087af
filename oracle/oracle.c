/*
 * oracle.c - plain fp64 reference for GQA attention forward and split-K
 * paged decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * What it computes is the plain definition of softmax attention, written out
 * row by row with the whole softmax row materialised: no tiling, no online
 * rescaling, no exp2 domain.  The method on the pages (a FlashAttention forward
 * with an online softmax) reaches exactly this result up to rounding order, so
 * the definition itself is the oracle.  Sources, by page:
 *
 *   [P1] causal_forward_kernel.py (flash-attention-scratch),
 *        `_flash_attention_forward_gqa_kernel`: query head h of a group reads
 *        K/V head h // (Hq/Hkv) ("Part 1" head mapping); S = scale * Q K^T;
 *        output O = softmax(S) V and a per-row log-sum-exp.
 *   [P2] gpt-o3 / triton6fd1ef (FlashInfer-style GQA prefill),
 *        `_gqa_prefill_kernel`: with delta = kv_len - q_len, query i sees
 *        the keys j < min(kv_len, i + 1 + delta) (bottom-right causal mask).
 *   [P4] splitk_kernels.py (xformers split-K), `_fwd_kernel_splitK`: the
 *        log-sum-exp is written in the natural base; a row or chunk with no
 *        visible key gives O = 0 (and its LSE is log(0) = -inf); K/V of a
 *        paged cache are found through a per-sequence block table;
 *        `_splitK_reduce`: partial results merge as
 *        M = max_s L_s, w_s = exp(L_s - M), O = sum w_s O_s / sum w_s,
 *        L = M + log(sum w_s), and (0, -inf) when every L_s is -inf;
 *        with HAS_ADDITIVE_BIAS a bias block (layout [B, G, H, Mq, N] by
 *        strides) is added to the scaled scores before the softmax;
 *        `_splitK_reduce_varargs_backward`: the gradients of that merge with
 *        respect to the partial results.
 *
 * Every input element is the exact value the GPU receives (fp64, fp32, fp16
 * or bf16 storage), widened to double here; all arithmetic is in double.
 *
 * Layouts (row-major, contiguous):
 *   dense  q [B, Hq, q_len, D], k/v [B, Hkv, kv_len, D]
 *   paged  k/v cache [num_pages, page_size, Hkv, D], block_table [B, max_pages]
 *   decode q [B, Hq, D]
 * A "row" is one (b, h, i) query; its flat id is (b * Hq + h) * q_len + i.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F64 = 0, ORACLE_F32 = 1, ORACLE_F16 = 2, ORACLE_BF16 = 3, ORACLE_FP8E4M3 = 4 };

/* ---- storage formats -> double ------------------------------------------ */

/* IEEE 754 binary16: sign, 5-bit exponent (bias 15), 10-bit fraction. */
static double half_bits_to_double(uint16_t h) {
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);            /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25); /* 1.m * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit float E4M3 ("fn" variant): sign, 4-bit exponent (bias 7), 3-bit
 * fraction; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no
 * infinities.  Largest finite value 448. */
static double e4m3_bits_to_double(uint8_t b) {
    int sign = b >> 7;
    int e = (b >> 3) & 0xf;
    int m = b & 0x7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(m | 0x8), e - 10);  /* 1.m * 2^(e-7) */
    return sign ? -v : v;
}

static double elem(const void* base, int64_t idx, int dt) {
    switch (dt) {
    case ORACLE_F64: return ((const double*)base)[idx];
    case ORACLE_F32: return (double)((const float*)base)[idx];
    case ORACLE_F16: return half_bits_to_double(((const uint16_t*)base)[idx]);
    case ORACLE_FP8E4M3: return e4m3_bits_to_double(((const uint8_t*)base)[idx]);
    default:         return bf16_bits_to_double(((const uint16_t*)base)[idx]);
    }
}

/* Exposed so the tests can check the widening against library conversions. */
void oracle_widen(const void* src, int dt, int64_t n, double* dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = elem(src, i, dt);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- one query row against an explicit list of key positions -------------
 *
 * Accessors give the flat element index of K/V token t, feature d, so the
 * same plain definition serves dense prefill, dense decode and paged decode.
 */
typedef struct {
    const void* k;
    const void* v;
    int dt;
    int D;
    /* dense: base offset of the (b, kv-head) slab; row stride D */
    int64_t dense_base;
    /* paged: block table row of this sequence, geometry of the pool */
    const int* bt_row;
    int page_size;
    int Hkv;
    int g;
    /* fp8 cache: per (token row, K/V head) a uint32 holding two binary16,
     * the scale in bits 0-15 and the shift in bits 16-31 ([P4]
     * `cast_uint32_to_half2`); NULL for an unquantized cache */
    const uint32_t* k_ss;
    const uint32_t* v_ss;
} kv_view;

static int64_t kv_index(const kv_view* kv, int64_t t, int d);

/* [P4] `dequantize` (fp8 branch): value = stored * scale + shift, with the
 * scale and shift of the element's token row and head; the index of that pair
 * is the element index divided by D (one pair per D-element row). */
static double kv_value(const kv_view* kv, const void* base, const uint32_t* ss, int64_t t, int d) {
    int64_t idx = kv_index(kv, t, d);
    double x = elem(base, idx, kv->dt);
    if (!ss) return x;
    uint32_t w = ss[idx / kv->D];
    return x * half_bits_to_double((uint16_t)(w & 0xffff)) + half_bits_to_double((uint16_t)(w >> 16));
}

static int64_t kv_index(const kv_view* kv, int64_t t, int d) {
    if (kv->bt_row) {
        /* [P4] paged branch: page = block_table[b, t / page_size],
         * row t % page_size inside it; pool is [page, row, Hkv, D]. */
        int64_t page = kv->bt_row[t / kv->page_size];
        int64_t row = t % kv->page_size;
        return ((page * kv->page_size + row) * kv->Hkv + kv->g) * (int64_t)kv->D + d;
    }
    return kv->dense_base + t * (int64_t)kv->D + d;
}

/* An additive bias row: the bias of key t is element off + t of p (in
 * storage format dt); p == NULL means no bias. */
typedef struct {
    const void* p;
    int dt;
    int64_t off;
} bias_view;

static const bias_view NO_BIAS = {NULL, 0, 0};

/*
 * Attention of one query over keys t in [lo, hi) that satisfy t < vis_end.
 * Steps, in the order of the definition:
 *   1. s_t = scale * sum_d q_d k_{t,d}  (+ bias_t when a bias is given: [P4]
 *      HAS_ADDITIVE_BIAS adds it to the scaled score, in the softmax's
 *      natural units)
 *   2. visible set V = { t in [lo, hi) : t < vis_end }
 *   3. V empty, or every s_t on V is -inf (a bias of -inf masks a key)
 *      -> O = 0, L = -inf
 *   4. m = max_{t in V} s_t, Z = sum_{t in V} exp(s_t - m), L = m + log Z
 *   5. P_t = exp(s_t - L) on V
 *   6. O = sum_{t in V} P_t v_t
 * `s` is caller scratch of at least hi - lo doubles.  If p_out is given,
 * P_t (0 outside V) is stored at p_out[t - lo].
 */
static void attend_one(const void* q, int64_t q_off, int q_dt, const kv_view* kv,
                       int64_t lo, int64_t hi, int64_t vis_end, double scale, bias_view bias,
                       double* s, double* o, double* lse, double* p_out) {
    const int D = kv->D;
    int64_t end = hi < vis_end ? hi : vis_end;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (p_out)
        for (int64_t t = lo; t < hi; ++t) p_out[t - lo] = 0.0;
    if (end <= lo) {
        *lse = -INFINITY;
        return;
    }
    for (int64_t t = lo; t < end; ++t) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += elem(q, q_off + d, q_dt) * kv_value(kv, kv->k, kv->k_ss, t, d);
        s[t - lo] = scale * acc;
        if (bias.p) s[t - lo] += elem(bias.p, bias.off + t, bias.dt);
    }
    double m = -INFINITY;
    for (int64_t t = lo; t < end; ++t)
        if (s[t - lo] > m) m = s[t - lo];
    if (m == -INFINITY) { *lse = m; return; }  /* every visible key masked by the bias */
    double z = 0.0;
    for (int64_t t = lo; t < end; ++t) z += exp(s[t - lo] - m);
    double L = m + log(z);
    *lse = L;
    for (int64_t t = lo; t < end; ++t) {
        double p = exp(s[t - lo] - L);
        if (p_out) p_out[t - lo] = p;
        for (int d = 0; d < D; ++d) o[d] += p * kv_value(kv, kv->v, kv->v_ss, t, d);
    }
}

static int check_fwd_args(int B, int Hq, int Hkv, int q_len, int kv_len, int D) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || q_len < 0 || kv_len < 0 || D <= 0) return 1;
    if (Hq % Hkv) return 1;
    return 0;
}

/*
 * Prefill / general forward.  [P1] head map, [P2] bottom-right causal mask,
 * [P4] natural-base LSE and empty-row convention.
 *
 * rows == NULL computes every row in flat order; otherwise rows[n] are flat
 * row ids.  o_out is [n_rows, D], lse_out is [n_rows].  Returns 0, or 1 on a
 * bad argument.
 */
int oracle_attn_fwd(const void* q, const void* k, const void* v, int dt,
                    int B, int Hq, int Hkv, int q_len, int kv_len, int D,
                    double scale, int causal,
                    const int64_t* rows, int64_t n_rows,
                    double* o_out, double* lse_out) {
    if (check_fwd_args(B, Hq, Hkv, q_len, kv_len, D)) return 1;
    const int64_t total = (int64_t)B * Hq * q_len;
    if (!rows) n_rows = total;
    const int group = Hq / Hkv;
    const int64_t delta = (int64_t)kv_len - q_len;
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t n = 0; n < n_rows; ++n) {
            int64_t r = rows ? rows[n] : n;
            if (r < 0 || r >= total) { bad = 1; continue; }
            int64_t i = r % q_len;
            int64_t bh = r / q_len;
            int h = (int)(bh % Hq);
            int b = (int)(bh / Hq);
            int g = h / group;
            kv_view kv = {k, v, dt, D, ((int64_t)b * Hkv + g) * kv_len * (int64_t)D,
                          NULL, 0, Hkv, g, NULL, NULL};
            int64_t vis_end = causal ? i + 1 + delta : (int64_t)kv_len;
            attend_one(q, r * (int64_t)D, dt, &kv, 0, kv_len, vis_end, scale, NO_BIAS, s,
                       o_out + n * (int64_t)D, lse_out + n, NULL);
        }
        free(s);
    }
    return bad;
}

/*
 * The materialised softmax matrix P [q_len, kv_len] of one (b, h), with the
 * same masking as oracle_attn_fwd (zeros where masked; an all-zero row where
 * no key is visible).
 */
int oracle_softmax_matrix(const void* q, const void* k, int dt,
                          int B, int Hq, int Hkv, int q_len, int kv_len, int D,
                          double scale, int causal, int b, int h, double* p_out) {
    if (check_fwd_args(B, Hq, Hkv, q_len, kv_len, D)) return 1;
    if (b < 0 || b >= B || h < 0 || h >= Hq) return 1;
    const int g = h / (Hq / Hkv);
    const int64_t delta = (int64_t)kv_len - q_len;
    double* s = (double*)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
    double* o = (double*)malloc(sizeof(double) * (size_t)D);
    /* V is not needed for P; point it at K so the accumulation is harmless. */
    kv_view kv = {k, k, dt, D, ((int64_t)b * Hkv + g) * kv_len * (int64_t)D, NULL, 0, Hkv, g, NULL, NULL};
    for (int64_t i = 0; i < q_len; ++i) {
        double lse;
        int64_t vis_end = causal ? i + 1 + delta : (int64_t)kv_len;
        attend_one(q, (((int64_t)b * Hq + h) * q_len + i) * D, dt, &kv, 0, kv_len, vis_end,
                   scale, NO_BIAS, s, o, &lse, p_out + i * (int64_t)kv_len);
    }
    free(o);
    free(s);
    return 0;
}

/*
 * Decode (one query per sequence and head).  [P4] `_fwd_kernel_splitK` with
 * USE_SEQ_LEN: sequence b has seq_lens[b] keys, all visible.
 *
 * block_table != NULL: k/v are a paged pool [num_pages, page_size, Hkv, D],
 *   token t of sequence b lives in page block_table[b * max_pages + t / page_size].
 * block_table == NULL: k/v are dense [B, Hkv, max_kv_len, D].
 * rows are flat (b * Hq + h) ids (NULL = all).  o_out [n_rows, D], lse_out [n_rows].
 */
int oracle_attn_decode(const void* q, const void* k, const void* v, int dt,
                       const int* seq_lens, const int* block_table, int max_pages,
                       int page_size, int B, int Hq, int Hkv, int D, int max_kv_len,
                       double scale, const int64_t* rows, int64_t n_rows,
                       double* o_out, double* lse_out) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv || max_kv_len < 0) return 1;
    if (block_table && (page_size <= 0 || max_pages <= 0)) return 1;
    const int64_t total = (int64_t)B * Hq;
    if (!rows) n_rows = total;
    const int group = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(max_kv_len > 0 ? max_kv_len : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_rows; ++n) {
            int64_t r = rows ? rows[n] : n;
            if (r < 0 || r >= total) { bad = 1; continue; }
            int h = (int)(r % Hq);
            int b = (int)(r / Hq);
            int g = h / group;
            int64_t len = seq_lens[b];
            if (len < 0 || len > max_kv_len) { bad = 1; continue; }
            kv_view kv = {k, v, dt, D, ((int64_t)b * Hkv + g) * max_kv_len * (int64_t)D,
                          block_table ? block_table + (int64_t)b * max_pages : NULL,
                          page_size, Hkv, g, NULL, NULL};
            attend_one(q, r * (int64_t)D, dt, &kv, 0, len, len, scale, NO_BIAS, s,
                       o_out + n * (int64_t)D, lse_out + n, NULL);
        }
        free(s);
    }
    return bad;
}

/*
 * Decode with q_len queries per sequence.  [P4] `_fwd_kernel_splitK` with
 * IS_CAUSAL and NUM_QUERIES_CAUSAL: the queries of sequence b sit at its last
 * q_len positions, so query i has position seq_lens[b] - q_len + i and sees
 * the keys at or before it; a query before the first key sees none.
 *
 * q is [B, Hq, q_len, D]; rows are flat ((b * Hq + h) * q_len + i) ids (NULL
 * = all).  K/V addressing as in oracle_attn_decode.  o_out [n_rows, D],
 * lse_out [n_rows].
 */
int oracle_attn_decode_multi(const void* q, const void* k, const void* v, int dt,
                             const int* seq_lens, const int* block_table, int max_pages,
                             int page_size, int B, int Hq, int Hkv, int q_len, int D,
                             int max_kv_len, double scale, const int64_t* rows, int64_t n_rows,
                             double* o_out, double* lse_out) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv || max_kv_len < 0 || q_len <= 0) return 1;
    if (block_table && (page_size <= 0 || max_pages <= 0)) return 1;
    const int64_t total = (int64_t)B * Hq * q_len;
    if (!rows) n_rows = total;
    const int group = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(max_kv_len > 0 ? max_kv_len : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_rows; ++n) {
            int64_t r = rows ? rows[n] : n;
            if (r < 0 || r >= total) { bad = 1; continue; }
            int64_t i = r % q_len;
            int64_t bh = r / q_len;
            int h = (int)(bh % Hq);
            int b = (int)(bh / Hq);
            int g = h / group;
            int64_t len = seq_lens[b];
            if (len < 0 || len > max_kv_len) { bad = 1; continue; }
            kv_view kv = {k, v, dt, D, ((int64_t)b * Hkv + g) * max_kv_len * (int64_t)D,
                          block_table ? block_table + (int64_t)b * max_pages : NULL,
                          page_size, Hkv, g, NULL, NULL};
            /* position of query i: len - q_len + i; keys t <= that position */
            int64_t vis_end = len - q_len + i + 1;
            attend_one(q, r * (int64_t)D, dt, &kv, 0, len, vis_end, scale, NO_BIAS, s,
                       o_out + n * (int64_t)D, lse_out + n, NULL);
        }
        free(s);
    }
    return bad;
}

/*
 * Batched prefill of ragged requests over a paged KV cache.  [P2]
 * `_gqa_prefill_kernel` and its entry point: request b owns the query tokens
 * [qo_indptr[b], qo_indptr[b+1]) of the token-major q [total_q, Hq, D] and the
 * pages kv_indices[kv_indptr[b] .. kv_indptr[b+1]) of the pool
 * [num_pages, page_size, Hkv, D] (its key t is row t % page_size of page
 * kv_indices[kv_indptr[b] + t / page_size]).  With n_b pages, kv_len_b =
 * (n_b - 1) * page_size + kv_last_page_len[b], or n_b * page_size when
 * kv_last_page_len is NULL.  Query i of the request sees key t iff
 * !causal or t <= i + kv_len_b - q_len_b ([P2] bottom-right mask).
 *
 * rows are flat (token * Hq + h) ids (NULL = all total_q * Hq).
 * o_out [n_rows, D], lse_out [n_rows].  Returns 0, or 1 on a bad argument.
 */
int oracle_attn_prefill_paged(const void* q, const void* k, const void* v, int dt,
                              const int* qo_indptr, const int* kv_indptr, const int* kv_indices,
                              const int* kv_last_page_len, int B, int Hq, int Hkv, int D,
                              int page_size, double scale, int causal,
                              const int64_t* rows, int64_t n_rows,
                              double* o_out, double* lse_out) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv || page_size <= 0) return 1;
    const int64_t total_q = B > 0 ? qo_indptr[B] : 0;
    const int64_t total = total_q * Hq;
    if (!rows) n_rows = total;
    const int group = Hq / Hkv;
    int64_t max_kv = 1;
    for (int b = 0; b < B; ++b) {
        int64_t n = kv_indptr[b + 1] - kv_indptr[b];
        if (n < 0 || qo_indptr[b + 1] < qo_indptr[b]) return 1;
        if (n * page_size > max_kv) max_kv = n * page_size;
    }
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)max_kv);
#pragma omp for schedule(dynamic, 4)
        for (int64_t n = 0; n < n_rows; ++n) {
            int64_t r = rows ? rows[n] : n;
            if (r < 0 || r >= total) { bad = 1; continue; }
            int64_t tok = r / Hq;
            int h = (int)(r % Hq);
            int b = 0;
            while (b + 1 < B && qo_indptr[b + 1] <= tok) ++b;  /* request holding the token */
            int64_t i = tok - qo_indptr[b];
            int64_t q_len = qo_indptr[b + 1] - qo_indptr[b];
            int64_t n_pages = kv_indptr[b + 1] - kv_indptr[b];
            int64_t kv_len = 0;
            if (n_pages > 0)
                kv_len = (n_pages - 1) * page_size + (kv_last_page_len ? kv_last_page_len[b] : page_size);
            int g = h / group;
            kv_view kv = {k, v, dt, D, 0, kv_indices + kv_indptr[b], page_size, Hkv, g, NULL, NULL};
            int64_t vis_end = causal ? i + 1 + (kv_len - q_len) : kv_len;
            attend_one(q, r * (int64_t)D, dt, &kv, 0, kv_len, vis_end, scale, NO_BIAS, s,
                       o_out + n * (int64_t)D, lse_out + n, NULL);
        }
        free(s);
    }
    return bad;
}

/*
 * Decode over an fp8 KV cache.  [P4] `_fwd_kernel_splitK` with FP8_QUANTIZED:
 * K and V hold one 8-bit float per element (E4M3) and every (token, K/V head)
 * row has a binary16 scale and shift, so the key or value used is
 * stored * scale + shift (`dequantize`); attention is then the plain decode
 * of oracle_attn_decode over those values, in double.  q (and the output) are
 * in q_dt.  k_ss / v_ss are laid out like the cache without its last
 * dimension: [num_pages, page_size, Hkv] (paged) or [B, Hkv, max_kv_len]
 * (dense).
 */
int oracle_attn_decode_fp8(const void* q, int q_dt, const void* k, const void* v,
                           const uint32_t* k_ss, const uint32_t* v_ss,
                           const int* seq_lens, const int* block_table, int max_pages,
                           int page_size, int B, int Hq, int Hkv, int D, int max_kv_len,
                           double scale, const int64_t* rows, int64_t n_rows,
                           double* o_out, double* lse_out) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv || max_kv_len < 0) return 1;
    if (!k_ss || !v_ss) return 1;
    if (block_table && (page_size <= 0 || max_pages <= 0)) return 1;
    const int64_t total = (int64_t)B * Hq;
    if (!rows) n_rows = total;
    const int group = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(max_kv_len > 0 ? max_kv_len : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_rows; ++n) {
            int64_t r = rows ? rows[n] : n;
            if (r < 0 || r >= total) { bad = 1; continue; }
            int h = (int)(r % Hq);
            int b = (int)(r / Hq);
            int g = h / group;
            int64_t len = seq_lens[b];
            if (len < 0 || len > max_kv_len) { bad = 1; continue; }
            kv_view kv = {k, v, ORACLE_FP8E4M3, D, ((int64_t)b * Hkv + g) * max_kv_len * (int64_t)D,
                          block_table ? block_table + (int64_t)b * max_pages : NULL,
                          page_size, Hkv, g, k_ss, v_ss};
            attend_one(q, r * (int64_t)D, q_dt, &kv, 0, len, len, scale, NO_BIAS, s,
                       o_out + n * (int64_t)D, lse_out + n, NULL);
        }
        free(s);
    }
    return bad;
}

/*
 * Split-K decode by the split/merge route, for the invariant tests.
 * bounds is [B, n_splits + 1]: chunk s of sequence b covers tokens
 * [bounds[b][s], bounds[b][s+1]) clipped to seq_lens[b].  Each chunk's
 * (O_s, L_s) is the plain definition restricted to that chunk ([P4]
 * `_fwd_kernel_splitK`: an empty chunk gives (0, -inf)); the chunks are then
 * merged as in [P4] `_splitK_reduce`.
 * o_parts [n_rows, n_splits, D] and lse_parts [n_rows, n_splits] may be NULL.
 */
int oracle_decode_split_merge(const void* q, const void* k, const void* v, int dt,
                              const int* seq_lens, const int* block_table, int max_pages,
                              int page_size, int B, int Hq, int Hkv, int D, int max_kv_len,
                              double scale, const int* bounds, int n_splits,
                              const int64_t* rows, int64_t n_rows,
                              double* o_out, double* lse_out,
                              double* o_parts, double* lse_parts) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv || n_splits < 1) return 1;
    if (block_table && (page_size <= 0 || max_pages <= 0)) return 1;
    const int64_t total = (int64_t)B * Hq;
    if (!rows) n_rows = total;
    const int group = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(max_kv_len > 0 ? max_kv_len : 1));
        double* os = (double*)malloc(sizeof(double) * (size_t)n_splits * D);
        double* ls = (double*)malloc(sizeof(double) * (size_t)n_splits);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_rows; ++n) {
            int64_t r = rows ? rows[n] : n;
            if (r < 0 || r >= total) { bad = 1; continue; }
            int h = (int)(r % Hq);
            int b = (int)(r / Hq);
            int g = h / group;
            int64_t len = seq_lens[b];
            if (len < 0 || len > max_kv_len) { bad = 1; continue; }
            kv_view kv = {k, v, dt, D, ((int64_t)b * Hkv + g) * max_kv_len * (int64_t)D,
                          block_table ? block_table + (int64_t)b * max_pages : NULL,
                          page_size, Hkv, g, NULL, NULL};
            const int* bb = bounds + (int64_t)b * (n_splits + 1);
            for (int sp = 0; sp < n_splits; ++sp) {
                int64_t lo = bb[sp], hi = bb[sp + 1];
                if (lo < 0) lo = 0;
                if (hi > len) hi = len;
                if (hi < lo) hi = lo;
                attend_one(q, r * (int64_t)D, dt, &kv, lo, hi, len, scale, NO_BIAS, s,
                           os + (int64_t)sp * D, ls + sp, NULL);
            }
            /* merge */
            double M = -INFINITY;
            for (int sp = 0; sp < n_splits; ++sp)
                if (ls[sp] > M) M = ls[sp];
            double* o = o_out + n * (int64_t)D;
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            if (M == -INFINITY) {
                lse_out[n] = -INFINITY;
            } else {
                double wsum = 0.0;
                for (int sp = 0; sp < n_splits; ++sp) {
                    double w = exp(ls[sp] - M);
                    wsum += w;
                    for (int d = 0; d < D; ++d) o[d] += w * os[(int64_t)sp * D + d];
                }
                for (int d = 0; d < D; ++d) o[d] /= wsum;
                lse_out[n] = M + log(wsum);
            }
            if (o_parts) memcpy(o_parts + n * (int64_t)n_splits * D, os, sizeof(double) * (size_t)n_splits * D);
            if (lse_parts) memcpy(lse_parts + n * (int64_t)n_splits, ls, sizeof(double) * (size_t)n_splits);
        }
        free(ls);
        free(os);
        free(s);
    }
    return bad;
}

/*
 * Forward with an additive attention bias.  [P4] `_fwd_kernel_splitK` with
 * HAS_ADDITIVE_BIAS: the bias of (b, h, i, j) is added to the scaled score,
 * s_ij = scale * q_i . k_j + bias(b, h, i, j), before the softmax (the kernel
 * adds it in its base-2 units, i.e. multiplied by log2 e, which is the same
 * softmax); the causal rule of oracle_attn_fwd still applies on top.
 * bias(b, h, i, j) = bias[b * sb + h * sh + i * sq + j] in storage format
 * bias_dt (strides in elements; a stride of 0 broadcasts).  A row whose
 * visible scores are all -inf gives (0, -inf).  Layouts and rows as for
 * oracle_attn_fwd.
 */
int oracle_attn_fwd_bias(const void* q, const void* k, const void* v, int dt,
                         const void* bias, int bias_dt, int64_t sb, int64_t sh, int64_t sq,
                         int B, int Hq, int Hkv, int q_len, int kv_len, int D,
                         double scale, int causal,
                         const int64_t* rows, int64_t n_rows,
                         double* o_out, double* lse_out) {
    if (check_fwd_args(B, Hq, Hkv, q_len, kv_len, D) || !bias) return 1;
    const int64_t total = (int64_t)B * Hq * q_len;
    if (!rows) n_rows = total;
    const int group = Hq / Hkv;
    const int64_t delta = (int64_t)kv_len - q_len;
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t n = 0; n < n_rows; ++n) {
            int64_t r = rows ? rows[n] : n;
            if (r < 0 || r >= total) { bad = 1; continue; }
            int64_t i = r % q_len;
            int64_t bh = r / q_len;
            int h = (int)(bh % Hq);
            int b = (int)(bh / Hq);
            const int g = h / group;  /* K/V head of query head h */
            const int64_t kv_base = ((int64_t)b * Hkv + g) * kv_len * (int64_t)D;
            kv_view kv = {k, v, dt, D, kv_base, NULL, 0, Hkv, g, NULL, NULL};
            bias_view bv = {bias, bias_dt, b * sb + h * sh + i * sq};
            int64_t vis_end = causal ? (i + 1) + delta : (int64_t)kv_len;
            attend_one(q, r * (int64_t)D, dt, &kv, 0, kv_len, vis_end, scale, bv, s,
                       o_out + n * (int64_t)D, lse_out + n, NULL);
        }
        free(s);
    }
    return bad;
}

/*
 * Decode (q_len >= 1 queries per sequence, placed and masked as in
 * oracle_attn_decode_multi) with an additive bias: [P4] `_fwd_kernel_splitK`
 * with HAS_ADDITIVE_BIAS.  Query i of sequence b, head h, key t gets
 * bias[b * sb + h * sh + i * sq + t] (storage format bias_dt) added to its
 * scaled score.  K/V addressing, rows and outputs as for
 * oracle_attn_decode_multi.
 */
int oracle_attn_decode_bias(const void* q, const void* k, const void* v, int dt,
                            const int* seq_lens, const int* block_table, int max_pages,
                            int page_size, int B, int Hq, int Hkv, int q_len, int D,
                            int max_kv_len, double scale,
                            const void* bias, int bias_dt, int64_t sb, int64_t sh, int64_t sq,
                            const int64_t* rows, int64_t n_rows,
                            double* o_out, double* lse_out) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv || max_kv_len < 0 || q_len <= 0) return 1;
    if (block_table && (page_size <= 0 || max_pages <= 0)) return 1;
    if (!bias) return 1;
    const int64_t total = (int64_t)B * Hq * q_len;
    if (!rows) n_rows = total;
    const int group = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(max_kv_len > 0 ? max_kv_len : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_rows; ++n) {
            int64_t r = rows ? rows[n] : n;
            if (r < 0 || r >= total) { bad = 1; continue; }
            int64_t i = r % q_len;
            int64_t bh = r / q_len;
            int h = (int)(bh % Hq);
            int b = (int)(bh / Hq);
            int g = h / group;
            int64_t len = seq_lens[b];
            if (len < 0 || len > max_kv_len) { bad = 1; continue; }
            kv_view kv = {k, v, dt, D, ((int64_t)b * Hkv + g) * max_kv_len * (int64_t)D,
                          block_table ? block_table + (int64_t)b * max_pages : NULL,
                          page_size, Hkv, g, NULL, NULL};
            bias_view bv = {bias, bias_dt, (int64_t)b * sb + (int64_t)h * sh + i * sq};
            int64_t vis_end = (len - q_len) + i + 1;  /* query i at position len - q_len + i */
            attend_one(q, r * (int64_t)D, dt, &kv, 0, len, vis_end, scale, bv, s,
                       o_out + n * (int64_t)D, lse_out + n, NULL);
        }
        free(s);
    }
    return bad;
}

/*
 * Merge of n_splits partial results per row, [P4] `_splitK_reduce`:
 * M = max_s L_s, w_s = exp(L_s - M), O = sum_s w_s O_s / sum_s w_s,
 * L = M + log(sum_s w_s); (0, -inf) when every L_s is -inf.
 * o_parts [n_rows, n_splits, D], lse_parts [n_rows, n_splits];
 * o_out [n_rows, D], lse_out [n_rows].
 */
int oracle_splitk_merge(const double* o_parts, const double* lse_parts, int64_t n_rows, int n_splits, int D,
                        double* o_out, double* lse_out) {
    if (n_rows < 0 || n_splits < 1 || D <= 0) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_rows; ++n) {
        const double* ls = lse_parts + n * n_splits;
        const double* os = o_parts + n * (int64_t)n_splits * D;
        double* o = o_out + n * (int64_t)D;
        double M = -INFINITY;
        for (int sp = 0; sp < n_splits; ++sp)
            if (ls[sp] > M) M = ls[sp];
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (M == -INFINITY) {
            lse_out[n] = M;
            continue;
        }
        double wtot = 0.0;
        for (int sp = 0; sp < n_splits; ++sp) {
            double wt = exp(ls[sp] - M);
            wtot += wt;
            for (int d = 0; d < D; ++d) o[d] += wt * os[(int64_t)sp * D + d];
        }
        for (int d = 0; d < D; ++d) o[d] /= wtot;
        lse_out[n] = log(wtot) + M;
    }
    return 0;
}

/*
 * Gradients of that merge, [P4] `_splitK_reduce_varargs_backward`.  With the
 * merged (O, L) of the partials (O_s, L_s) and the incoming gradients dO, dL:
 * the weight of partial s in O is w_s = exp(L_s - L) (the weights sum to 1),
 * O = sum_s w_s O_s and L = log sum_s exp(L_s), so
 *   dO/dO_s = w_s,  dL/dO_s = 0,  dO/dL_s = w_s (O_s - O),  dL/dL_s = w_s,
 * and by the chain rule
 *   dO_s = w_s dO,
 *   dL_s = w_s (dL + sum_d (O_s - O)_d dO_d).
 * A partial with L_s = -inf (an empty chunk), and every partial of a row
 * with L = -inf, gets zero gradients.
 * o_parts / d_o_parts [n_rows, n_splits, D], lse_parts / d_lse_parts
 * [n_rows, n_splits], o / d_o [n_rows, D], lse / d_lse [n_rows].
 */
int oracle_splitk_merge_backward(const double* o_parts, const double* lse_parts, const double* o,
                                 const double* lse, const double* d_o, const double* d_lse,
                                 int64_t n_rows, int n_splits, int D,
                                 double* d_o_parts, double* d_lse_parts) {
    if (n_rows < 0 || n_splits < 1 || D <= 0) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_rows; ++n) {
        const double* orow = o + n * (int64_t)D;
        const double* dorow = d_o + n * (int64_t)D;
        for (int sp = 0; sp < n_splits; ++sp) {
            const int64_t ps = n * n_splits + sp;
            const double* os = o_parts + ps * D;
            double* dos = d_o_parts + ps * D;
            const double ls = lse_parts[ps];
            const double w = (ls == -INFINITY || lse[n] == -INFINITY) ? 0.0 : exp(ls - lse[n]);
            double dot = 0.0;
            for (int d = 0; d < D; ++d) {
                dos[d] = w * dorow[d];
                dot += (os[d] - orow[d]) * dorow[d];
            }
            d_lse_parts[ps] = w == 0.0 ? 0.0 : w * (d_lse[n] + dot);
        }
    }
    return 0;
}
