/*
 * kvdec_oracle.c -- slow, plain, obviously correct CPU reference for the
 * single-token KV-cached decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: it is used by the tests, by the smoke check and by the
 * CPU-baseline leg of the benchmark, nowhere else.  It shares no source,
 * header, table or helper with the HIP library; the two only ever see the
 * same seeded input arrays.
 *
 * Arithmetic: every product and sum is carried in double (IEEE binary64),
 * in a fixed ascending order, with the C library's exp().  No SIMD
 * intrinsics, no -ffast-math, no blocking, no reordering.
 *
 * Sources (docs.rs source pages; cited by page and item):
 *   [WA-DEC]  whisper-apr 0.3.3, src/model/decoder_generated.rs
 *   [WA-CUDA] whisper-apr 0.3.0, src/cuda/impl_generated.rs
 *   [FO-Q2]   franken_ocr 0.8.0, src/native_engine/decoder_qwen2.rs
 *   [CERA]    cera 0.5.4, src/model/whisper.rs
 *   [LAT-Q8]  lattice-inference 0.4.0, src/forward/cpu_q8.rs
 *
 * Parity pins: every function here is pinned by tests/test_oracle.py
 * (closed forms, invariants, brute-force re-prefill, a library routine and
 * a worked example printed on [FO-Q2]).  No function is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_E_SHAPE 2
#define ORACLE_E_NOMEM 7

/* Element decode.  dtype 0: IEEE binary32.  dtype 1: bfloat16, i.e. the
 * upper 16 bits of a binary32; widening is exact (append 16 zero bits). */
static double load_elem(const void* base, int dtype, int64_t idx)
{
    if (dtype == 0) {
        return (double)((const float*)base)[idx];
    }
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * One query row against n cached key/value rows (one head).
 *
 * Follows the per-head decode of [FO-Q2] `decode_attn_head` and the
 * per-query-head loop of [LAT-Q8] `full_attention_step_q8`:
 *   s_j  = scale * (q . k_j)                 for j = 0 .. n-1
 *   m    = max_j s_j                          (stable softmax shift)
 *   e_j  = exp(s_j - m),  Z = sum_j e_j
 *   out  = (sum_j e_j v_j) / Z
 * Fail-closed rule of [LAT-Q8] `full_attention_step_q8` (softmax block):
 * when Z is not > 0 (this includes NaN) the output row is all zeros.  An
 * empty key set (n == 0) also gives zeros (the zero-filled context of the
 * same function when no position is attended).
 *
 * k_row(j) / v_row(j) address row j; rows are D elements apart inside a row
 * block and `row_stride` elements apart between rows.
 */
static int attend_one(const float* q, const void* K, const void* V, int dtype,
                      int64_t n, int64_t D, int64_t row_stride, double scale,
                      double* out)
{
    for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
    if (n <= 0) return ORACLE_OK;

    double* s = (double*)malloc((size_t)n * sizeof(double));
    if (!s) return ORACLE_E_NOMEM;

    for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d)
            dot += (double)q[d] * load_elem(K, dtype, j * row_stride + d);
        s[j] = scale * dot;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j)
        if (s[j] > m) m = s[j];

    double Z = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        Z += s[j];
    }
    if (!(Z > 0.0)) {           /* fail closed: zeros */
        free(s);
        return ORACLE_OK;
    }
    for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t j = 0; j < n; ++j)
            acc += s[j] * load_elem(V, dtype, j * row_stride + d);
        out[d] = acc / Z;
    }
    free(s);
    return ORACLE_OK;
}

/*
 * Batched decode attention over a head-major padded cache.
 *
 *   q    : float  [B][Hq][D]
 *   K, V : dtype  [B][Hkv][cap][D]   (cap = padded rows per (b, kv head))
 *   lens : int32  [B]                rows attended for sequence b (<= cap)
 *   out  : double [B][Hq][D]
 *
 * Query head h reads KV head h / (Hq / Hkv): the contiguous grouping of
 * [FO-Q2] `decode_attn_head` (kv lane h / kv_group) and of [LAT-Q8]
 * `full_attention_step_q8` (kvh = qh / groups).  Hq must be a positive
 * multiple of Hkv ([FO-Q2] DecoderConfig GQA validation), else ORACLE_E_SHAPE.
 *
 * Causality is implicit: the caller passes lens that already include the
 * row appended for the current token, and every cached row is attended with
 * no mask ([FO-Q2] `qwen2_decode_attention` doc; [CERA] `decode_step_into`
 * attends k[..pos+1]).
 */
int kvdec_oracle_attend(const float* q, const void* K, const void* V, int dtype,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t cap,
                        const int32_t* lens, double scale, double* out)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || cap < 0) return ORACLE_E_SHAPE;
    if (Hq % Hkv != 0) return ORACLE_E_SHAPE;
    if (dtype != 0 && dtype != 1) return ORACLE_E_SHAPE;
    const int64_t group = Hq / Hkv;
    const size_t esz = dtype == 0 ? 4 : 2;
    for (int64_t b = 0; b < B; ++b) {
        int64_t n = lens[b];
        if (n < 0 || n > cap) return ORACLE_E_SHAPE;
        for (int64_t h = 0; h < Hq; ++h) {
            int64_t g = h / group;
            int64_t off = ((b * Hkv + g) * cap) * D;
            const char* kb = (const char*)K + (size_t)off * esz;
            const char* vb = (const char*)V + (size_t)off * esz;
            int rc = attend_one(q + (b * Hq + h) * D, kb, vb, dtype, n, D, D, scale,
                                out + (b * Hq + h) * D);
            if (rc) return rc;
        }
    }
    return ORACLE_OK;
}

/*
 * Full-causal prefill attention with an explicit additive mask -- the
 * O(n^2) re-prefill route that [FO-Q2] keeps as its parity oracle for the
 * KV-cache decode (`generate_greedy` re-runs the whole prefill each step;
 * `prefill_attention_gqa` / `broadcast_kv` give the GQA head sharing) and
 * that [WA-DEC] builds with its causal mask (0 on and below the diagonal,
 * -inf above).
 *
 *   Q   : double [n][Hq][D]   token-major, one row per position
 *   K,V : double [n][Hkv][D]
 *   out : double [n][Hq][D]
 *
 * This route deliberately shares nothing with kvdec_oracle_attend: it
 * broadcasts K/V to the full query-head width first, materialises the n x n
 * mask, and normalises each row with its own max over all n columns.
 */
int kvdec_oracle_prefill_causal(const double* Q, const double* K, const double* V,
                                int64_t n, int64_t Hq, int64_t Hkv, int64_t D,
                                double scale, double* out)
{
    if (n < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return ORACLE_E_SHAPE;
    if (n == 0) return ORACLE_OK;
    const int64_t group = Hq / Hkv;

    /* broadcast-to-MHA copy of K and V: [n][Hq][D] */
    double* Kf = (double*)malloc((size_t)(n * Hq * D) * sizeof(double));
    double* Vf = (double*)malloc((size_t)(n * Hq * D) * sizeof(double));
    double* mask = (double*)malloc((size_t)(n * n) * sizeof(double));
    double* row = (double*)malloc((size_t)n * sizeof(double));
    if (!Kf || !Vf || !mask || !row) {
        free(Kf); free(Vf); free(mask); free(row);
        return ORACLE_E_NOMEM;
    }
    for (int64_t r = 0; r < n; ++r)
        for (int64_t g = 0; g < Hkv; ++g)
            for (int64_t rep = 0; rep < group; ++rep) {
                int64_t h = g * group + rep;
                memcpy(Kf + (r * Hq + h) * D, K + (r * Hkv + g) * D, (size_t)D * sizeof(double));
                memcpy(Vf + (r * Hq + h) * D, V + (r * Hkv + g) * D, (size_t)D * sizeof(double));
            }
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < n; ++j)
            mask[i * n + j] = (j <= i) ? 0.0 : -INFINITY;

    for (int64_t i = 0; i < n; ++i) {
        for (int64_t h = 0; h < Hq; ++h) {
            const double* qi = Q + (i * Hq + h) * D;
            for (int64_t j = 0; j < n; ++j) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += qi[d] * Kf[(j * Hq + h) * D + d];
                row[j] = scale * dot + mask[i * n + j];
            }
            double m = -INFINITY;
            for (int64_t j = 0; j < n; ++j)
                if (row[j] > m) m = row[j];
            double Z = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                row[j] = exp(row[j] - m);   /* masked columns: exp(-inf) = 0 */
                Z += row[j];
            }
            double* o = out + (i * Hq + h) * D;
            for (int64_t d = 0; d < D; ++d) {
                if (!(Z > 0.0)) { o[d] = 0.0; continue; }
                double acc = 0.0;
                for (int64_t j = 0; j < n; ++j) acc += row[j] * Vf[(j * Hq + h) * D + d];
                o[d] = acc / Z;
            }
        }
    }
    free(Kf); free(Vf); free(mask); free(row);
    return ORACLE_OK;
}

/*
 * Append one new K row and one new V row per (sequence, KV head) at slot
 * lens[b], then lens[b] += 1: the copy-then-grow of [WA-DEC]
 * `LayerKVCache::append`, [FO-Q2] `Qwen2KvCache::append`, and the scatter to
 * row `pos` of every head of the head-first GPU cache in [WA-CUDA]
 * `forward_decoder_block_gpu` (`kv_cache_scatter_gpu`).
 *
 *   cacheK, cacheV : elem [B][Hkv][cap][D]   (bytes, esz per element)
 *   k_new, v_new   : elem [B][Hkv][D]
 *
 * Overflow is rejected before anything is written, as in
 * `LayerKVCache::append` ("cache overflow" check ahead of the copy).
 */
int kvdec_oracle_append(void* cacheK, void* cacheV, const void* k_new, const void* v_new,
                        int64_t esz, int64_t B, int64_t Hkv, int64_t D, int64_t cap,
                        int32_t* lens)
{
    if (esz <= 0 || B < 0 || Hkv <= 0 || D <= 0 || cap < 0) return ORACLE_E_SHAPE;
    for (int64_t b = 0; b < B; ++b)
        if (lens[b] < 0 || (int64_t)lens[b] + 1 > cap) return 3; /* overflow */
    const size_t row = (size_t)(D * esz);
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t g = 0; g < Hkv; ++g) {
            size_t dst = (size_t)(((b * Hkv + g) * cap + lens[b]) * D * esz);
            size_t src = (size_t)((b * Hkv + g) * D * esz);
            memcpy((char*)cacheK + dst, (const char*)k_new + src, row);
            memcpy((char*)cacheV + dst, (const char*)v_new + src, row);
        }
        lens[b] += 1;
    }
    return ORACLE_OK;
}

/*
 * Append with a sliding window that keeps an overlap, the streaming cache of
 * [WA-DEC] `StreamingKVCache` (`append_with_slide`, `slide_window`): when the
 * new row would take a sequence past `window` rows, the sequence first keeps
 * only its last `overlap` rows (rows len - overlap .. len - 1 become rows
 * 0 .. overlap - 1; the overlap is at most half the window, as the page's
 * constructor caps it) and its length becomes `overlap`; then the row is
 * appended as kvdec_oracle_append does.  `window` <= cap; slid[b] (may be
 * NULL) is set to 1 where sequence b slid, else 0.
 */
int kvdec_oracle_append_slide(void* cacheK, void* cacheV, const void* k_new, const void* v_new,
                              int64_t esz, int64_t B, int64_t Hkv, int64_t D, int64_t cap,
                              int64_t window, int64_t overlap, int32_t* lens, int32_t* slid)
{
    if (esz <= 0 || B < 0 || Hkv <= 0 || D <= 0 || window < 1 || window > cap || overlap < 0)
        return ORACLE_E_SHAPE;
    const int64_t keep = overlap < window / 2 ? overlap : window / 2;
    for (int64_t b = 0; b < B; ++b)
        if (lens[b] < 0 || lens[b] > window) return ORACLE_E_SHAPE;
    const size_t row = (size_t)(D * esz);
    for (int64_t b = 0; b < B; ++b) {
        int slide = (int64_t)lens[b] + 1 > window;
        if (slide) {
            const int64_t keep_from = lens[b] - keep;
            for (int64_t g = 0; g < Hkv; ++g) {
                char* k = (char*)cacheK + (size_t)((b * Hkv + g) * cap * D * esz);
                char* v = (char*)cacheV + (size_t)((b * Hkv + g) * cap * D * esz);
                memmove(k, k + (size_t)keep_from * row, (size_t)keep * row);
                memmove(v, v + (size_t)keep_from * row, (size_t)keep * row);
            }
            lens[b] = (int32_t)keep;
        }
        if (slid) slid[b] = slide;
        for (int64_t g = 0; g < Hkv; ++g) {
            size_t dst = (size_t)(((b * Hkv + g) * cap + lens[b]) * D * esz);
            size_t src = (size_t)((b * Hkv + g) * D * esz);
            memcpy((char*)cacheK + dst, (const char*)k_new + src, row);
            memcpy((char*)cacheV + dst, (const char*)v_new + src, row);
        }
        lens[b] += 1;
    }
    return ORACLE_OK;
}

/*
 * Token-major -> head-major import: the interleaved-to-head-first permute of
 * [WA-CUDA] `populate_cross_kv_caches_gpu` (`interleaved_to_head_first`),
 * [L, H*D] -> [H, L, D] per sequence, written into the padded cache.
 *
 *   src : elem [B][rows][Hkv*D]
 *   dst : elem [B][Hkv][cap][D]   rows >= `rows` are left untouched
 */
int kvdec_oracle_seed(void* dst, const void* src, int64_t esz, int64_t B, int64_t rows,
                      int64_t Hkv, int64_t D, int64_t cap)
{
    if (esz <= 0 || B < 0 || rows < 0 || Hkv <= 0 || D <= 0 || rows > cap) return ORACLE_E_SHAPE;
    const size_t row = (size_t)(D * esz);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < rows; ++t)
            for (int64_t g = 0; g < Hkv; ++g) {
                size_t s = (size_t)(((b * rows + t) * Hkv + g) * D * esz);
                size_t d = (size_t)(((b * Hkv + g) * cap + t) * D * esz);
                memcpy((char*)dst + d, (const char*)src + s, row);
            }
    return ORACLE_OK;
}

/*
 * Rotary position embedding, NEOX rotate-half form, on rows of D values:
 * dims (i, i + D/2) form a pair rotated by the angle pos * theta^(-2i/D):
 *   x_i'       = x_i cos(a) - x_{i+D/2} sin(a)
 *   x_{i+D/2}' = x_i sin(a) + x_{i+D/2} cos(a)
 * Stride-half pairing as in [LAT-Q8] `full_attention_step_q8` (pairs
 * (i, half + i)), frequencies theta^(-2i/D) with theta = 1e6 for Qwen2 as
 * named in [FO-Q2] (NEOX rotate-half, applied to q and k before the key is
 * cached).  Everything in double.
 *
 *   x   : double [n][D]   (D even)
 *   pos : int32  [n]      position of each row
 *   out : double [n][D]   (may alias x)
 */
int kvdec_oracle_rope(const double* x, int64_t n, int64_t D, const int32_t* pos, double theta,
                      double* out)
{
    if (n < 0 || D <= 0 || D % 2 != 0 || !(theta > 0.0)) return ORACLE_E_SHAPE;
    const int64_t half = D / 2;
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t i = 0; i < half; ++i) {
            const double inv_freq = pow(theta, -2.0 * (double)i / (double)D);
            const double a = (double)pos[r] * inv_freq;
            const double c = cos(a), s = sin(a);
            const double x0 = x[r * D + i], x1 = x[r * D + half + i];
            out[r * D + i] = x0 * c - x1 * s;
            out[r * D + half + i] = x0 * s + x1 * c;
        }
    }
    return ORACLE_OK;
}
