/*
 * CPU oracle for the gated sparse attention hot path (indexer -> Top-K ->
 * exact sparse attention -> sigmoid output gate).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header, table or constant with the HIP library.
 *
 * Plain, slow, obviously correct: every input is decoded exactly to double,
 * every sum runs in double in the order the definition states, and the only
 * parallelism is over independent output rows (OpenMP), which does not change
 * any row's arithmetic.
 *
 * Pages cited (by title):
 *   [HAT] "Hybrid Attention Architectures: Engineering Trade-offs from Linear
 *          Attention to Gated Sparse Attention"
 *   [F2S] "From Full Attention to Sparsity: The Evolution of Hybrid Attention
 *          Architectures in Large Language Models"
 *   [SAD] "Sparse Attention and Hybrid Attention Architecture Design in Large
 *          Language Models"
 *   [SEL] "Hybrid Attention Architecture Evolution in LLMs: From Full
 *          Attention to Sparse Selection"
 *
 * Readings taken where the pages leave a step open (each is also pinned, or
 * marked "parity unpinned", by the oracle tests):
 *   - indexer score  I[i,s] = sum_h w[i,h] * max(0, q^I[i,h,:] . k^I[s,:]),
 *     one k^I row per position shared by all indexer heads; fp8 dots are
 *     multiplied by q_scale[i] * k_scale[s] after the dot (parity unpinned as
 *     a choice of form: the pages name a lightweight multi-head scorer but
 *     print no formula);
 *   - causal candidates of query token i are positions s <= pos(i);
 *   - Top-K orders by (score descending, position ascending);
 *   - rows with n <= K take all n positions, the rest of the row is -1;
 *   - output gate  y = o * sigmoid(G), G per channel or per head;
 *   - cache append: fp8 indexer keys as e4m3fn codes with a per-token scale
 *     max|x| / 448, nearest-even, saturating (see that section);
 *   - block-level selection: blocks are pages, pooled keys are block means,
 *     block scores sum the query heads' dots (see that section);
 *   - branch fusion: the local branch is causal attention over the last w
 *     positions, fused as g * sparse + (1 - g) * local (see that section);
 *   - backward: gradients of the attention and the gate over fixed indices,
 *     scatter-added into the cache rows (see that section).
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2 };

/* Ragged batch over a paged cache.  Query token j of sequence b sits at
 * position pos = ctx_len[b] - (q_start[b+1] - q_start[b]) + j, and its causal
 * candidates are the n = pos + 1 positions 0..pos.  Logical position s of
 * sequence b lives at physical cache row
 *     page_table[b*max_pages + s/page_size] * page_size + s % page_size. */
typedef struct {
    int32_t num_seqs;
    int32_t page_size;
    int32_t max_pages;
    int32_t pad_;
    const int32_t *q_start;
    const int32_t *ctx_len;
    const int32_t *page_table;
} orc_batch;

/* ---------------------------------------------------------------- decoding */

/* OCP fp8 e4m3fn: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN; there is
 * no infinity.  Built from that definition, not from any library table. */
double orc_fp8_e4m3fn(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

void orc_fp8_table(double *out256)
{
    for (int i = 0; i < 256; ++i)
        out256[i] = orc_fp8_e4m3fn((uint8_t)i);
}

/* bf16 is the top half of an IEEE binary32. */
double orc_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double load(int dtype, const void *base, int64_t i)
{
    switch (dtype) {
    case ORC_F32: return (double)((const float *)base)[i];
    case ORC_BF16: return orc_bf16(((const uint16_t *)base)[i]);
    default: return orc_fp8_e4m3fn(((const uint8_t *)base)[i]);
    }
}

/* ---------------------------------------------------------------- geometry */

static int seq_of(const orc_batch *bt, int64_t tok)
{
    for (int b = 0; b < bt->num_seqs; ++b)
        if (tok >= bt->q_start[b] && tok < bt->q_start[b + 1])
            return b;
    return -1;
}

static int64_t pos_of(const orc_batch *bt, int64_t tok, int *b_out)
{
    int b = seq_of(bt, tok);
    *b_out = b;
    int64_t nq = bt->q_start[b + 1] - bt->q_start[b];
    return (int64_t)bt->ctx_len[b] - nq + (tok - bt->q_start[b]);
}

static int64_t phys_row(const orc_batch *bt, int b, int64_t s)
{
    int64_t page = bt->page_table[(int64_t)b * bt->max_pages + s / bt->page_size];
    return page * bt->page_size + s % bt->page_size;
}

int orc_set_threads(int threads)
{
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
    return omp_get_max_threads();
#else
    (void)threads;
    return 1;
#endif
}

/* Number of causal candidates n = pos + 1 of each listed query token. */
void orc_row_lengths(const orc_batch *bt, const int64_t *rows, int64_t nrows, int64_t *n_out)
{
    for (int64_t r = 0; r < nrows; ++r) {
        int b;
        n_out[r] = pos_of(bt, rows[r], &b) + 1;
    }
}

/* ------------------------------------------------------- a1: indexer scores
 * [HAT §3.1 and §3.3]: a lightweight relevance score of the query against
 * every historical position, computed before selection.
 * [F2S "Fine-Grained Sparse Attention: Indexer Plus Top-K"]: a small scorer
 * with few heads and low dims, scoring content only (no positional encoding
 * enters here), producing one score per (query, history position) pair.
 * Form (the reading above): I[i,s] = sum_h w[i,h] * max(0, sum_d q[i,h,d] k[s,d])
 * with fp8 dots scaled by q_scale[i] * k_scale[s].
 * Row r of `scores` (stride ld) receives token rows[r]; entries [0, n) are
 * written, the rest of the row is left untouched. */
void orc_indexer(const orc_batch *bt, int dtype, const void *q_idx, int H, int D,
                 const float *q_scale, const float *w, const void *k_idx, const float *k_scale,
                 const int64_t *rows, int64_t nrows, double *scores, int64_t ld)
{
#pragma omp parallel
    {
        double *qd = (double *)malloc(sizeof(double) * (size_t)H * D);
        double *kd = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t i = rows[r];
            int b;
            int64_t pos = pos_of(bt, i, &b);
            for (int64_t e = 0; e < (int64_t)H * D; ++e)
                qd[e] = load(dtype, q_idx, i * (int64_t)H * D + e);
            double qs = (dtype == ORC_FP8) ? (double)q_scale[i] : 1.0;
            for (int64_t s = 0; s <= pos; ++s) {
                int64_t pr = phys_row(bt, b, s);
                for (int d = 0; d < D; ++d)
                    kd[d] = load(dtype, k_idx, pr * D + d);
                double ks = (dtype == ORC_FP8) ? (double)k_scale[pr] : 1.0;
                double acc = 0.0;
                for (int h = 0; h < H; ++h) {
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += qd[h * D + d] * kd[d];
                    dot = dot * qs * ks;
                    acc += (double)w[i * H + h] * (dot > 0.0 ? dot : 0.0);
                }
                scores[r * ld + s] = acc;
            }
        }
        free(kd);
        free(qd);
    }
}

/* ------------------------------------------------------------- a2: Top-K
 * [HAT §3.1]: keep the K highest-scoring positions as the candidate set.
 * [F2S "Fine-Grained Sparse Attention: Indexer Plus Top-K"]: per query, the
 * index tensor has shape [n, K].
 * [HAT §5 item 4]: when a row has fewer candidates than K, the set is padded.
 * Brute force: sort all n positions by (score desc, position asc), keep the
 * first min(K, n), emit them in ascending position order, pad with -1. */
typedef struct {
    const double *row;
} topk_ctx;

static int by_score_then_pos(const void *a, const void *b, void *arg)
{
    const double *row = ((const topk_ctx *)arg)->row;
    int32_t ia = *(const int32_t *)a, ib = *(const int32_t *)b;
    if (row[ia] > row[ib]) return -1;
    if (row[ia] < row[ib]) return 1;
    return (ia < ib) ? -1 : (ia > ib);
}

static int ascending_i32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x < y) ? -1 : (x > y);
}

void orc_topk(const double *scores, int64_t ld, const int64_t *n, int64_t nrows, int K, int32_t *idx_out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t len = n[r];
        int32_t *out = idx_out + r * (int64_t)K;
        int64_t take = len < K ? len : K;
        int32_t *ord = (int32_t *)malloc(sizeof(int32_t) * (size_t)(len > 0 ? len : 1));
        for (int64_t s = 0; s < len; ++s)
            ord[s] = (int32_t)s;
        if (len > K) {
            topk_ctx ctx = { scores + r * ld };
            qsort_r(ord, (size_t)len, sizeof(int32_t), by_score_then_pos, &ctx);
            qsort(ord, (size_t)take, sizeof(int32_t), ascending_i32);
        }
        for (int64_t j = 0; j < take; ++j)
            out[j] = ord[j];
        for (int64_t j = take; j < K; ++j)
            out[j] = -1;
        free(ord);
    }
}

/* ------------------------------------------- a3-a5: sparse attention + gate
 * [HAT §3.3]: exact attention over the gathered candidate rows, then the gate
 * scales the attention output.
 * [F2S "Fine-Grained Sparse Attention: Indexer Plus Top-K", pseudocode]:
 * attention(q, gather(k, idx), gather(v, idx)) followed by g = sigmoid(...).
 * [SEL §3.2]: the attention over the selected set is the standard one.
 * [SAD §4 "Output gating"]: per-channel or per-head scaling of the output.
 * [SAD §2]: query heads share one KV head (MQA); a latent row can serve as
 * both K and V (V = its first d_v dims).
 * For each listed token rows[r] and head h, over the valid entries s_j of
 * idx[r*K ...] (entries < 0 are padding and are skipped):
 *   z_j = scale * sum_d q[i,h,d] K[s_j,d];  m = max_j z_j;
 *   p_j = exp(z_j - m) / sum_j' exp(z_j' - m);  o[c] = sum_j p_j V[s_j,c];
 *   y[c] = o[c] / (1 + exp(-G));  lse = m + log(sum_j exp(z_j - m)).
 * A row with no valid entry yields y = 0 and lse = -inf. */
static double gate_of(int dtype, const void *gate, int per_channel, int64_t i, int h, int Hq, int dv, int c)
{
    double g = per_channel ? load(dtype, gate, ((int64_t)i * Hq + h) * dv + c)
                           : load(dtype, gate, (int64_t)i * Hq + h);
    return 1.0 / (1.0 + exp(-g));
}

void orc_sparse_attn(const orc_batch *bt, int dtype, const void *q, int Hq, int dqk,
                     const void *k_cache, const void *v_cache, int dv, int64_t row_stride,
                     const int32_t *idx, int K, const void *gate, int gate_per_channel, double scale,
                     const int64_t *rows, int64_t nrows, double *out, double *lse)
{
#pragma omp parallel
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        double *o = (double *)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int64_t r = 0; r < nrows; ++r) {
            for (int h = 0; h < Hq; ++h) {
                int64_t i = rows[r];
                int b = seq_of(bt, i);
                const int32_t *sel = idx + r * (int64_t)K;
                double m = -INFINITY;
                for (int j = 0; j < K; ++j) {
                    if (sel[j] < 0)
                        continue;
                    int64_t pr = phys_row(bt, b, sel[j]);
                    double dot = 0.0;
                    for (int d = 0; d < dqk; ++d)
                        dot += load(dtype, q, (i * Hq + h) * (int64_t)dqk + d) *
                               load(dtype, k_cache, pr * row_stride + d);
                    z[j] = scale * dot;
                    if (z[j] > m)
                        m = z[j];
                }
                double l = 0.0;
                for (int c = 0; c < dv; ++c)
                    o[c] = 0.0;
                for (int j = 0; j < K; ++j) {
                    if (sel[j] < 0)
                        continue;
                    double p = exp(z[j] - m);
                    l += p;
                    int64_t pr = phys_row(bt, b, sel[j]);
                    for (int c = 0; c < dv; ++c)
                        o[c] += p * load(dtype, v_cache, pr * row_stride + c);
                }
                double *y = out + (r * Hq + h) * (int64_t)dv;
                for (int c = 0; c < dv; ++c)
                    y[c] = (l > 0.0) ? (o[c] / l) * gate_of(dtype, gate, gate_per_channel, i, h, Hq, dv, c) : 0.0;
                if (lse)
                    lse[r * Hq + h] = (l > 0.0) ? m + log(l) : -INFINITY;
            }
        }
        free(o);
        free(z);
    }
}

/* ------------------------------------------------ dense control (no index)
 * [SEL §6 "Keep the structure reversible"]: the full-attention form stays as a
 * control branch.  Causal softmax attention of token i over every s <= pos(i),
 * then the same output gate.  Written separately from orc_sparse_attn; with
 * K >= n the sparse path must reproduce it. */
void orc_dense_attn(const orc_batch *bt, int dtype, const void *q, int Hq, int dqk,
                    const void *k_cache, const void *v_cache, int dv, int64_t row_stride,
                    const void *gate, int gate_per_channel, double scale,
                    const int64_t *rows, int64_t nrows, double *out)
{
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t r = 0; r < nrows; ++r) {
        for (int h = 0; h < Hq; ++h) {
            int64_t i = rows[r];
            int b;
            int64_t pos = pos_of(bt, i, &b);
            double *logit = (double *)malloc(sizeof(double) * (size_t)(pos + 1));
            double mx = -INFINITY;
            for (int64_t s = 0; s <= pos; ++s) {
                int64_t pr = phys_row(bt, b, s);
                double dot = 0.0;
                for (int d = 0; d < dqk; ++d)
                    dot += load(dtype, q, (i * Hq + h) * (int64_t)dqk + d) * load(dtype, k_cache, pr * row_stride + d);
                logit[s] = scale * dot;
                mx = logit[s] > mx ? logit[s] : mx;
            }
            double den = 0.0;
            for (int64_t s = 0; s <= pos; ++s)
                den += exp(logit[s] - mx);
            double *y = out + (r * Hq + h) * (int64_t)dv;
            for (int c = 0; c < dv; ++c) {
                double num = 0.0;
                for (int64_t s = 0; s <= pos; ++s)
                    num += exp(logit[s] - mx) * load(dtype, v_cache, phys_row(bt, b, s) * row_stride + c);
                y[c] = (num / den) * gate_of(dtype, gate, gate_per_channel, i, h, Hq, dv, c);
            }
            free(logit);
        }
    }
}

/* ------------------------------------------- cache append + fp8 quantisation
 * The step before the path: the new tokens' rows go into the paged caches.
 * [HAT §5 item 2]: the cache organisation decides indexing efficiency;
 * [F2S "Engineering Considerations" item 1]: paged cache management is on
 * the critical path; [HAT §5 item 3]: the indexer is sensitive to numeric
 * range in low precision.
 * Reading (the pages fix no format): an fp8 indexer key is stored as OCP
 * e4m3fn codes with one fp32 scale per token, s = max_d |x_d| / 448 (448 is
 * the largest e4m3fn value), code_d = e4m3fn(x_d / s) rounded to nearest,
 * ties to the even code, saturating at +-448.  s and x_d / s are single
 * precision operations: they decide an integer code, so the oracle takes
 * them in the kernel's precision.  A row of zeros gets s = 0 and codes 0. */

/* e4m3fn code of y: the representable value nearest to y, ties to the code
 * with an even mantissa; |y| >= 448 gives +-448; NaN gives S.1111.111. */
uint8_t orc_fp8_encode(float y)
{
    if (isnan(y))
        return 0x7F;
    int sign = signbit(y) ? 1 : 0;
    double a = fabs((double)y);
    if (a >= 448.0)
        return (uint8_t)((sign << 7) | 0x7E);
    /* binade [2^E, 2^(E+1)) holds 8 steps of 2^(E-3) for E >= -6; below 2^-6
     * (subnormals) the step stays 2^-9 */
    int E = a > 0.0 ? ilogb(a) : -6;
    if (E < -6)
        E = -6;
    double q = ldexp(1.0, E - 3);
    double r = rint(a / q);               /* a / q is exact; rint: nearest, ties to even */
    double v = r * q;                     /* <= 448 since a < 448 */
    int ef, mant;
    if (v < ldexp(1.0, -6)) {
        ef = 0;
        mant = (int)(v / ldexp(1.0, -9));
    } else {
        int E2 = ilogb(v);
        ef = E2 + 7;
        mant = (int)(v / ldexp(1.0, E2 - 3)) - 8;
    }
    return (uint8_t)((sign << 7) | (ef << 3) | mant);
}

static float loadf(int dtype, const void *base, int64_t i)
{
    return dtype == ORC_F32 ? ((const float *)base)[i] : (float)orc_bf16(((const uint16_t *)base)[i]);
}

/* One fp8 scale per row of x [rows, cols] (bf16 or f32), codes per element. */
void orc_quantize_rows(int src_dtype, const void *x, int64_t rows, int64_t cols, uint8_t *codes, float *scales)
{
    for (int64_t r = 0; r < rows; ++r) {
        float amax = 0.0f;
        for (int64_t c = 0; c < cols; ++c) {
            float v = fabsf(loadf(src_dtype, x, r * cols + c));
            amax = v > amax ? v : amax;
        }
        const float s = amax / 448.0f;
        scales[r] = s;
        for (int64_t c = 0; c < cols; ++c) {
            const float v = loadf(src_dtype, x, r * cols + c);
            codes[r * cols + c] = amax > 0.0f ? orc_fp8_encode(v / s) : 0;
        }
    }
}

/* Write new token i's rows at the physical row of its position pos(i):
 *   k_cache[row, 0:d_qk] = k_new[i, :]; v_cache[row, 0:d_v] = v_new[i, :]
 *   (v_new NULL: the latent layout, V is part of the K row);
 *   k_idx_cache[row, :] = k_idx_new[i, :] (copied when idx_dtype ==
 *   src_dtype) or its fp8 codes with k_scale_cache[row] = its scale.
 * Caches are raw element arrays indexed by physical row (row stride
 * row_stride elements for K/V, d_i for the indexer keys). */
void orc_cache_append(const orc_batch *bt, int64_t T, int kv_dtype, const void *k_new, int d_qk, const void *v_new,
                      int d_v, void *k_cache, void *v_cache, int64_t row_stride, int src_dtype,
                      const void *k_idx_new, int d_i, int idx_dtype, void *k_idx_cache, float *k_scale_cache)
{
    const int64_t esz = kv_dtype == ORC_F32 ? 4 : 2;
    const int64_t isz = src_dtype == ORC_F32 ? 4 : 2;
    for (int64_t i = 0; i < T; ++i) {
        int b;
        const int64_t pos = pos_of(bt, i, &b);
        const int64_t row = phys_row(bt, b, pos);
        memcpy((char *)k_cache + row * row_stride * esz, (const char *)k_new + i * d_qk * esz, (size_t)(d_qk * esz));
        if (v_new)
            memcpy((char *)v_cache + row * row_stride * esz, (const char *)v_new + i * d_v * esz,
                   (size_t)(d_v * esz));
        if (idx_dtype == ORC_FP8)
            orc_quantize_rows(src_dtype, (const char *)k_idx_new + i * d_i * isz, 1, d_i,
                              (uint8_t *)k_idx_cache + row * d_i, k_scale_cache + row);
        else
            memcpy((char *)k_idx_cache + row * d_i * isz, (const char *)k_idx_new + i * d_i * isz,
                   (size_t)(d_i * isz));
    }
}

/* --------------------------------------------- block-level selection
 * [SEL §3.2], pseudocode: pool the keys by block, score the blocks with the
 * queries, keep the top-k blocks, gather them and run exact attention within
 * them; [SAD §3] "block sparsity with top-k routing": query-to-block relevance
 * at block granularity, only the top blocks take part in the fine-grained
 * computation; [SEL §4.1]: the effective length drops from N to k*b.
 * Readings (the pages fix none of these):
 *   - a block is one page of the paged cache (b = page_size): block j of
 *     sequence b covers positions [j*b, min((j+1)*b, L_b));
 *   - the pooled key of a block is the mean of its K rows (first d_qk
 *     elements of each cache row);
 *   - the query heads share one selection (they share a KV head, [SAD §2]),
 *     so a block's score sums their dots:
 *         S[i, j] = sum_h q[i,h,:] . kbar_j
 *     over the candidate blocks of token i, those whose first position is
 *     <= pos(i);
 *   - the selected blocks' positions s <= pos(i) form the index list of the
 *     exact attention (a2-a5 unchanged). */

/* kbar[page, :] for every page a sequence uses, indexed by physical page. */
void orc_block_pool(const orc_batch *bt, int dtype, const void *k_cache, int dqk, int64_t row_stride, double *kbar)
{
    const int ps = bt->page_size;
    for (int b = 0; b < bt->num_seqs; ++b) {
        const int64_t L = bt->ctx_len[b];
        const int64_t nb = (L + ps - 1) / ps;
        for (int64_t j = 0; j < nb; ++j) {
            const int64_t page = bt->page_table[(int64_t)b * bt->max_pages + j];
            const int64_t len = (L - j * ps) < ps ? (L - j * ps) : ps;
            for (int d = 0; d < dqk; ++d) {
                double sum = 0.0;
                for (int64_t t = 0; t < len; ++t)
                    sum += load(dtype, k_cache, (page * ps + t) * row_stride + d);
                kbar[page * dqk + d] = sum / (double)len;
            }
        }
    }
}

/* S[r, j] for the candidate blocks j of token rows[r]; the rest of the row is left untouched. */
void orc_block_scores(const orc_batch *bt, int dtype, const void *q, int Hq, int dqk, const double *kbar,
                      const int64_t *rows, int64_t nrows, double *scores, int64_t ld)
{
    const int ps = bt->page_size;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows[r];
        int b;
        const int64_t pos = pos_of(bt, i, &b);
        for (int64_t j = 0; j <= pos / ps; ++j) {
            const int64_t page = bt->page_table[(int64_t)b * bt->max_pages + j];
            double s = 0.0;
            for (int h = 0; h < Hq; ++h) {
                double dot = 0.0;
                for (int d = 0; d < dqk; ++d)
                    dot += load(dtype, q, (i * Hq + h) * (int64_t)dqk + d) * kbar[page * dqk + d];
                s += dot;
            }
            scores[r * ld + j] = s;
        }
    }
}

/* Positions of the selected blocks (blk[r, :], block ids, -1 = none) that are
 * <= pos(rows[r]), in the order the blocks are listed, then -1 up to kb*b. */
void orc_block_expand(const orc_batch *bt, const int32_t *blk, int kb, const int64_t *rows, int64_t nrows,
                      int32_t *out)
{
    const int ps = bt->page_size;
    const int64_t w = (int64_t)kb * ps;
    for (int64_t r = 0; r < nrows; ++r) {
        int b;
        const int64_t pos = pos_of(bt, rows[r], &b);
        int64_t n = 0;
        for (int k = 0; k < kb; ++k) {
            const int32_t j = blk[r * kb + k];
            if (j < 0)
                continue;
            for (int t = 0; t < ps; ++t) {
                const int64_t p = (int64_t)j * ps + t;
                if (p <= pos)
                    out[r * w + n++] = (int32_t)p;
            }
        }
        for (; n < w; ++n)
            out[r * w + n] = -1;
    }
}

/* ------------------------------------------ branch fusion with a local branch
 * [SAD §3] pseudocode and §4 "branch fusion gating": a sparse branch and a
 * sliding-window local branch, combined by a sigmoid gate,
 *     y = g * sparse_out + (1 - g) * local_out,  g = sigmoid(G);
 * the local branch keeps nearby context whatever the selection.
 * Readings: the local branch is exact causal softmax attention of token i over
 * the window positions max(0, pos(i) - w + 1) .. pos(i), with the same q, K,
 * V and softmax scale; G is per head or per channel like the output gate.
 * Each branch is the path's attention with its gate at +inf (sigmoid = 1):
 * the fusion applies the gate once. */

/* The window positions of each listed token, ascending, then -1 up to w. */
void orc_window_indices(const orc_batch *bt, int w, const int64_t *rows, int64_t nrows, int32_t *out)
{
    for (int64_t r = 0; r < nrows; ++r) {
        int b;
        const int64_t pos = pos_of(bt, rows[r], &b);
        const int64_t lo = pos - w + 1 > 0 ? pos - w + 1 : 0;
        int64_t n = 0;
        for (int64_t s = lo; s <= pos; ++s)
            out[r * w + n++] = (int32_t)s;
        for (; n < w; ++n)
            out[r * w + n] = -1;
    }
}

/* y[r, h, c] = g * a + (1 - g) * b with g = sigmoid(G) of token rows[r]
 * (a, b, y: [nrows, Hq, dv] double; G raw in dtype, [T, Hq, dv] or [T, Hq]). */
void orc_branch_fuse(int dtype, const double *a, const double *b, const void *gate, int per_channel, int Hq, int dv,
                     const int64_t *rows, int64_t nrows, double *y)
{
    for (int64_t r = 0; r < nrows; ++r)
        for (int h = 0; h < Hq; ++h)
            for (int c = 0; c < dv; ++c) {
                const double g = gate_of(dtype, gate, per_channel, rows[r], h, Hq, dv, c);
                const int64_t e = (r * Hq + h) * (int64_t)dv + c;
                y[e] = g * a[e] + (1.0 - g) * b[e];
            }
}

/* ------------------------------------------ backward over fixed indices
 * The training-side pass the pages imply for the selected set ([HAT §3.3]:
 * exact attention over kv_history[idx] times the gate; [F2S] pseudocode: the
 * indices come from a non-differentiable Top-K, so gradients flow through the
 * attention and the gate only, not through the selection or the indexer).
 * For token i, head h, valid entries s_j of idx[i, :], with the forward's
 *     z_j = scale q.K_j, P_j = softmax(z)_j, o = sum_j P_j V_j, y = o * g, g = sigmoid(G):
 *     dG   = dy * o * g * (1 - g)           (per channel; summed over c per head)
 *     do   = dy * g
 *     dP_j = do . V_j,  D = sum_j P_j dP_j,  dz_j = P_j (dP_j - D)
 *     dq  += scale * sum_j dz_j K_j
 *     dK[row(s_j)] += scale * dz_j q,   dV[row(s_j)] += P_j do   (scatter-add)
 * All in double from the exactly decoded inputs; dK and dV are indexed by
 * physical cache row (row stride row_stride), and for the latent layout the
 * caller passes the same array for both. */
void orc_sparse_attn_bwd(const orc_batch *bt, int dtype, const void *q, int Hq, int dqk, const void *k_cache,
                         const void *v_cache, int dv, int64_t row_stride, const int32_t *idx, int K, const void *gate,
                         int gate_per_channel, double scale, const void *dy, int64_t T, double *dq, double *dk,
                         double *dvv, double *dgate)
{
    double *z = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    double *dp = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    double *o = (double *)malloc(sizeof(double) * (size_t)dv);
    double *dov = (double *)malloc(sizeof(double) * (size_t)dv);
    for (int64_t i = 0; i < T; ++i) {
        const int b = seq_of(bt, i);
        const int32_t *sel = idx + i * (int64_t)K;
        for (int h = 0; h < Hq; ++h) {
            const int64_t qo = (i * Hq + h) * (int64_t)dqk;
            double m = -INFINITY;
            for (int j = 0; j < K; ++j) {
                if (sel[j] < 0)
                    continue;
                const int64_t pr = phys_row(bt, b, sel[j]);
                double dot = 0.0;
                for (int d = 0; d < dqk; ++d)
                    dot += load(dtype, q, qo + d) * load(dtype, k_cache, pr * row_stride + d);
                z[j] = scale * dot;
                if (z[j] > m)
                    m = z[j];
            }
            double l = 0.0;
            for (int j = 0; j < K; ++j)
                if (sel[j] >= 0)
                    l += exp(z[j] - m);
            for (int c = 0; c < dv; ++c)
                o[c] = 0.0;
            for (int j = 0; j < K; ++j) {
                if (sel[j] < 0)
                    continue;
                z[j] = exp(z[j] - m) / l;            /* z now holds P_j */
                const int64_t pr = phys_row(bt, b, sel[j]);
                for (int c = 0; c < dv; ++c)
                    o[c] += z[j] * load(dtype, v_cache, pr * row_stride + c);
            }
            const int64_t yo = (i * Hq + h) * (int64_t)dv;
            double dgh = 0.0;
            for (int c = 0; c < dv; ++c) {
                const double g = gate_of(dtype, gate, gate_per_channel, i, h, Hq, dv, c);
                const double dyc = load(dtype, dy, yo + c);
                dov[c] = dyc * g;
                const double dgc = dyc * o[c] * g * (1.0 - g);
                if (gate_per_channel)
                    dgate[yo + c] = dgc;
                else
                    dgh += dgc;
            }
            if (!gate_per_channel)
                dgate[i * Hq + h] = dgh;
            if (l <= 0.0) {
                for (int d = 0; d < dqk; ++d)
                    dq[qo + d] = 0.0;
                continue;
            }
            double D = 0.0;
            for (int j = 0; j < K; ++j) {
                if (sel[j] < 0)
                    continue;
                const int64_t pr = phys_row(bt, b, sel[j]);
                double s = 0.0;
                for (int c = 0; c < dv; ++c)
                    s += dov[c] * load(dtype, v_cache, pr * row_stride + c);
                dp[j] = s;
                D += z[j] * s;
            }
            for (int d = 0; d < dqk; ++d)
                dq[qo + d] = 0.0;
            for (int j = 0; j < K; ++j) {
                if (sel[j] < 0)
                    continue;
                const int64_t pr = phys_row(bt, b, sel[j]);
                const double dz = z[j] * (dp[j] - D);
                for (int d = 0; d < dqk; ++d) {
                    dq[qo + d] += scale * dz * load(dtype, k_cache, pr * row_stride + d);
                    dk[pr * row_stride + d] += scale * dz * load(dtype, q, qo + d);
                }
                for (int c = 0; c < dv; ++c)
                    dvv[pr * row_stride + c] += z[j] * dov[c];
            }
        }
    }
    free(dov);
    free(o);
    free(dp);
    free(z);
}
