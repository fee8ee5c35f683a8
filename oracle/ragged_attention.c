/*
 * Plain fp64 CPU oracle for ragged (varlen) batched prefill attention.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark use this file.  It shares no code, header, table or
 * helper with the GPU library: it is the textbook definition written out, so
 * that a reader can check it against the pages by eye.
 *
 * What it computes (page "Module flashinfer", module doc: N requests' attention
 * located by q_indptr / kv_indptr ragged offsets; functions
 * ragged_prefill_bf16_hd128 / _hd256: BF16, GQA, causal selectable):
 *
 *   for request b, query row i (0 <= i < qo_len), qo head h:
 *     kv head     hk = h / (num_qo_heads / num_kv_heads)        (GQA groups)
 *     visible j:  0 <= j < kv_len, and if causal j <= i + kv_len - qo_len
 *                 (bottom-right alignment; page "flashinfer-ai/flashinfer",
 *                 benchmarks README, attention flag --causal)
 *     s_j   = sm_scale * sum_d q[i,h,d] * k[j,hk,d]
 *     O     = sum_j exp(s_j - m) v[j,hk,:] / sum_j exp(s_j - m),  m = max_j s_j
 *     LSE   = m + log(sum_j exp(s_j - m))   (natural log of sum_j exp(s_j);
 *             the per-row log-sum-exp returned by the *_return_lse prefill
 *             entry points, page "flashinfer-ai/flashinfer", attention API,
 *             single request prefill)
 *   rows that see no key: O = 0, LSE = -inf.
 *
 * Inputs are the exact bf16 bit patterns the GPU receives; they are widened
 * to double (bf16 is the top half of an IEEE binary32).  All arithmetic is in
 * double, sums in ascending key order.  O is returned unrounded.
 *
 * An optional request-relative key window [key_lo, key_hi) further restricts
 * the visible keys; it yields the partial attention state of a key subset,
 * which merge_state (below) combines.
 *
 * OpenMP parallelises over independent (row, head) pairs only; each pair is
 * computed by the same sequential loop whatever the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* The number of keys visible to query row i: keys j < limit (before the key
 * window).  Causal masking aligns the diagonal with the end of the KV. */
static int64_t visible_limit(int64_t i, int64_t qo_len, int64_t kv_len, int causal)
{
    if (!causal)
        return kv_len;
    int64_t lim = i + kv_len - qo_len + 1;
    if (lim < 0)
        lim = 0;
    if (lim > kv_len)
        lim = kv_len;
    return lim;
}

/* Attention of one query row against keys [j_lo, j_hi) of one kv head. */
static void attend_one(const uint16_t *qrow, const uint16_t *kreq, const uint16_t *vreq,
                       int64_t kv_row_stride, int head_dim, int64_t j_lo, int64_t j_hi,
                       double sm_scale, double *s, double *out, double *lse_out)
{
    if (j_hi <= j_lo) {
        for (int d = 0; d < head_dim; ++d)
            out[d] = 0.0;
        *lse_out = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int64_t j = j_lo; j < j_hi; ++j) {
        const uint16_t *krow = kreq + j * kv_row_stride;
        double dot = 0.0;
        for (int d = 0; d < head_dim; ++d)
            dot += bf16_bits_to_double(qrow[d]) * bf16_bits_to_double(krow[d]);
        s[j - j_lo] = sm_scale * dot;
        if (s[j - j_lo] > m)
            m = s[j - j_lo];
    }
    for (int d = 0; d < head_dim; ++d)
        out[d] = 0.0;
    double z = 0.0;
    for (int64_t j = j_lo; j < j_hi; ++j) {
        double w = exp(s[j - j_lo] - m);
        z += w;
        const uint16_t *vrow = vreq + j * kv_row_stride;
        for (int d = 0; d < head_dim; ++d)
            out[d] += w * bf16_bits_to_double(vrow[d]);
    }
    for (int d = 0; d < head_dim; ++d)
        out[d] /= z;
    *lse_out = m + log(z);
}

static int check_args(const int32_t *q_indptr, const int32_t *kv_indptr, int batch,
                      int num_qo_heads, int num_kv_heads, int head_dim)
{
    if (batch < 0 || num_qo_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0)
        return -1;
    if (num_qo_heads % num_kv_heads != 0)
        return -1;
    for (int b = 0; b < batch; ++b) {
        if (q_indptr[b + 1] < q_indptr[b] || kv_indptr[b + 1] < kv_indptr[b])
            return -1;
    }
    if (batch > 0 && (q_indptr[0] < 0 || kv_indptr[0] < 0))
        return -1;
    return 0;
}

/* One (request, row, head) of the definition above, written to out/lse_out. */
static void attend_request_row(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const int32_t *q_indptr, const int32_t *kv_indptr, int b,
                               int64_t i, int h, int num_qo_heads, int num_kv_heads,
                               int head_dim, int causal, double sm_scale, int64_t key_lo,
                               int64_t key_hi, double *s, double *out, double *lse_out)
{
    int64_t q0 = q_indptr[b], k0 = kv_indptr[b];
    int64_t qo_len = q_indptr[b + 1] - q0;
    int64_t kv_len = kv_indptr[b + 1] - k0;
    int group = num_qo_heads / num_kv_heads;
    int hk = h / group;
    int64_t lim = visible_limit(i, qo_len, kv_len, causal);
    int64_t j_lo = key_lo > 0 ? key_lo : 0;
    int64_t j_hi = (key_hi >= 0 && key_hi < lim) ? key_hi : lim;
    const int64_t kv_row_stride = (int64_t)num_kv_heads * head_dim;
    const uint16_t *qrow = q + ((q0 + i) * num_qo_heads + h) * (int64_t)head_dim;
    const uint16_t *kreq = k + k0 * kv_row_stride + (int64_t)hk * head_dim;
    const uint16_t *vreq = v + k0 * kv_row_stride + (int64_t)hk * head_dim;
    attend_one(qrow, kreq, vreq, kv_row_stride, head_dim, j_lo, j_hi, sm_scale, s, out,
               lse_out);
}

static int64_t max_kv_len(const int32_t *kv_indptr, int batch)
{
    int64_t mx = 1;
    for (int b = 0; b < batch; ++b) {
        int64_t n = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
        if (n > mx)
            mx = n;
    }
    return mx;
}

/*
 * Full batch.  o: double [rows, num_qo_heads, head_dim], lse: double
 * [rows, num_qo_heads] with rows indexed like q; only rows inside some
 * request are written.  key_hi < 0 means "no upper bound".
 * Returns 0, or -1 on malformed arguments (nothing written).
 */
int oracle_ragged_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            double *o, double *lse, const int32_t *q_indptr,
                            const int32_t *kv_indptr, int batch, int num_qo_heads,
                            int num_kv_heads, int head_dim, int causal, double sm_scale,
                            int64_t key_lo, int64_t key_hi)
{
    if (check_args(q_indptr, kv_indptr, batch, num_qo_heads, num_kv_heads, head_dim))
        return -1;
    const int64_t smax = max_kv_len(kv_indptr, batch);
    for (int b = 0; b < batch; ++b) {
        const int64_t q0 = q_indptr[b];
        const int64_t qo_len = q_indptr[b + 1] - q0;
        const int64_t n = qo_len * num_qo_heads;
#pragma omp parallel
        {
            double *s = (double *)malloc((size_t)smax * sizeof(double));
#pragma omp for schedule(dynamic, 4)
            for (int64_t t = 0; t < n; ++t) {
                int64_t i = t / num_qo_heads;
                int h = (int)(t % num_qo_heads);
                double *out = o + ((q0 + i) * num_qo_heads + h) * (int64_t)head_dim;
                double *lo = lse + (q0 + i) * num_qo_heads + h;
                attend_request_row(q, k, v, q_indptr, kv_indptr, b, i, h, num_qo_heads,
                                   num_kv_heads, head_dim, causal, sm_scale, key_lo, key_hi,
                                   s, out, lo);
            }
            free(s);
        }
    }
    return 0;
}

/*
 * A chosen subset of (token row, qo head) pairs, for full-size checks where the
 * whole batch would take too long: row tokens[n] (index into q's rows, which
 * must lie inside some request) and heads[n].  o_out: double [n, head_dim],
 * lse_out: double [n].  Returns 0, or -1 on malformed arguments or a token
 * outside every request.
 */
int oracle_ragged_attention_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 const int32_t *q_indptr, const int32_t *kv_indptr,
                                 int batch, int num_qo_heads, int num_kv_heads,
                                 int head_dim, int causal, double sm_scale,
                                 const int64_t *tokens, const int32_t *heads, int64_t n,
                                 double *o_out, double *lse_out)
{
    if (check_args(q_indptr, kv_indptr, batch, num_qo_heads, num_kv_heads, head_dim))
        return -1;
    int *req = (int *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int));
    for (int64_t t = 0; t < n; ++t) {
        req[t] = -1;
        for (int b = 0; b < batch; ++b) {
            if (tokens[t] >= q_indptr[b] && tokens[t] < q_indptr[b + 1]) {
                req[t] = b;
                break;
            }
        }
        if (req[t] < 0 || heads[t] < 0 || heads[t] >= num_qo_heads) {
            free(req);
            return -1;
        }
    }
    const int64_t smax = max_kv_len(kv_indptr, batch);
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)smax * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n; ++t) {
            int b = req[t];
            attend_request_row(q, k, v, q_indptr, kv_indptr, b, tokens[t] - q_indptr[b],
                               heads[t], num_qo_heads, num_kv_heads, head_dim, causal,
                               sm_scale, 0, -1, s, o_out + t * (int64_t)head_dim, lse_out + t);
        }
        free(s);
    }
    free(req);
    return 0;
}

/*
 * Merge two attention states over disjoint key sets (the merge_state operation
 * of the cascade API, page "flashinfer-ai/flashinfer", "Merge Attention
 * States"): state (o, lse) is the softmax-weighted mean o of V over a key set
 * and the log-sum-exp lse of its scores; over the union,
 *   lse = log(exp(lse_a) + exp(lse_b))
 *   o   = o_a * exp(lse_a - lse) + o_b * exp(lse_b - lse).
 * An empty set has lse = -inf and leaves the other state unchanged.
 * o_*: double [n, head_dim]; lse_*: double [n].
 */
void oracle_merge_state(const double *o_a, const double *lse_a, const double *o_b,
                        const double *lse_b, double *o_out, double *lse_out, int64_t n,
                        int head_dim)
{
    for (int64_t r = 0; r < n; ++r) {
        double a = lse_a[r], b = lse_b[r];
        const double *va = o_a + r * (int64_t)head_dim;
        const double *vb = o_b + r * (int64_t)head_dim;
        double *vo = o_out + r * (int64_t)head_dim;
        if (a == -INFINITY && b == -INFINITY) {
            for (int d = 0; d < head_dim; ++d)
                vo[d] = 0.0;
            lse_out[r] = -INFINITY;
            continue;
        }
        double m = a > b ? a : b;
        double lse = m + log(exp(a - m) + exp(b - m));
        double wa = exp(a - lse), wb = exp(b - lse);
        for (int d = 0; d < head_dim; ++d)
            vo[d] = va[d] * wa + vb[d] * wb;
        lse_out[r] = lse;
    }
}

/*
 * Merge k attention states per row over pairwise disjoint key sets (the
 * merge_states operation of the same cascade API section).  By the
 * definition of the state, over the union of the k sets
 *   lse = log(sum_i exp(lse_i))
 *   o   = sum_i exp(lse_i - lse) * o_i,
 * with exp(lse_i - lse) the share of state i's softmax mass.  The largest
 * lse_i is factored out of the sum (exact in real arithmetic).  Empty states
 * (lse_i = -inf) carry no mass; if all are empty, o = 0 and lse = -inf.
 * o: double [n, k, head_dim]; lse: double [n, k]; out: [n, head_dim], [n].
 */
void oracle_merge_states(const double *o, const double *lse, double *o_out, double *lse_out,
                         int64_t n, int k, int head_dim)
{
    for (int64_t r = 0; r < n; ++r) {
        const double *l = lse + r * (int64_t)k;
        double *vo = o_out + r * (int64_t)head_dim;
        double m = -INFINITY;
        for (int i = 0; i < k; ++i)
            if (l[i] > m)
                m = l[i];
        for (int d = 0; d < head_dim; ++d)
            vo[d] = 0.0;
        if (m == -INFINITY) {
            lse_out[r] = -INFINITY;
            continue;
        }
        double total = 0.0;
        for (int i = 0; i < k; ++i)
            total += exp(l[i] - m);
        const double merged = m + log(total);
        for (int i = 0; i < k; ++i) {
            const double w = exp(l[i] - merged);
            const double *vi = o + (r * (int64_t)k + i) * head_dim;
            for (int d = 0; d < head_dim; ++d)
                vo[d] += w * vi[d];
        }
        lse_out[r] = merged;
    }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
