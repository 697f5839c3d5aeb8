/*
 * gqa_oracle.c -- plain, slow, fp64 CPU oracle for grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code with the HIP kernels.
 *
 * What it computes (per output row, all arithmetic in double):
 *   The ADR-0060 page ("AHBM GQA Fused Attention kernel (Llama3-70B)")
 *   describes FlashAttention tiling plus an online softmax and states in its
 *   "Algorithm lineage" paragraph that it introduces no new mathematics: the
 *   tiled kernel reaches exactly softmax(scale * Q K^T + causal mask) V.
 *   So this oracle is that definition written out directly, in the two-pass
 *   form (row max first, then exponentials and sums), which is also how the
 *   pccx page ("Gemma 3N E4B on pccx v002 -- Execution / Scheduling",
 *   section 3, per-token decode flow) runs decode attention: a score pass
 *   that finds the max, a softmax pass, then scores times V.
 *
 *   For a query row (b, t, h) with KV head kv = h / G, G = H_q / H_kv
 *   (the G query heads of one KV head are the group folded into M, ADR-0060
 *   TL;DR and section 5.2):
 *     s_j   = scale * sum_x Q[b,t,h,x] * K[b,j,kv,x]     for visible j
 *     m     = max_j s_j
 *     l     = sum_j exp(s_j - m)
 *     O[x]  = sum_j exp(s_j - m) * V[b,j,kv,x] / l
 *     LSE   = m + ln(l)                                  (natural log)
 *   Visible keys, causal prefill (ADR-0060 section 5.4 tile classes; diagonal
 *   included, query at absolute position q_offset + t sees key j iff
 *   j <= q_offset + t); non-causal prefill: every key j < S_kv; decode
 *   (section 5.2): every key of the sequence, j < kv_len[b].
 *
 *   The split form follows ADR-0060 section 4 (Reduction): each KV shard
 *   yields an unnormalised partial (m_i, l_i, O_i); partials are merged by
 *   m = max(m_a, m_b), s_a = exp(m_a - m), s_b = exp(m_b - m),
 *   l = l_a s_a + l_b s_b, O = O_a s_a + O_b s_b, and O / l is taken once at
 *   the end.
 *
 *   Sink + local-window mask (pccx page, "Gemma 3N E4B on pccx v002 --
 *   Execution / Scheduling", section 4, KV cache management of the
 *   fixed-size ring cache).  Reading used here: key j is visible to the
 *   query at absolute position p iff j <= p and (j < sink or j > p - window),
 *   so a query keeps the leading `sink` positions plus the `window` newest
 *   positions ending at its own.
 *   gqa_oracle_prefill_window computes exactly that over the logical
 *   (unwrapped) key sequence; where a ring buffer stores the keys is the
 *   kernel's business, not the oracle's.
 *
 * Layouts (all row-major, contiguous):
 *   prefill  Q, O [B, T_q, H_q, d]   K, V [B, S_kv, H_kv, d]   LSE [B, T_q, H_q]
 *   decode   Q, O [B, H_q, d]        K, V packed [sum_b kv_len[b], H_kv, d],
 *            sequence b starting at row sum_{b' < b} kv_len[b'].
 * Inputs are float (the bf16 test inputs are exactly representable in float);
 * every product and sum is formed in double from those exact values.
 *
 * `rows` (nullable) selects a subset of output rows by flat index
 * (prefill: (b*T_q + t)*H_q + h; decode: b*H_q + h); results are then written
 * densely, row i of the output holding rows[i].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EARG 1
#define ORACLE_ENOMEM 2

static int set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

int gqa_oracle_num_threads(int nthreads) { return set_threads(nthreads); }

/* Attention of one query vector against keys [j0, j1) of one (sequence, KV
 * head) slice.  kbase/vbase point at key row 0 of the slice; `stride` is the
 * distance in floats between consecutive key rows.  Writes the unnormalised
 * partial: *m_out = max score, *l_out = sum exp(s - m), acc[x] = sum exp(s - m) V.
 * `s` is scratch of at least (j1 - j0) doubles.  An empty range gives
 * m = -inf, l = 0, acc = 0. */
static void partial_row(const float *qrow, const float *kbase, const float *vbase,
                        int64_t stride, int64_t j0, int64_t j1, int d, double scale,
                        double *s, double *m_out, double *l_out, double *acc) {
    double m = -INFINITY;
    for (int64_t j = j0; j < j1; ++j) {
        const float *krow = kbase + j * stride;
        double dot = 0.0;
        for (int x = 0; x < d; ++x) dot += (double)qrow[x] * (double)krow[x];
        double sj = scale * dot;
        s[j - j0] = sj;
        if (sj > m) m = sj;
    }
    double l = 0.0;
    for (int x = 0; x < d; ++x) acc[x] = 0.0;
    for (int64_t j = j0; j < j1; ++j) {
        double p = exp(s[j - j0] - m);
        l += p;
        const float *vrow = vbase + j * stride;
        for (int x = 0; x < d; ++x) acc[x] += p * (double)vrow[x];
    }
    *m_out = m;
    *l_out = l;
}

static int check_heads(int H_q, int H_kv, int d) {
    return H_q < 1 || H_kv < 1 || d < 1 || (H_q % H_kv) != 0;
}

int gqa_oracle_prefill(const float *q, const float *k, const float *v, double *o,
                       double *lse, int B, int T_q, int S_kv, int H_q, int H_kv, int d,
                       double scale, int causal, int q_offset, const int64_t *rows,
                       int64_t n_rows, int nthreads) {
    if (!q || !k || !v || !o || B < 1 || T_q < 1 || S_kv < 1 || check_heads(H_q, H_kv, d))
        return ORACLE_EARG;
    if (causal && (q_offset < 0 || (int64_t)q_offset + T_q > S_kv)) return ORACLE_EARG;
    const int G = H_q / H_kv;
    const int64_t total = (int64_t)B * T_q * H_q;
    const int64_t n = rows ? n_rows : total;
    const int64_t kstride = (int64_t)H_kv * d;
    int bad = 0;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)S_kv);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !acc) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t i = 0; i < n; ++i) {
                int64_t r = rows ? rows[i] : i;
                if (r < 0 || r >= total) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                int h = (int)(r % H_q);
                int64_t bt = r / H_q;
                int t = (int)(bt % T_q);
                int b = (int)(bt / T_q);
                int kv = h / G;
                int64_t nvis = causal ? (int64_t)q_offset + t + 1 : S_kv;
                const float *qrow = q + r * d;
                const float *kb = k + ((int64_t)b * S_kv * H_kv + kv) * d;
                const float *vb = v + ((int64_t)b * S_kv * H_kv + kv) * d;
                double m, l;
                partial_row(qrow, kb, vb, kstride, 0, nvis, d, scale, s, &m, &l, acc);
                for (int x = 0; x < d; ++x) o[i * d + x] = acc[x] / l;
                if (lse) lse[i] = m + log(l);
            }
        }
        free(s);
        free(acc);
    }
    return bad ? ORACLE_EARG : ORACLE_OK;
}

/* Sink + local-window prefill: like gqa_oracle_prefill with causal = 1, but
 * query t (position p = q_offset + t) sees key j iff j <= p and
 * (j < sink or j > p - window); window >= 1, sink >= 0.  Two-pass softmax over
 * the visible keys, taken one by one in key order. */
int gqa_oracle_prefill_window(const float *q, const float *k, const float *v, double *o,
                              double *lse, int B, int T_q, int S_kv, int H_q, int H_kv, int d,
                              double scale, int q_offset, int window, int sink,
                              const int64_t *rows, int64_t n_rows, int nthreads) {
    if (!q || !k || !v || !o || B < 1 || T_q < 1 || S_kv < 1 || check_heads(H_q, H_kv, d))
        return ORACLE_EARG;
    if (q_offset < 0 || (int64_t)q_offset + T_q > S_kv || window < 1 || sink < 0)
        return ORACLE_EARG;
    const int G = H_q / H_kv;
    const int64_t total = (int64_t)B * T_q * H_q;
    const int64_t n = rows ? n_rows : total;
    const int64_t kstride = (int64_t)H_kv * d;
    int bad = 0;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)S_kv);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !acc) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t i = 0; i < n; ++i) {
                int64_t r = rows ? rows[i] : i;
                if (r < 0 || r >= total) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                int h = (int)(r % H_q);
                int64_t bt = r / H_q;
                int t = (int)(bt % T_q);
                int b = (int)(bt / T_q);
                int kv = h / G;
                int64_t p = (int64_t)q_offset + t;
                const float *qrow = q + r * d;
                const float *kb = k + ((int64_t)b * S_kv * H_kv + kv) * d;
                const float *vb = v + ((int64_t)b * S_kv * H_kv + kv) * d;
                /* pass 1: scores of the visible keys and their max */
                double m = -INFINITY;
                for (int64_t j = 0; j <= p; ++j) {
                    if (!(j < sink || j > p - window)) continue;
                    const float *krow = kb + j * kstride;
                    double dot = 0.0;
                    for (int x = 0; x < d; ++x) dot += (double)qrow[x] * (double)krow[x];
                    s[j] = scale * dot;
                    if (s[j] > m) m = s[j];
                }
                /* pass 2: exponentials, their sum and the weighted sum of V */
                double l = 0.0;
                for (int x = 0; x < d; ++x) acc[x] = 0.0;
                for (int64_t j = 0; j <= p; ++j) {
                    if (!(j < sink || j > p - window)) continue;
                    double pj = exp(s[j] - m);
                    l += pj;
                    const float *vrow = vb + j * kstride;
                    for (int x = 0; x < d; ++x) acc[x] += pj * (double)vrow[x];
                }
                for (int x = 0; x < d; ++x) o[i * d + x] = acc[x] / l;
                if (lse) lse[i] = m + log(l);
            }
        }
        free(s);
        free(acc);
    }
    return bad ? ORACLE_EARG : ORACLE_OK;
}

static int decode_offsets(int B, const int32_t *kv_len, int64_t *off) {
    int64_t acc = 0;
    for (int b = 0; b < B; ++b) {
        if (kv_len[b] < 1) return ORACLE_EARG;
        off[b] = acc;
        acc += kv_len[b];
    }
    off[B] = acc;
    return ORACLE_OK;
}

/* Decode, unsplit when num_splits == 0.  With num_splits > 0 each sequence's
 * keys are cut into min(num_splits, kv_len) contiguous near-equal shards
 * [floor(i n / ns), floor((i+1) n / ns)); each shard's unnormalised partial
 * is folded into the running result with the ADR-0060 section 4 merge, in
 * shard order, and O / l is taken once at the end. */
int gqa_oracle_decode(const float *q, const float *k, const float *v, double *o,
                      double *lse, int B, int H_q, int H_kv, int d, const int32_t *kv_len,
                      double scale, int num_splits, const int64_t *rows, int64_t n_rows,
                      int nthreads) {
    if (!q || !k || !v || !o || !kv_len || B < 1 || check_heads(H_q, H_kv, d) ||
        num_splits < 0)
        return ORACLE_EARG;
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * ((size_t)B + 1));
    if (!off) return ORACLE_ENOMEM;
    if (decode_offsets(B, kv_len, off) != ORACLE_OK) {
        free(off);
        return ORACLE_EARG;
    }
    int32_t maxlen = 0;
    for (int b = 0; b < B; ++b)
        if (kv_len[b] > maxlen) maxlen = kv_len[b];
    const int G = H_q / H_kv;
    const int64_t total = (int64_t)B * H_q;
    const int64_t n = rows ? n_rows : total;
    const int64_t kstride = (int64_t)H_kv * d;
    int bad = 0;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)maxlen);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        double *run = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !acc || !run) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t i = 0; i < n; ++i) {
                int64_t r = rows ? rows[i] : i;
                if (r < 0 || r >= total) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                int h = (int)(r % H_q);
                int b = (int)(r / H_q);
                int kv = h / G;
                int64_t len = kv_len[b];
                const float *qrow = q + r * d;
                const float *kb = k + (off[b] * H_kv + kv) * d;
                const float *vb = v + (off[b] * H_kv + kv) * d;
                double m, l;
                if (num_splits == 0) {
                    partial_row(qrow, kb, vb, kstride, 0, len, d, scale, s, &m, &l, acc);
                    for (int x = 0; x < d; ++x) run[x] = acc[x];
                } else {
                    int64_t ns = num_splits < len ? num_splits : len;
                    m = -INFINITY;
                    l = 0.0;
                    for (int x = 0; x < d; ++x) run[x] = 0.0;
                    for (int64_t sp = 0; sp < ns; ++sp) {
                        int64_t j0 = sp * len / ns, j1 = (sp + 1) * len / ns;
                        double mb, lb;
                        partial_row(qrow, kb, vb, kstride, j0, j1, d, scale, s, &mb, &lb, acc);
                        /* merge (m, l, run) with (mb, lb, acc) */
                        double mm = m > mb ? m : mb;
                        double sa = (m == -INFINITY) ? 0.0 : exp(m - mm);
                        double sb = (mb == -INFINITY) ? 0.0 : exp(mb - mm);
                        l = l * sa + lb * sb;
                        for (int x = 0; x < d; ++x) run[x] = run[x] * sa + acc[x] * sb;
                        m = mm;
                    }
                }
                for (int x = 0; x < d; ++x) o[i * d + x] = run[x] / l;
                if (lse) lse[i] = m + log(l);
            }
        }
        free(s);
        free(acc);
        free(run);
    }
    free(off);
    return bad ? ORACLE_EARG : ORACLE_OK;
}
