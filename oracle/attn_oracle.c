/*
 * attn_oracle.c -- plain, slow, fp64 CPU oracle for scaled dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the HIP library; neither includes or links the other.
 *
 * What it computes (page "Shape-Aware Attention", section "Inspiration",
 * the attention equation: Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V), written out as its
 * plain definition with an explicit softmax, one query row at a time:
 *
 *   p_i   = kv_len - S_q + i          absolute position of query row i
 *                                     (queries sit at the end of the valid
 *                                      K/V prefix; equals i when S_q = kv_len)
 *   Vis_i = { j : 0 <= j < kv_len }   non-causal
 *         = { j : 0 <= j <= p_i }     causal (key j visible to query i iff j <= p_i)
 *   s_ij  = scale * sum_d q[i,d] k[j,d]                  (j in Vis_i)
 *   m_i   = max_j s_ij
 *   e_ij  = exp(s_ij - m_i),   l_i = sum_j e_ij
 *   o[i,d] = (sum_j e_ij v[j,d]) / l_i
 *
 * Subtracting m_i is the textbook stable softmax and leaves the value unchanged
 * in exact arithmetic.  The online (running max / running sum / rescaled
 * accumulator) formulation the fast path uses reaches this same value exactly
 * in real arithmetic (page "GPU Kernel for a Transformer Layer", section "What
 * we learned"), so the oracle is the definition, not the tiled algorithm.
 *
 * Precision: every product, sum, exp and divide is IEEE double with libm exp.
 * Inputs are float32 arrays holding the exact stored values of the fp32, fp16
 * or bf16 tensors (every fp16 and bf16 value is exactly a float32), so the
 * oracle sees the same rounded inputs the device sees.  No intermediate value
 * (scores, probabilities, accumulator) is ever rounded to a narrower type
 * (page "Shape-Aware Attention", section "Challenges we ran into": the fused
 * path keeps the probabilities unrounded).
 *
 * Layout: q is [B,H,S_q,D], k and v are [B,H,S_kv,D], contiguous, row-major.
 * Only K/V rows j < kv_len are read.  o is double, [B,H,S_q,D], or
 * [B,H,n_rows,D] when a row list is given (then only those query rows of every
 * (b,h) are computed, in the given order).
 *
 * Work is split over (b,h,row) with OpenMP; each row's summation order is
 * fixed (ascending j, ascending d), so results do not depend on the thread
 * count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Return codes. */
#define ORACLE_OK 0
#define ORACLE_E_ARG 1
#define ORACLE_E_ROWS 2
#define ORACLE_E_NOMEM 3

/* One query row of one (b,h) head.  qi points at the row (D floats), kh/vh at
 * the head's K/V ([S_kv, D]), out at D doubles; s is scratch for n_vis doubles. */
static void one_row(const float *qi, const float *kh, const float *vh, double *out,
                    int64_t D, int64_t n_vis, double scale, double *s)
{
    /* scores over the visible keys */
    for (int64_t j = 0; j < n_vis; ++j) {
        const float *kj = kh + j * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d)
            dot += (double)qi[d] * (double)kj[d];
        s[j] = scale * dot;
    }
    /* explicit softmax: max, exponentials, normaliser */
    double m = s[0];
    for (int64_t j = 1; j < n_vis; ++j)
        if (s[j] > m) m = s[j];
    double l = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    /* probability-weighted sum of value rows */
    for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t j = 0; j < n_vis; ++j)
            acc += s[j] * (double)vh[j * D + d];
        out[d] = acc / l;
    }
}

/*
 * oracle_attn_f64: see the file header for the definition.
 *   rows/n_rows: optional list of query row indices (each in [0,S_q)); NULL
 *                computes every row.
 *   n_threads:   OpenMP threads, <= 0 for the runtime default.
 * Returns ORACLE_OK, or an ORACLE_E_* code without writing o.
 */
int oracle_attn_f64(const float *q, const float *k, const float *v, double *o,
                    int64_t B, int64_t H, int64_t S_q, int64_t S_kv, int64_t D,
                    int causal, double scale, int64_t kv_len,
                    const int64_t *rows, int64_t n_rows, int n_threads)
{
    if (!q || !k || !v || !o) return ORACLE_E_ARG;
    if (B < 1 || H < 1 || S_q < 1 || S_kv < 1 || D < 1) return ORACLE_E_ARG;
    if (kv_len < 1 || kv_len > S_kv) return ORACLE_E_ARG;
    if (causal && S_q > kv_len) return ORACLE_E_ARG;  /* some row would see no key */
    if (!isfinite(scale)) return ORACLE_E_ARG;
    int64_t nr = rows ? n_rows : S_q;
    if (nr < 1) return ORACLE_E_ROWS;
    if (rows)
        for (int64_t r = 0; r < nr; ++r)
            if (rows[r] < 0 || rows[r] >= S_q) return ORACLE_E_ROWS;

    const int64_t total = B * H * nr;
    int failed = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)kv_len * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < total; ++t) {
            if (!s) continue;
            const int64_t bh = t / nr, r = t % nr;
            const int64_t i = rows ? rows[r] : r;
            const int64_t p = kv_len - S_q + i;
            const int64_t n_vis = causal ? p + 1 : kv_len;
            one_row(q + (bh * S_q + i) * D,
                    k + bh * S_kv * D, v + bh * S_kv * D,
                    o + (bh * nr + r) * D, D, n_vis, scale, s);
        }
        free(s);
    }
    return failed ? ORACLE_E_NOMEM : ORACLE_OK;
}

/* Threads the OpenMP runtime would use by default (for reporting). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
