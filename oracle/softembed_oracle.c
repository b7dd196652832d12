/*
 * softembed_oracle.c -- plain fp64 CPU oracle of the self-conditioning soft
 * embedding.  TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg load this file's library.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * What it computes, with the passages it follows (calvarado04.com/tag/vllm,
 * "Where the shapes stop agreeing" and "The fix"; agentlenshq DiffusionGemma
 * overview, "sampling loop and entropy-bound denoising" and "self-conditioning
 * for stability"):
 *
 *   p_i      = softmax over the FULL vocabulary of logits row i (the sampler
 *              works on gathered, full-width logits)               [page 1, "Where the shapes stop agreeing"]
 *   m_i      = max_v l_iv, argmax_i = smallest v with l_iv = m_i  [page 2, convergence uses argmax]
 *   lse_i    = m_i + log sum_v exp(l_iv - m_i)                    (log-sum-exp, exact in real arithmetic)
 *   H_i      = -sum_v p_iv log p_iv  (nats, 0 log 0 = 0)          [page 2, entropy-bound acceptance]
 *   S_i,:    = sum_{v=s}^{e-1} p_iv W_shard[v-s, :]               [page 1, "The fix", the per-rank partial S^(r)]
 *   out_i,:  = gamma * S_i,:                                      [page 1, "The fix", the normaliser gamma]
 *
 * Everything is double precision; sums run sequentially in index order; there
 * is no blocking or reordering.  Rows are independent and are distributed over
 * OpenMP threads, which does not change any row's arithmetic.
 *
 * A diagnostic switch rounds each p_iv to bfloat16 (round to nearest, ties to
 * even) before the contraction, mirroring the cast of the probabilities to the
 * embedding dtype on page 1 ("The fix").  The gating comparisons use the
 * unrounded p.
 *
 * Preconditions: logits are finite.  Violations abort via the return code.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 bit pattern -> value: the 16 stored bits are the top half of an IEEE
 * binary32. */
static double bf16_bits_value(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a non-negative finite double to the nearest bfloat16 value (8
 * significant bits, exponent range of binary32), ties to even.  Written from
 * the definition of the format: normal numbers keep 8 significant bits; below
 * 2^-126 the spacing is fixed at 2^-133. */
double oracle_round_bf16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    double a = fabs(x);
    int e;
    (void)frexp(a, &e);             /* a = f * 2^e, f in [0.5, 1) */
    int q = e - 8;                  /* spacing of 8-significant-bit numbers */
    if (q < -133) q = -133;         /* subnormal spacing of bf16 */
    double r = ldexp(nearbyint(ldexp(a, -q)), q);   /* default mode: ties-to-even */
    return x < 0 ? -r : r;
}

/* Returns 0 on success, 1 if a non-finite logit was found. */
int oracle_row_stats(const float* logits, int64_t ld, int64_t n_rows, int64_t vocab,
                     double* row_max, int32_t* row_argmax, double* row_lse,
                     double* row_entropy)
{
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|| : bad)
    for (int64_t i = 0; i < n_rows; ++i) {
        const float* x = logits + i * ld;
        double m = (double)x[0];
        int64_t am = 0;
        for (int64_t v = 0; v < vocab; ++v) {
            if (!isfinite(x[v])) bad = 1;
            if ((double)x[v] > m) { m = (double)x[v]; am = v; }
        }
        double z = 0.0;
        for (int64_t v = 0; v < vocab; ++v) z += exp((double)x[v] - m);
        double lse = m + log(z);
        double h = 0.0;
        for (int64_t v = 0; v < vocab; ++v) {
            double p = exp((double)x[v] - lse);
            if (p > 0.0) h -= p * log(p);
        }
        row_max[i] = m;
        row_argmax[i] = (int32_t)am;
        row_lse[i] = lse;
        row_entropy[i] = h;
    }
    return bad;
}

/* Soft embedding of rows of `logits` over the slice [s, e).
 * The table is given either as fp32 (w_f32) or as bf16 bit patterns (w_bf16);
 * exactly one must be non-NULL.  Row r of the table is vocab id s + r.
 * out is [n_rows, ld_out] doubles.  Returns 0 on success. */
int oracle_soft_embed(const float* logits, int64_t ld, int64_t n_rows, int64_t vocab,
                      int64_t s, int64_t e,
                      const float* w_f32, const uint16_t* w_bf16, int64_t ld_w, int64_t d,
                      double gamma, int round_p_bf16, double* out, int64_t ld_out)
{
    if ((w_f32 == NULL) == (w_bf16 == NULL)) return 2;
    if (s < 0 || e < s || e > vocab) return 3;
    int bad = 0;
#pragma omp parallel reduction(|| : bad)
    {
        double* acc = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            const float* x = logits + i * ld;
            double m = (double)x[0];
            for (int64_t v = 0; v < vocab; ++v) {
                if (!isfinite(x[v])) bad = 1;
                if ((double)x[v] > m) m = (double)x[v];
            }
            double z = 0.0;
            for (int64_t v = 0; v < vocab; ++v) z += exp((double)x[v] - m);
            double lse = m + log(z);
            for (int64_t j = 0; j < d; ++j) acc[j] = 0.0;
            for (int64_t v = s; v < e; ++v) {
                double p = exp((double)x[v] - lse);
                if (round_p_bf16) p = oracle_round_bf16(p);
                int64_t r = v - s;
                if (w_f32) {
                    const float* wr = w_f32 + r * ld_w;
                    for (int64_t j = 0; j < d; ++j) acc[j] += p * (double)wr[j];
                } else {
                    const uint16_t* wr = w_bf16 + r * ld_w;
                    for (int64_t j = 0; j < d; ++j) acc[j] += p * bf16_bits_value(wr[j]);
                }
            }
            for (int64_t j = 0; j < d; ++j) out[i * ld_out + j] = gamma * acc[j];
        }
        free(acc);
    }
    return bad;
}

/* Soft embedding of rows of `logits` over the slice [s, e), computed range by range as
 * the one-read step forms it (each range's probabilities taken against the range's own
 * maximum, the ranges rescaled to the full row's log-sum-exp; calvarado04.com, "The
 * fix": the product split over disjoint vocabulary pieces and summed):
 *
 *   lse        = log-sum-exp of the FULL row
 *   m_r        = max of l over range r = [bounds[r], bounds[r+1])
 *   q_v        = exp(l_v - m_r)            (rounded to bf16 if round_q_bf16)
 *   out_i,:    = gamma * sum_r exp(m_r - lse) * sum_{v in range r} q_v W[v - s, :]
 *
 * bounds holds n_ranges + 1 increasing vocab ids with bounds[0] = s and
 * bounds[n_ranges] = e.  Without rounding this is oracle_soft_embed's result up to the
 * order of fp64 roundings.  With rounding it is a diagnostic of a kernel that rounds
 * e^(l - m_r) to bf16 before an fp32 contraction.  Returns 0 on success. */
int oracle_soft_embed_ranges(const float* logits, int64_t ld, int64_t n_rows, int64_t vocab,
                             int64_t s, int64_t e, const int64_t* bounds, int64_t n_ranges,
                             const float* w_f32, const uint16_t* w_bf16, int64_t ld_w,
                             int64_t d, double gamma, int round_q_bf16, double* out,
                             int64_t ld_out)
{
    if ((w_f32 == NULL) == (w_bf16 == NULL)) return 2;
    if (s < 0 || e < s || e > vocab || n_ranges < 1) return 3;
    if (bounds[0] != s || bounds[n_ranges] != e) return 4;
    for (int64_t r = 0; r < n_ranges; ++r)
        if (bounds[r + 1] <= bounds[r]) return 4;
    int bad = 0;
#pragma omp parallel reduction(|| : bad)
    {
        double* acc = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
        double* tot = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            const float* x = logits + i * ld;
            double m = (double)x[0];
            for (int64_t v = 0; v < vocab; ++v) {
                if (!isfinite(x[v])) bad = 1;
                if ((double)x[v] > m) m = (double)x[v];
            }
            double z = 0.0;
            for (int64_t v = 0; v < vocab; ++v) z += exp((double)x[v] - m);
            double lse = m + log(z);
            for (int64_t j = 0; j < d; ++j) tot[j] = 0.0;
            for (int64_t r = 0; r < n_ranges; ++r) {
                double mr = (double)x[bounds[r]];
                for (int64_t v = bounds[r]; v < bounds[r + 1]; ++v)
                    if ((double)x[v] > mr) mr = (double)x[v];
                for (int64_t j = 0; j < d; ++j) acc[j] = 0.0;
                for (int64_t v = bounds[r]; v < bounds[r + 1]; ++v) {
                    double q = exp((double)x[v] - mr);
                    if (round_q_bf16) q = oracle_round_bf16(q);
                    int64_t k = v - s;
                    if (w_f32) {
                        const float* wr = w_f32 + k * ld_w;
                        for (int64_t j = 0; j < d; ++j) acc[j] += q * (double)wr[j];
                    } else {
                        const uint16_t* wr = w_bf16 + k * ld_w;
                        for (int64_t j = 0; j < d; ++j) acc[j] += q * bf16_bits_value(wr[j]);
                    }
                }
                double f = exp(mr - lse);
                for (int64_t j = 0; j < d; ++j) tot[j] += f * acc[j];
            }
            for (int64_t j = 0; j < d; ++j) out[i * ld_out + j] = gamma * tot[j];
        }
        free(acc);
        free(tot);
    }
    return bad;
}
