/*
 * Cross-entropy oracle: plain, slow, obviously correct CPU code in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg use it.  It shares no code, header, table
 * or constant with the HIP library.
 *
 * What it computes (KernelIndex, "Cross-entropy loss", description and
 * Semantics block; "Vocab-parallel cross-entropy, Megatron layout",
 * description and Semantics block): for every token row i of a
 * tokens x vocab logit matrix z and an integer target t_i in [0, vocab),
 *
 *     loss_i = ln( sum_j exp(z_ij) ) - z_{i, t_i}          (natural log)
 *
 * and, for the scalar output of the first page, the mean of loss_i over all
 * tokens.  The pages never print the formula; this is the textbook softmax
 * cross-entropy, the plainest reading of "cross-entropy loss over
 * tokens x vocab logits against integer targets".
 *
 * Evaluation: every logit is decoded exactly to double, then two plain passes
 * over the row: m = max_j z_ij, s = sum_j exp(z_ij - m) (sequential fp64 sum),
 * loss = m + log(s) - z_t.  Subtracting m changes nothing mathematically; it
 * only keeps exp() in range.  A target outside [0, vocab) is a contract
 * violation and yields NaN for that row.
 *
 * Rows are independent, so OpenMP spreads them over host threads; the order
 * of the arithmetic inside a row is fixed and sequential.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

/* bf16 is the upper half of an IEEE binary32 pattern: widen by a 16-bit shift. */
static double bf16_bits_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double logit_at(const void* base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F32) {
        float f;
        memcpy(&f, (const char*)base + 4 * idx, 4);
        return (double)f;
    }
    if (dtype == ORACLE_BF16) {
        uint16_t h;
        memcpy(&h, (const char*)base + 2 * idx, 2);
        return bf16_bits_to_double(h);
    }
    double d;
    memcpy(&d, (const char*)base + 8 * idx, 8);
    return d;
}

/* Decode one row of `vocab` logits to double. */
static void decode_row(const void* logits, int dtype, int64_t row, int64_t vocab,
                       double* dst)
{
    const int64_t base = row * vocab;
    for (int64_t j = 0; j < vocab; ++j)
        dst[j] = logit_at(logits, dtype, base + j);
}

/* Per-token losses for `rows` rows.  Returns 0, or -1 on a bad argument. */
int oracle_xent_rows(const void* logits, int dtype, int64_t rows, int64_t vocab,
                     const int64_t* target, double* loss, int nthreads)
{
    if (rows < 0 || vocab < 1 || (rows > 0 && (!logits || !target || !loss)))
        return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64)
        return -1;
    if (nthreads < 1)
        nthreads = 1;

#pragma omp parallel num_threads(nthreads)
    {
        double* z = (double*)malloc((size_t)vocab * sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < rows; ++i) {
            const int64_t t = target[i];
            if (t < 0 || t >= vocab || !z) {
                loss[i] = NAN;
                continue;
            }
            decode_row(logits, dtype, i, vocab, z);

            double m = -INFINITY; /* pass 1: row maximum */
            for (int64_t j = 0; j < vocab; ++j)
                if (z[j] > m)
                    m = z[j];

            double s = 0.0; /* pass 2: sum of exp(z - m), in index order */
            for (int64_t j = 0; j < vocab; ++j)
                s += exp(z[j] - m);

            loss[i] = m + log(s) - z[t];
        }
        free(z);
    }
    return 0;
}

/*
 * Shard statistics for the vocab-parallel layout (KernelIndex "Vocab-parallel
 * cross-entropy, Megatron layout", description: the vocab axis is split across
 * devices; the page itself measures one device).  `logits` holds, for every
 * row, the `shard` consecutive vocab columns [v0, v0 + shard) of the full
 * vocab.  For each row i, written to out[3i .. 3i+2]:
 *
 *     m_i  = max_j z_ij
 *     s_i  = sum_j exp(z_ij - m_i)          (so ln sum_j exp(z_ij) = m_i + ln s_i)
 *     zt_i = z_{i, t_i - v0}  if v0 <= t_i < v0 + shard, else NaN (not this shard's)
 *
 * A shard row of -inf only has sum_j exp(z_ij) = 0, written as (-inf, 0).
 *
 * Same two plain passes as oracle_xent_rows.  Returns 0, or -1 on a bad argument.
 */
int oracle_xent_partial(const void* logits, int dtype, int64_t rows, int64_t shard, int64_t v0,
                        const int64_t* target, double* out, int nthreads)
{
    if (rows < 0 || shard < 1 || v0 < 0 || (rows > 0 && (!logits || !target || !out)))
        return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64)
        return -1;
    if (nthreads < 1)
        nthreads = 1;

#pragma omp parallel num_threads(nthreads)
    {
        double* z = (double*)malloc((size_t)shard * sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < rows; ++i) {
            if (!z) {
                out[3 * i] = out[3 * i + 1] = out[3 * i + 2] = NAN;
                continue;
            }
            decode_row(logits, dtype, i, shard, z);
            double m = -INFINITY;
            for (int64_t j = 0; j < shard; ++j)
                if (z[j] > m)
                    m = z[j];
            double s = 0.0;
            if (m != -INFINITY)
                for (int64_t j = 0; j < shard; ++j)
                    s += exp(z[j] - m);
            const int64_t t = target[i];
            out[3 * i] = m;
            out[3 * i + 1] = s;
            out[3 * i + 2] = (t >= v0 && t < v0 + shard) ? z[t - v0] : NAN;
        }
        free(z);
    }
    return 0;
}

/*
 * Loss of each row from the statistics of the `shards` vocab shards that
 * together cover the row (partials[p][i][0..2] = (m, s, zt) as above, shards
 * in vocab order):
 *
 *     ln sum_j exp(z_ij) = M + ln( sum_p s_pi * exp(m_pi - M) ),  M = max_p m_pi
 *     loss_i = that - zt_i
 *
 * where zt_i is the target logit reported by the one shard that holds the
 * target.  NaN if t_i is outside [0, vocab) or no shard reports it.
 */
int oracle_xent_merge(const double* partials, int64_t shards, int64_t rows,
                      const int64_t* target, int64_t vocab, double* loss)
{
    if (shards < 1 || rows < 0 || vocab < 1 || (rows > 0 && (!partials || !target || !loss)))
        return -1;
    for (int64_t i = 0; i < rows; ++i) {
        double M = -INFINITY;
        for (int64_t p = 0; p < shards; ++p) {
            const double m = partials[3 * (p * rows + i)];
            if (m > M)
                M = m;
        }
        double s = 0.0, zt = NAN;
        for (int64_t p = 0; p < shards; ++p) {
            const double* q = partials + 3 * (p * rows + i);
            if (q[0] != -INFINITY) /* a shard of -inf only adds nothing */
                s += q[1] * exp(q[0] - M);
            if (!isnan(q[2]))
                zt = q[2];
        }
        const int64_t t = target[i];
        loss[i] = (t < 0 || t >= vocab) ? NAN : M + log(s) - zt;
    }
    return 0;
}

/*
 * Gradient of the loss with respect to the logits.  The pages give only the
 * forward; this is the derivative of the loss above, written out:
 *
 *     d loss_i / d z_ij = e^(z_ij - lse_i) - [j == t_i],   lse_i = ln sum_k e^(z_ik)
 *
 * scaled by the gradient flowing into the loss output: g_i = grad[i] for the
 * per-token losses (mean == 0), g_i = grad[0] / rows for their mean (mean != 0).
 * A row with a target outside [0, vocab) has a NaN loss; its gradient row is NaN.
 * lse_i comes from the same two plain passes as oracle_xent_rows.
 * dlogits is [rows, vocab] doubles.  Returns 0, or -1 on a bad argument.
 */
int oracle_xent_bwd_rows(const void* logits, int dtype, int64_t rows, int64_t vocab,
                         const int64_t* target, int mean, const double* grad, double* dlogits,
                         int nthreads)
{
    if (rows < 0 || vocab < 1 || (rows > 0 && (!logits || !target || !grad || !dlogits)))
        return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64)
        return -1;
    if (nthreads < 1)
        nthreads = 1;

#pragma omp parallel num_threads(nthreads)
    {
        double* z = (double*)malloc((size_t)vocab * sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < rows; ++i) {
            double* dz = dlogits + i * vocab;
            const int64_t t = target[i];
            if (t < 0 || t >= vocab || !z) {
                for (int64_t j = 0; j < vocab; ++j)
                    dz[j] = NAN;
                continue;
            }
            decode_row(logits, dtype, i, vocab, z);
            double m = -INFINITY;
            for (int64_t j = 0; j < vocab; ++j)
                if (z[j] > m)
                    m = z[j];
            double s = 0.0;
            for (int64_t j = 0; j < vocab; ++j)
                s += exp(z[j] - m);
            const double lse = m + log(s);
            const double g = mean ? grad[0] / (double)rows : grad[i];
            for (int64_t j = 0; j < vocab; ++j)
                dz[j] = g * (exp(z[j] - lse) - (j == t ? 1.0 : 0.0));
        }
        free(z);
    }
    return 0;
}

/* Mean of n per-token losses, summed in index order.  n == 0 gives 0/0 = NaN. */
double oracle_mean(const double* loss, int64_t n)
{
    double acc = 0.0;
    for (int64_t i = 0; i < n; ++i)
        acc += loss[i];
    return acc / (double)n;
}

/* Number of threads OpenMP would use by default (for reporting). */
int oracle_default_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
