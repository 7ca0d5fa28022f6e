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
