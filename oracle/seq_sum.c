/*
 * Oracle: the plain in-order fp64 loop.  TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load or run this file's library.  It shares no code, header or constant
 * with the HIP path and must never serve as a fallback for it.
 *
 * What it computes (Research-1433 "Forming the CPU's sequential double sums
 * on a GPU, bit for bit", Question; Research-1424 "integer_ssim_cuda and the
 * CPU's frame sum", Findings 1): one double accumulator, each term added in
 * index order with the IEEE-754 binary64 add, round to nearest, ties to
 * even.  The accumulator starts at `init`; the pages' extractors start at
 * +0.0 (one double through the whole frame), which is the default the
 * Python wrapper passes.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fexcess-precision=standard
 * on x86-64 (SSE2 addsd, no x87 extended precision, no reassociation).
 */
#include <stddef.h>
#include <stdint.h>

double oracle_seq_sum_f64(const double *x, size_t n, double init)
{
    double s = init;
    for (size_t i = 0; i < n; i++)
        s += x[i];
    return s;
}

/* `count` independent loops; sum k covers x[offsets[k] .. offsets[k] + ns[k]).
 * Each is the same plain loop (pyramid batch: many independent running sums,
 * ADR-1391 "The CUDA ssimulacra2 twin is device-resident", Decision step 2). */
void oracle_seq_sum_f64_many(const double *x, const int64_t *offsets,
                             const int64_t *ns, int64_t count,
                             const double *inits, double *out)
{
    for (int64_t k = 0; k < count; k++)
        out[k] = oracle_seq_sum_f64(x + offsets[k], (size_t)ns[k], inits[k]);
}

/* k interleaved loops over records of k doubles, and the float mean of each
 * (ADR-1464 "float_ssim_cuda adds its frame sums in the CPU's raster order,
 * on the host", Context and Decision): one accumulator per field, started at
 * inits[j]; the records are read in index order and each field is added into
 * its own accumulator, so every accumulator sees its terms in index order;
 * the mean is the double quotient by the record count rounded to float. */
void oracle_seq_sum_f64_interleaved(const double *x, size_t windows, int64_t k,
                                    const double *inits, double *out, float *means)
{
    for (int64_t j = 0; j < k; j++)
        out[j] = inits[j];
    for (size_t w = 0; w < windows; w++)
        for (int64_t j = 0; j < k; j++)
            out[j] += x[w * (size_t)k + (size_t)j];
    for (int64_t j = 0; j < k; j++)
        means[j] = (float)(out[j] / (double)windows);
}
