/*
 * oracle_reduce.c -- plain CPU reference for the sum of a float array.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle_sgemm.c): shares nothing with the HIP
 * path and is never called by the product library.
 *
 * What is computed: s = sum_{i=0}^{n-1} x_i (page "GPU 访存与计算优化"
 * (aerisun.top), section "Reduce 的分层归约"), together with
 * a = sum_i |x_i|, the size of the terms, which callers use to state an error
 * bound (the same page notes that the order of float additions changes the
 * last bits, so GPU results are compared with a tolerance).
 *
 * How: each x_i is widened to double and added in ascending i into a double
 * accumulator -- the definition written out, nothing else.
 */
#include <math.h>
#include <stdint.h>

int oracle_sum(int64_t n, const float *x, double *sum, double *abs_sum)
{
    if (n < 0 || !sum) return -1;
    double s = 0.0, a = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double v = (double)x[i];
        s += v;
        a += fabs(v);
    }
    *sum = s;
    if (abs_sum) *abs_sum = a;
    return 0;
}
