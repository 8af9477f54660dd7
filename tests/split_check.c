/*
 * Property check of a three-piece BF16 split over a range of FP32 bit
 * patterns (test code: used by the split sweeps in tests/, shares no code
 * with the oracle or the HIP library; it only reads the pieces it is given).
 *
 * The split is the one of "Unlocking Tensor Core Performance for Machine
 * Learning Interatomic Potentials", section "How Tensor Core FP32 bridges
 * the hardware gap", Figure 1 (three scaled BF16 pieces per FP32 value), read
 * as hi = R(a), mid' = R(2^8 (a - hi)), lo' = 2^8 (2^8 (a - hi) - mid') with R
 * round to nearest even, saturating.  What the mathematics fixes, checked
 * here for the pieces of the value with bit pattern (first + i) mod 2^32:
 *
 *   finite a:  a == hi + 2^-8 mid' + 2^-16 lo' exactly (checked as
 *              (a - hi) - 2^-8 mid' == 2^-16 lo' in double, each subtraction
 *              required to be exact by an error-free TwoSum), every piece
 *              finite, and, below the saturated corner
 *              |a| >= 0x7F7F8000, each piece at most half a BF16 spacing of
 *              the one before: |2^-8 mid'| <= ulp(hi)/2, |2^-16 lo'| <=
 *              ulp(2^-8 mid')/2 (ulp = BF16 spacing at that magnitude,
 *              2^-133 below the normal range);
 *   +-inf:     hi = 0x7F80 | sign, mid' = lo' = 0;
 *   NaN:       hi = 0x7FC0 | sign, mid' = lo' = 0.
 *
 * Built with gcc -O2 -fopenmp -ffp-contract=off (tests/split_check.py).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static double bf16_to_double(uint16_t h)
{
    const uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* BF16 spacing at magnitude |v| (v a double). */
static double bf16_ulp(double v)
{
    v = fabs(v);
    if (v < ldexp(1.0, -126)) return ldexp(1.0, -133);
    int e;
    frexp(v, &e);               /* v = f 2^e, f in [0.5, 1) */
    return ldexp(1.0, e - 1 - 7);
}

static int piece_finite(uint16_t h) { return (h & 0x7F80u) != 0x7F80u; }

/* *out = x - y rounded to double; returns 1 iff that is exact (Knuth's
 * TwoSum error term is zero). */
static int exact_diff(double x, double y, double* out)
{
    const double ny = -y;
    const double s = x + ny;
    const double bb = s - x;
    const double err = (x - (s - bb)) + (ny - bb);
    *out = s;
    return err == 0.0;
}

static int check_one(uint32_t bits, uint16_t hi, uint16_t mid, uint16_t lo)
{
    const uint32_t mag = bits & 0x7FFFFFFFu;
    const uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (mag == 0x7F800000u) return hi == (sign | 0x7F80u) && mid == 0 && lo == 0;
    if (mag > 0x7F800000u) return hi == (sign | 0x7FC0u) && mid == 0 && lo == 0;
    if (!piece_finite(hi) || !piece_finite(mid) || !piece_finite(lo)) return 0;
    float a;
    memcpy(&a, &bits, 4);
    const double h = bf16_to_double(hi);
    const double m = ldexp(bf16_to_double(mid), -8);
    const double l = ldexp(bf16_to_double(lo), -16);
    double d1, d2;
    if (!exact_diff((double)a, h, &d1) || !exact_diff(d1, m, &d2) || d2 != l) return 0;
    if (mag < 0x7F7F8000u) {
        if (fabs(m) > 0.5 * bf16_ulp(h)) return 0;
        if (fabs(l) > 0.5 * bf16_ulp(m)) return 0;
    }
    return 1;
}

/* Number of patterns (first + i) mod 2^32, i < n, whose pieces fail the
 * checks; *first_bad = the smallest failing i, or -1. */
int64_t split_check_range(uint64_t first, int64_t n, const uint16_t* hi, const uint16_t* mid,
                          const uint16_t* lo, int64_t* first_bad)
{
    int64_t bad = 0, first_i = INT64_MAX;
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : first_i)
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t bits = (uint32_t)((first + (uint64_t)i) & 0xFFFFFFFFu);
        if (!check_one(bits, hi[i], mid[i], lo[i])) {
            ++bad;
            if (i < first_i) first_i = i;
        }
    }
    *first_bad = bad ? first_i : -1;
    return bad;
}
