/*
 * CPU oracle for the NVFP4 block-scaled batched GEMV.  TEST INFRASTRUCTURE
 * ONLY: nothing in the product path may link, load or call this file.
 *
 * It evaluates the definition directly, one output at a time, with no
 * blocking, vectorisation tricks or reordering:
 *
 *   S[b,r] = sum over kk = 0 .. k-1, in increasing kk, of
 *            e2m1(A[b,r,kk]) * e4m3(sfA[b,r,kk/16]) * e2m1(x[b,kk]) * e4m3(sfx[b,kk/16])
 *
 * The formula is the NVFP4 batched GEMV of "nvFP4 Batch GEMV算子系列(下)",
 * section "NVFP4 Batched GEMV 概念阐述": 16 consecutive elements along the
 * reduced dimension K share one FP8 scale, element kk belongs to block
 * floor(kk/16).  The E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} and the block
 * size 16 are the constants of the CuTeDSL bridge page (section "Constants");
 * the sign is bit 3 of a code (the quantisers on that page add 8 for negative
 * values) and the element with the even index sits in the low nibble of each
 * byte (they pack odd << 4 | even).
 *
 * Every product of two E2M1 values and two E4M3 values has at most
 * 2 + 2 + 4 + 4 = 12 significant bits, so each term is exact in double; the
 * sum is accumulated in double starting from +0.0.  The final scaling and the
 * fp32 / fp16 roundings are done by the Python wrapper (oracle/reference.py).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no -ffast-math).
 */
#include <math.h>
#include <stdint.h>

/* E2M1 magnitudes indexed by the low three bits of a code. */
static const double kE2M1Magnitude[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Value of a 4-bit E2M1 code: bit 3 is the sign, bits 2:0 index the table. */
double oracle_e2m1(unsigned code)
{
    double v = kE2M1Magnitude[code & 7u];
    return (code & 8u) ? -v : v;
}

/*
 * Value of an 8-bit E4M3 ("fn": no infinities) code, from the format's
 * definition: sign bit 7, exponent bits 6:3 with bias 7, mantissa bits 2:0.
 * Exponent field 0 is subnormal, m * 2^-9; exponent 15 with mantissa 7 is NaN
 * (there is no infinity, so 0x7E = 448 is the largest finite value).
 */
double oracle_e4m3(unsigned code)
{
    unsigned sign = (code >> 7) & 1u;
    unsigned expo = (code >> 3) & 15u;
    unsigned mant = code & 7u;
    double v;
    if (expo == 15u && mant == 7u)
        return NAN;
    if (expo == 0u)
        v = ldexp((double)mant, -9);
    else
        v = ldexp(1.0 + (double)mant / 8.0, (int)expo - 7);
    return sign ? -v : v;
}

/* Code of element kk of a packed row: even kk in bits 3:0, odd kk in 7:4. */
static unsigned nibble(const uint8_t *row, int64_t kk)
{
    uint8_t byte = row[kk >> 1];
    return (kk & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u);
}

/*
 * S has l*m doubles, S[b*m + r].  Rows are independent, so they are spread
 * over threads; each row's sum is sequential in kk.
 */
void oracle_gemv_sums(const uint8_t *A, const uint8_t *sfA,
                      const uint8_t *x, const uint8_t *sfx,
                      int64_t l, int64_t m, int64_t k,
                      double *S, int nthreads)
{
    int64_t rows = l * m;
    int64_t half = k / 2, nblk = k / 16;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        int64_t b = row / m;
        const uint8_t *a_row = A + row * half;
        const uint8_t *sa_row = sfA + row * nblk;
        const uint8_t *x_row = x + b * half;
        const uint8_t *sx_row = sfx + b * nblk;
        double sum = 0.0;
        for (int64_t kk = 0; kk < k; ++kk) {
            double a = oracle_e2m1(nibble(a_row, kk)) * oracle_e4m3(sa_row[kk >> 4]);
            double v = oracle_e2m1(nibble(x_row, kk)) * oracle_e4m3(sx_row[kk >> 4]);
            sum += a * v;
        }
        S[row] = sum;
    }
}
