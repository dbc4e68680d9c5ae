/*
 * The C part of the CPU oracle (oracle/nvfp4_ref.c) under the address and
 * undefined-behaviour sanitizers: built with gcc by
 * tests/test_host_sanitized.py.  Every buffer is allocated at exactly the
 * size the shape needs, so a read past any row, scale block or batch is
 * reported.  The hand-derived single-block examples of the GEMV pin the
 * values (tests/golden/hand_examples.txt carries their derivations).
 *
 * Prints "oracle_check ok" and exits 0, or names the failed check and exits 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_gemv_sums(const uint8_t *A, const uint8_t *sfA, const uint8_t *x, const uint8_t *sfx,
                      int64_t l, int64_t m, int64_t k, double *S, int nthreads);
double oracle_e4m3(unsigned code);
double oracle_e2m1(unsigned code);

static int failures = 0;
#define CHECK(cond)                                                               \
    do {                                                                          \
        if (!(cond)) {                                                            \
            printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);              \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static uint8_t *filled(size_t n, uint8_t v)
{
    uint8_t *p = malloc(n);
    memset(p, v, n);
    return p;
}

/* One 16-element block, l = m = 1: S for A bytes a, scale sa, x bytes xb, scale sx. */
static double one_block(uint8_t a, uint8_t sa, uint8_t xb, uint8_t sx)
{
    uint8_t *A = filled(8, a), *SA = filled(1, sa), *X = filled(8, xb), *SX = filled(1, sx);
    double S = -1.0;
    oracle_gemv_sums(A, SA, X, SX, 1, 1, 16, &S, 1);
    free(A);
    free(SA);
    free(X);
    free(SX);
    return S;
}

int main(void)
{
    /* H1: A byte 0x21 holds codes 1 (0.5) and 2 (1.0), x byte 0x3C codes 12 (-2)
       and 3 (1.5); sfA 0x38 = 1, sfx 0x40 = 2: 8 * (0.5*-2 + 1*1.5) * 2 = 8 */
    CHECK(one_block(0x21, 0x38, 0x3C, 0x40) == 8.0);
    /* H2: subnormal scales 2^-9 both: 8 * (6*6 + 6*6) * 2^-18 */
    CHECK(one_block(0x77, 0x01, 0x77, 0x01) == ldexp(576.0, -18));
    /* H8: codes 15 (-6) against 7 (6) */
    CHECK(one_block(0xFF, 0x38, 0x77, 0x38) == -576.0);
    /* H9: a zero scale gives +0 */
    double z = one_block(0x77, 0x00, 0x77, 0x7E);
    CHECK(z == 0.0 && !signbit(z));
    /* NaN scale propagates */
    CHECK(isnan(one_block(0x11, 0x7F, 0x11, 0x38)));

    /* every E4M3 code decodes to a finite value or NaN (0x7F, 0xFF), and the
       E2M1 table is odd in the sign bit */
    for (unsigned b = 0; b < 256; ++b) {
        double v = oracle_e4m3(b);
        CHECK((b & 0x7F) == 0x7F ? isnan(v) : fabs(v) <= 448.0);
    }
    for (unsigned c = 0; c < 8; ++c) CHECK(oracle_e2m1(c) == -oracle_e2m1(c + 8));

    /* a ragged multi-batch shape with exact-size buffers: l=3, m=5, k=48,
       every block scale 1.0 and every x code 1 (0.5): S is half the sum of the
       row's A values */
    {
        const int64_t l = 3, m = 5, k = 48;
        uint8_t *A = malloc(l * m * k / 2), *SA = filled(l * m * k / 16, 0x38);
        uint8_t *X = filled(l * k / 2, 0x11), *SX = filled(l * k / 16, 0x38);
        double *S = malloc(sizeof(double) * l * m);
        for (int64_t i = 0; i < l * m * k / 2; ++i) A[i] = (uint8_t)(i * 37 + 11);
        oracle_gemv_sums(A, SA, X, SX, l, m, k, S, 2);
        for (int64_t r = 0; r < l * m; ++r) {
            double want = 0.0;
            for (int64_t j = 0; j < k / 2; ++j) {
                uint8_t byte = A[r * (k / 2) + j];
                want += 0.5 * (oracle_e2m1(byte & 15u) + oracle_e2m1(byte >> 4));
            }
            CHECK(S[r] == want);
        }
        free(A);
        free(SA);
        free(X);
        free(SX);
        free(S);
    }
    if (failures) {
        printf("oracle_check: %d failed checks\n", failures);
        return 1;
    }
    printf("oracle_check ok\n");
    return 0;
}
