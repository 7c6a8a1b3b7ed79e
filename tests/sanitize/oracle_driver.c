/*
 * oracle_driver.c -- drives every entry point of the C oracle (oracle/bonsai_oracle.c) on small
 * inputs held in heap buffers of exactly the documented sizes: dense dequantisation of row
 * ranges, the matmul of all four weight forms over index subsets and in full, the exact
 * fixed-point sums, and every error path (shape, reserved code, non-finite input).  Built with
 * -fsanitize=address,undefined by tests/test_sanitizers.py, so an access past a buffer or an
 * undefined operation anywhere in the oracle is reported.  The oracle has no header (Python
 * loads it through ctypes); its prototypes are restated here.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define BO_OK 0
#define BO_ERR_SHAPE 2
#define BO_ERR_CODE 5
#define BO_ERR_NONFINITE 7

double bo_f16_to_f64(uint16_t h);
int bo_q1_dequant(const uint32_t *, const uint16_t *, int64_t, int64_t, int64_t, int64_t, double *);
int bo_q1a_dequant(const uint32_t *, const uint16_t *, const uint16_t *, int64_t, int64_t, int64_t, int64_t,
                   double *);
int bo_q2t_dequant(const uint32_t *, const uint16_t *, int64_t, int64_t, int64_t, int64_t, double *);
int bo_t5_dequant(const uint8_t *, const uint16_t *, int64_t, int64_t, int64_t, int64_t, double *);
int bo_q1_matmul(const uint32_t *, const uint16_t *, const uint16_t *, int64_t, int64_t, int64_t,
                 const int64_t *, int64_t, const int64_t *, int64_t, double *, double *);
int bo_q1a_matmul(const uint32_t *, const uint16_t *, const uint16_t *, const uint16_t *, int64_t, int64_t,
                  int64_t, const int64_t *, int64_t, const int64_t *, int64_t, double *, double *);
int bo_q2t_matmul(const uint32_t *, const uint16_t *, const uint16_t *, int64_t, int64_t, int64_t,
                  const int64_t *, int64_t, const int64_t *, int64_t, double *, double *);
int bo_t5_matmul(const uint8_t *, const uint16_t *, const uint16_t *, int64_t, int64_t, int64_t,
                 const int64_t *, int64_t, const int64_t *, int64_t, double *, double *);
int bo_q1_exact(const uint32_t *, const uint16_t *, const uint16_t *, int64_t, int64_t, int64_t,
                const int64_t *, int64_t, const int64_t *, int64_t, double *);
int bo_q2t_exact(const uint32_t *, const uint16_t *, const uint16_t *, int64_t, int64_t, int64_t,
                 const int64_t *, int64_t, const int64_t *, int64_t, double *);

static int failures = 0;
#define CHECK(cond)                                                                  \
    do {                                                                             \
        if (!(cond)) {                                                               \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                              \
        }                                                                            \
    } while (0)

static uint64_t rng_state = 0x2545F4914F6CDD1Dull;
static uint32_t next_u32(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 16);
}

static void *xalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

/* small integers as binary16: |v| <= 4, so every product and sum below is exact in double */
static uint16_t small_f16(int v)
{
    static const uint16_t mag[5] = {0x0000, 0x3C00, 0x4000, 0x4200, 0x4400};   /* 0, 1, 2, 3, 4 */
    return (uint16_t)((v < 0 ? 0x8000u : 0u) | mag[v < 0 ? -v : v]);
}

static void f16_decoder(void)
{
    CHECK(bo_f16_to_f64(0x0000) == 0.0 && !signbit(bo_f16_to_f64(0x0000)));
    CHECK(bo_f16_to_f64(0x8000) == 0.0 && signbit(bo_f16_to_f64(0x8000)));
    CHECK(bo_f16_to_f64(0x0001) == ldexp(1.0, -24));
    CHECK(bo_f16_to_f64(0x3C00) == 1.0);
    CHECK(bo_f16_to_f64(0x7BFF) == 65504.0);
    CHECK(isinf(bo_f16_to_f64(0x7C00)) && isnan(bo_f16_to_f64(0x7E00)));
}

/* y over index subsets equals the full product at those entries, and the dense sum of the
 * dequantised row with x, for one weight form */
typedef int (*dequant_fn)(const void *, const uint16_t *, const uint16_t *, int64_t, int64_t, int64_t, int64_t,
                          double *);

static int dq_q1(const void *w, const uint16_t *s, const uint16_t *b, int64_t N, int64_t K, int64_t n0, int64_t n1,
                 double *W)
{
    (void)b;
    return bo_q1_dequant((const uint32_t *)w, s, N, K, n0, n1, W);
}
static int dq_q1a(const void *w, const uint16_t *s, const uint16_t *b, int64_t N, int64_t K, int64_t n0,
                  int64_t n1, double *W)
{
    return bo_q1a_dequant((const uint32_t *)w, s, b, N, K, n0, n1, W);
}
static int dq_q2t(const void *w, const uint16_t *s, const uint16_t *b, int64_t N, int64_t K, int64_t n0,
                  int64_t n1, double *W)
{
    (void)b;
    return bo_q2t_dequant((const uint32_t *)w, s, N, K, n0, n1, W);
}
static int dq_t5(const void *w, const uint16_t *s, const uint16_t *b, int64_t N, int64_t K, int64_t n0, int64_t n1,
                 double *W)
{
    (void)b;
    return bo_t5_dequant((const uint8_t *)w, s, N, K, n0, n1, W);
}

static int mm(int form, const void *w, const uint16_t *s, const uint16_t *b, const uint16_t *x, int64_t M,
              int64_t N, int64_t K, const int64_t *mi, int64_t mc, const int64_t *ni, int64_t nc, double *y,
              double *a)
{
    switch (form) {
    case 0: return bo_q1_matmul((const uint32_t *)w, s, x, M, N, K, mi, mc, ni, nc, y, a);
    case 1: return bo_q2t_matmul((const uint32_t *)w, s, x, M, N, K, mi, mc, ni, nc, y, a);
    case 2: return bo_q1a_matmul((const uint32_t *)w, s, b, x, M, N, K, mi, mc, ni, nc, y, a);
    default: return bo_t5_matmul((const uint8_t *)w, s, x, M, N, K, mi, mc, ni, nc, y, a);
    }
}

static void one_form(int form, const void *w, const uint16_t *s, const uint16_t *b, const uint16_t *x, int64_t M,
                     int64_t N, int64_t K)
{
    static const dequant_fn dq[4] = {dq_q1, dq_q2t, dq_q1a, dq_t5};
    double *W = xalloc(sizeof(double) * (size_t)(N * K));
    double *y = xalloc(sizeof(double) * (size_t)(M * N)), *a = xalloc(sizeof(double) * (size_t)(M * N));
    CHECK(dq[form](w, s, b, N, K, 0, N, W) == BO_OK);
    CHECK(mm(form, w, s, b, x, M, N, K, NULL, 0, NULL, 0, y, a) == BO_OK);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = W[n * K + k] * bo_f16_to_f64(x[m * K + k]);
                acc += p;
                mag += fabs(p);
            }
            CHECK(y[m * N + n] == acc && a[m * N + n] == mag);
        }
    /* a row range of the dequantisation matches the full one */
    double *part = xalloc(sizeof(double) * (size_t)K);
    CHECK(dq[form](w, s, b, N, K, N - 1, N, part) == BO_OK);
    CHECK(memcmp(part, W + (N - 1) * K, sizeof(double) * (size_t)K) == 0);
    /* index subsets (repeated and out of order), without the magnitude output */
    const int64_t mi[3] = {M - 1, 0, M - 1}, ni[2] = {N - 1, 0};
    double ys[6];
    CHECK(mm(form, w, s, b, x, M, N, K, mi, 3, ni, 2, ys, NULL) == BO_OK);
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 2; ++j) CHECK(ys[i * 2 + j] == y[mi[i] * N + ni[j]]);
    /* errors: an index past the shape, a row range past N, K not a multiple of 128 */
    const int64_t bad_n[1] = {N};
    CHECK(mm(form, w, s, b, x, M, N, K, NULL, 0, bad_n, 1, ys, NULL) == BO_ERR_SHAPE);
    CHECK(dq[form](w, s, b, N, K, 0, N + 1, W) == BO_ERR_SHAPE);
    CHECK(mm(form, w, s, b, x, M, N, K - 64, NULL, 0, NULL, 0, y, a) == BO_ERR_SHAPE);
    /* empty products */
    CHECK(mm(form, w, s, b, x, 0, N, K, NULL, 0, NULL, 0, y, a) == BO_OK);
    free(W);
    free(y);
    free(a);
    free(part);
}

int main(void)
{
    f16_decoder();
    const int64_t M = 3, N = 5, K = 384, G = K / 128;
    uint32_t *sign = xalloc(sizeof(uint32_t) * (size_t)(N * K / 32));
    uint32_t *tern = xalloc(sizeof(uint32_t) * (size_t)(N * K / 16));
    const int64_t t5_row = 32 * ((K + 159) / 160);
    uint8_t *t5 = xalloc((size_t)(N * t5_row));
    uint16_t *s = xalloc(sizeof(uint16_t) * (size_t)(N * G)), *b = xalloc(sizeof(uint16_t) * (size_t)(N * G));
    uint16_t *x = xalloc(sizeof(uint16_t) * (size_t)(M * K));
    for (int64_t i = 0; i < N * K / 32; ++i) sign[i] = next_u32();
    for (int64_t i = 0; i < N * K / 16; ++i) {
        uint32_t wd = 0;
        for (int j = 0; j < 16; ++j) {
            const uint32_t c = next_u32() % 3;
            wd |= (c == 2 ? 3u : c) << (2 * j);
        }
        tern[i] = wd;
    }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t c = 0; c < t5_row; ++c) {
            /* zero digits for the weights past K, any digits below it */
            const int64_t blk = c / 32, byte = c % 32;
            unsigned v = 0, place = 1;
            for (int i = 0; i < 5; ++i, place *= 3)
                if (160 * blk + byte + 32 * i < K) v += (next_u32() % 3) * place;
            t5[n * t5_row + c] = (uint8_t)v;
        }
    for (int64_t i = 0; i < N * G; ++i) {
        s[i] = small_f16(1 + (int)(next_u32() % 4));
        b[i] = small_f16(-(int)(next_u32() % 3));
    }
    for (int64_t i = 0; i < M * K; ++i) x[i] = small_f16((int)(next_u32() % 9) - 4);

    for (int form = 0; form < 4; ++form) {
        const void *w = form == 0 || form == 2 ? (const void *)sign : form == 1 ? (const void *)tern : (const void *)t5;
        one_form(form, w, s, b, x, M, N, K);
    }

    /* the exact sums agree with the double ones on small integers (every partial sum is exact) */
    double *y = xalloc(sizeof(double) * (size_t)(M * N)), *ye = xalloc(sizeof(double) * (size_t)(M * N));
    CHECK(bo_q1_matmul(sign, s, x, M, N, K, NULL, 0, NULL, 0, y, NULL) == BO_OK);
    CHECK(bo_q1_exact(sign, s, x, M, N, K, NULL, 0, NULL, 0, ye) == BO_OK);
    CHECK(memcmp(y, ye, sizeof(double) * (size_t)(M * N)) == 0);
    CHECK(bo_q2t_matmul(tern, s, x, M, N, K, NULL, 0, NULL, 0, y, NULL) == BO_OK);
    CHECK(bo_q2t_exact(tern, s, x, M, N, K, NULL, 0, NULL, 0, ye) == BO_OK);
    CHECK(memcmp(y, ye, sizeof(double) * (size_t)(M * N)) == 0);
    const int64_t ni[1] = {N}, mi[1] = {-1};
    CHECK(bo_q1_exact(sign, s, x, M, N, K, NULL, 0, ni, 1, ye) == BO_ERR_SHAPE);
    CHECK(bo_q2t_exact(tern, s, x, M, N, K, mi, 1, NULL, 0, ye) == BO_ERR_SHAPE);

    /* reserved codes and non-finite inputs */
    double *W = xalloc(sizeof(double) * (size_t)(N * K));
    const uint32_t keep = tern[2];
    tern[2] = (tern[2] & ~(3u << 6)) | (2u << 6);            /* field 3 of word 2 = 0b10 */
    CHECK(bo_q2t_dequant(tern, s, N, K, 0, N, W) == BO_ERR_CODE);
    CHECK(bo_q2t_exact(tern, s, x, M, N, K, NULL, 0, NULL, 0, ye) == BO_ERR_CODE);
    tern[2] = keep;
    const uint8_t keep5 = t5[7];
    t5[7] = 250;
    CHECK(bo_t5_dequant(t5, s, N, K, 0, N, W) == BO_ERR_CODE);
    CHECK(bo_t5_matmul(t5, s, x, M, N, K, NULL, 0, NULL, 0, y, NULL) == BO_ERR_CODE);
    t5[7] = keep5;
    x[5] = 0x7C00;                                            /* +inf */
    CHECK(bo_q1_exact(sign, s, x, M, N, K, NULL, 0, NULL, 0, ye) == BO_ERR_NONFINITE);
    CHECK(bo_q1_matmul(sign, s, x, M, N, K, NULL, 0, NULL, 0, y, NULL) == BO_OK && isinf(y[0]));

    free(W);
    free(y);
    free(ye);
    free(sign);
    free(tern);
    free(t5);
    free(s);
    free(b);
    free(x);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
