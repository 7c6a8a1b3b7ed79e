/*
 * abi_from_c.c -- the C ABI used from plain C, with no Python and no torch: host pack, device
 * buffers and a stream from the HIP runtime, the GPU entry points, and the results checked
 * bit for bit.  Inputs are small integers times power-of-two scales, so every partial sum is
 * exactly representable in float32 and each output has one correct value, computed here on the
 * host in double precision.  Built by __graft_entry__.build() with gcc against include/bonsai.h
 * and libbonsai.so; run by tests/test_gpu_parity.py.  Exit status 0 and "all checks passed" on
 * success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bonsai.h"

static int failures = 0;
#define CHECK(cond)                                                                  \
    do {                                                                             \
        if (!(cond)) {                                                               \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                              \
        }                                                                            \
    } while (0)
#define HIP_OK(expr)                                                        \
    do {                                                                    \
        hipError_t e_ = (expr);                                             \
        if (e_ != hipSuccess) {                                             \
            fprintf(stderr, "%s failed: %s\n", #expr, hipGetErrorString(e_)); \
            exit(2);                                                        \
        }                                                                   \
    } while (0)

static uint64_t rng_state = 0x853C49E6748FEA9Bull;
static uint32_t next_u32(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 16);
}

/* small integers and powers of two as binary16 bit patterns */
static uint16_t f16_int(int v)
{
    if (v == 0) return 0;
    const int a = v < 0 ? -v : v;
    int e = 0;
    while ((a >> e) > 1) ++e;                       /* a = 1.f * 2^e, a < 2048 */
    const uint16_t frac = (uint16_t)(((a << 10) >> e) & 0x3FF);
    return (uint16_t)((v < 0 ? 0x8000u : 0u) | (uint16_t)((e + 15) << 10) | frac);
}
static uint16_t f16_pow2(int e) { return (uint16_t)((e + 15) << 10); }

static void *dev_copy(const void *h, size_t bytes)
{
    void *d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 16));
    if (bytes) HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    return d;
}

/* y[m][n] = sum_k w[n][k] s[n][k/128] x[m][k], double (exact here) */
static void host_ref(const int8_t *w, const double *s, const double *x, int M, int N, int K, double *y)
{
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) acc += w[(size_t)n * K + k] * s[(size_t)n * (K / 128) + k / 128] * x[(size_t)m * K + k];
            y[(size_t)m * N + n] = acc;
        }
}

/* run entry point fn on (words, scales, x) and compare with the reference, bitwise */
typedef bonsai_status (*matmul_fn)(const uint32_t *, const uint16_t *, const uint16_t *, float *, int64_t, int64_t,
                                   int64_t, void *);

static void check_result(const char *what, const float *dy, const double *ref, int M, int N, hipStream_t st)
{
    float *y = malloc(sizeof(float) * (size_t)M * N);
    HIP_OK(hipStreamSynchronize(st));
    HIP_OK(hipMemcpy(y, dy, sizeof(float) * (size_t)M * N, hipMemcpyDeviceToHost));
    int bad = 0;
    for (int i = 0; i < M * N; ++i)
        if (y[i] != (float)ref[i]) ++bad;
    if (bad) fprintf(stderr, "%s: %d of %d outputs differ\n", what, bad, M * N);
    CHECK(bad == 0);
    free(y);
}

int main(void)
{
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    const int N = 1000, K = 1152, G = K / 128, MMAX = 200;

    /* weights: signs and trits, with one power-of-two scale per group */
    int8_t *signs = malloc((size_t)N * K), *trits = malloc((size_t)N * K);
    uint16_t *sc = malloc(sizeof(uint16_t) * (size_t)N * G);
    double *scd = malloc(sizeof(double) * (size_t)N * G);
    for (size_t i = 0; i < (size_t)N * K; ++i) {
        signs[i] = (next_u32() & 1) ? 1 : -1;
        trits[i] = (int8_t)((int)(next_u32() % 3) - 1);
    }
    for (size_t i = 0; i < (size_t)N * G; ++i) {
        const int e = (int)(next_u32() % 5) - 2;     /* 2^-2 .. 2^2 */
        sc[i] = f16_pow2(e);
        scd[i] = ldexp(1.0, e);
    }
    uint16_t *xh = malloc(sizeof(uint16_t) * (size_t)MMAX * K);
    double *xd = malloc(sizeof(double) * (size_t)MMAX * K);
    for (size_t i = 0; i < (size_t)MMAX * K; ++i) {
        const int v = (int)(next_u32() % 17) - 8;
        xh[i] = f16_int(v);
        xd[i] = v;
    }

    /* the host entry points pack the layouts */
    uint32_t *wbits = malloc(sizeof(uint32_t) * (size_t)N * (K / 32));
    uint32_t *wcodes = malloc(sizeof(uint32_t) * (size_t)N * (K / 16));
    const size_t t5_bytes = (size_t)N * 32 * ((K + 159) / 160);
    uint8_t *t5 = malloc(t5_bytes);
    CHECK(bonsai_q1_pack(signs, N, K, wbits) == BONSAI_OK);
    CHECK(bonsai_q2t_pack(trits, N, K, wcodes) == BONSAI_OK);
    CHECK(bonsai_t5_pack(trits, N, K, t5) == BONSAI_OK);
    uint16_t *ma = malloc(sizeof(uint16_t) * (size_t)N * G), *mb = malloc(sizeof(uint16_t) * (size_t)N * G);
    CHECK(bonsai_q1_to_affine(sc, (int64_t)N * G, ma, mb) == BONSAI_OK);

    uint32_t *d_wbits = dev_copy(wbits, sizeof(uint32_t) * (size_t)N * (K / 32));
    uint32_t *d_wcodes = dev_copy(wcodes, sizeof(uint32_t) * (size_t)N * (K / 16));
    uint8_t *d_t5 = dev_copy(t5, t5_bytes);
    uint16_t *d_sc = dev_copy(sc, sizeof(uint16_t) * (size_t)N * G);
    uint16_t *d_ma = dev_copy(ma, sizeof(uint16_t) * (size_t)N * G);
    uint16_t *d_mb = dev_copy(mb, sizeof(uint16_t) * (size_t)N * G);
    uint16_t *d_x = dev_copy(xh, sizeof(uint16_t) * (size_t)MMAX * K);
    float *d_y = NULL;
    HIP_OK(hipMalloc((void **)&d_y, sizeof(float) * (size_t)MMAX * N));
    double *ref_b = malloc(sizeof(double) * (size_t)MMAX * N), *ref_t = malloc(sizeof(double) * (size_t)MMAX * N);
    host_ref(signs, scd, xd, MMAX, N, K, ref_b);
    host_ref(trits, scd, xd, MMAX, N, K, ref_t);

    /* binary: the table GEMV (M = 1), the matrix-core GEMV (M = 5), the tile GEMM (M = 200) */
    CHECK(bonsai_q1_gemv(d_wbits, d_sc, d_x, d_y, 1, N, K, st) == BONSAI_OK);
    check_result("q1_gemv M=1", d_y, ref_b, 1, N, st);
    CHECK(bonsai_q1_gemv(d_wbits, d_sc, d_x, d_y, 5, N, K, st) == BONSAI_OK);
    check_result("q1_gemv M=5", d_y, ref_b, 5, N, st);
    CHECK(bonsai_q1_gemm(d_wbits, d_sc, d_x, d_y, MMAX, N, K, st) == BONSAI_OK);
    check_result("q1_gemm M=200", d_y, ref_b, MMAX, N, st);
    /* the same weights in MLX's affine form */
    CHECK(bonsai_q1a_matmul(d_wbits, d_ma, d_mb, d_x, d_y, 3, N, K, st) == BONSAI_OK);
    check_result("q1a_matmul M=3", d_y, ref_b, 3, N, st);
    /* ternary on the 2-bit codes and on the base-3 layout */
    CHECK(bonsai_q2t_gemv(d_wcodes, d_sc, d_x, d_y, 4, N, K, st) == BONSAI_OK);
    check_result("q2t_gemv M=4", d_y, ref_t, 4, N, st);
    CHECK(bonsai_q2t_gemm(d_wcodes, d_sc, d_x, d_y, MMAX, N, K, st) == BONSAI_OK);
    check_result("q2t_gemm M=200", d_y, ref_t, MMAX, N, st);
    CHECK(bonsai_t5_matmul(d_t5, d_sc, d_x, d_y, 2, N, K, st) == BONSAI_OK);
    check_result("t5_matmul M=2", d_y, ref_t, 2, N, st);

    /* refused calls return a status and enqueue nothing */
    CHECK(bonsai_q1_gemv(d_wbits, d_sc, d_x, d_y, 1, N, 100, st) == BONSAI_ERR_SHAPE);
    CHECK(bonsai_q1_gemv(d_wbits, d_sc, d_x, d_y, 9, N, K, st) == BONSAI_ERR_SHAPE);
    CHECK(bonsai_q1_gemv(NULL, d_sc, d_x, d_y, 1, N, K, st) == BONSAI_ERR_NULL);
    CHECK(bonsai_q1_gemv(d_wbits, d_sc, (const uint16_t *)((const char *)d_x + 2), d_y, 1, N, K, st) == BONSAI_ERR_ALIGN);
    CHECK(strlen(bonsai_status_str(BONSAI_ERR_SHAPE)) > 0);
    HIP_OK(hipStreamSynchronize(st));

    hipFree(d_wbits); hipFree(d_wcodes); hipFree(d_t5); hipFree(d_sc); hipFree(d_ma); hipFree(d_mb);
    hipFree(d_x); hipFree(d_y);
    HIP_OK(hipStreamDestroy(st));
    free(signs); free(trits); free(sc); free(scd); free(xh); free(xd); free(wbits); free(wcodes); free(t5);
    free(ma); free(mb); free(ref_b); free(ref_t);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("abi_from_c: all checks passed\n");
    return 0;
}
