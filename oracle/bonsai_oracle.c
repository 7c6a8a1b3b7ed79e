/*
 * bonsai_oracle.c -- CPU oracle for the binary / ternary g128 weight-only matmul.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark may load this library.  It shares no code, header, table or
 * helper with the GPU library; the two meet only through the seeded inputs.
 *
 * What it computes is the plain definition, evaluated densely in natural k
 * order in double precision, with no blocking, reordering or fusion:
 *
 *     y[m][n] = sum_{k=0}^{K-1} w(n,k) * x(m,k)          a[m][n] = sum_k |w(n,k) * x(m,k)|
 *
 * Binary weights ("1-bit Bonsai 27B" model card, section "Weight representation:
 * Binary g128"): each weight is one sign bit, bit 0 stands for -scale and bit 1
 * for +scale, and every 128 consecutive weights share one FP16 scale.
 *
 * Affine 1-bit weights (model card, "MLX packaging"): MLX's grouped low-bit format keeps a
 * scale a and a bias b per group of 128, and a 1-bit weight is a * q + b for its bit q; the
 * binary weights are packed there as a = 2 s, b = -s, which gives back +-s.
 *
 * Ternary weights ("Ternary Bonsai 27B" article, sections on the ternary format
 * and on its limitations): weights are {-1, 0, +1} times a per-128 FP16 scale,
 * held today in 2-bit storage.  The pages do not give the 2-bit code; the code
 * used here is 00 -> 0, 01 -> +1, 11 -> -1, with 10 reserved (rejected).
 *
 * Base-3 ternary weights (the same {-1, 0, +1} x scale, at the native density the ternary
 * article's limitations section anticipates: log2(3) bits per weight in theory).  The pages give
 * no layout; this library's is five trits per byte, described under "Storage" below.
 *
 * Storage (the pages are silent on bit order; this is the chosen layout):
 *   sign words  uint32 [N][K/32]: weight (n,k) is bit (k mod 32) of word k/32 of row n.
 *   trit words  uint32 [N][K/16]: weight (n,k) is the 2-bit field whose low bit is
 *               bit 2*(k mod 16) of word k/16 of row n.
 *   base-3      uint8 [N][32 * ceil(K/160)]: a row is a run of 32-byte superblocks of 160
 *               weights.  Byte c (0..31) of superblock b holds the five weights
 *               k = 160 b + c + 32 i, i = 0..4, as the base-3 number sum_i d_i 3^i with digit
 *               d = w mod 3 (0 -> 0, 1 -> +1, 2 -> -1).  Bytes 243..255 are reserved (rejected);
 *               weights past K are zero digits.
 *   scales      IEEE binary16 bit patterns [N][K/128]; weight (n,k) uses scale k/128.
 *   x           IEEE binary16 bit patterns [M][K].
 *
 * Every product of two binary16 values is exact in double, so the only
 * rounding is the left-to-right double sum (error at most about K * 2^-53 * a).
 * The exact_* entry points redo the sum in 128-bit integer fixed point (units
 * of 2^-48, which every binary16 x binary16 product is a whole multiple of) and
 * round once at the end; they exist to pin the double sum from outside.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define BO_OK 0
#define BO_ERR_SHAPE 2
#define BO_ERR_CODE 5
#define BO_ERR_NONFINITE 7
#define BO_ERR_NOMEM 8

/* IEEE 754 binary16 -> double, from the format's definition:
 * sign bit 15, 5-bit biased exponent (bias 15) in bits 10..14, 10-bit fraction. */
double bo_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1F;
    const int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* zero and subnormals: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static int shape_ok(int64_t M, int64_t N, int64_t K)
{
    return M >= 0 && N >= 0 && K >= 0 && K % 128 == 0;
}

/* Binary weight (n,k): sign bit 1 -> +scale, 0 -> -scale. */
static double q1_weight(const uint32_t *wbits, const uint16_t *scales, int64_t K, int64_t n, int64_t k)
{
    const uint32_t word = wbits[n * (K / 32) + k / 32];
    const unsigned bit = (word >> (k % 32)) & 1u;
    const double s = bo_f16_to_f64(scales[n * (K / 128) + k / 128]);
    return bit ? s : -s;
}

/* Affine 1-bit weight (n,k): a * q + b with q the bit and (a, b) the group's scale and bias. */
static double q1a_weight(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases, int64_t K,
                         int64_t n, int64_t k)
{
    const uint32_t word = wbits[n * (K / 32) + k / 32];
    const double q = (double)((word >> (k % 32)) & 1u);
    const int64_t g = n * (K / 128) + k / 128;
    return bo_f16_to_f64(scales[g]) * q + bo_f16_to_f64(biases[g]);
}

/* Ternary code of weight (n,k): 0 -> 0, 1 -> +1, 3 -> -1, 2 -> reserved (returns 0 on success). */
static int q2t_trit(const uint32_t *wcodes, int64_t K, int64_t n, int64_t k, int *t)
{
    const uint32_t word = wcodes[n * (K / 16) + k / 16];
    const unsigned code = (word >> (2 * (k % 16))) & 3u;
    switch (code) {
    case 0: *t = 0; return 0;
    case 1: *t = 1; return 0;
    case 3: *t = -1; return 0;
    default: return BO_ERR_CODE;
    }
}

/* Base-3 trit of weight (n,k): digit i of byte c of superblock b, where k = 160 b + 32 i + c. */
static int t5_trit(const uint8_t *codes, int64_t K, int64_t n, int64_t k, int *t)
{
    const int64_t row_bytes = 32 * ((K + 159) / 160);
    const int64_t b = k / 160, i = (k % 160) / 32, c = k % 32;
    const unsigned v = codes[n * row_bytes + 32 * b + c];
    if (v >= 243) return BO_ERR_CODE;
    unsigned place = 1;
    for (int64_t j = 0; j < i; ++j) place *= 3;
    switch ((v / place) % 3) {
    case 0: *t = 0; return 0;
    case 1: *t = 1; return 0;
    default: *t = -1; return 0;
    }
}

/* Dense dequantisation of rows [n0, n1) into W (row-major, K doubles per row). */
int bo_q1_dequant(const uint32_t *wbits, const uint16_t *scales, int64_t N, int64_t K,
                  int64_t n0, int64_t n1, double *W)
{
    if (!shape_ok(0, N, K) || n0 < 0 || n1 > N || n0 > n1) return BO_ERR_SHAPE;
    for (int64_t n = n0; n < n1; ++n)
        for (int64_t k = 0; k < K; ++k)
            W[(n - n0) * K + k] = q1_weight(wbits, scales, K, n, k);
    return BO_OK;
}

int bo_q1a_dequant(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases, int64_t N, int64_t K,
                   int64_t n0, int64_t n1, double *W)
{
    if (!shape_ok(0, N, K) || n0 < 0 || n1 > N || n0 > n1) return BO_ERR_SHAPE;
    for (int64_t n = n0; n < n1; ++n)
        for (int64_t k = 0; k < K; ++k)
            W[(n - n0) * K + k] = q1a_weight(wbits, scales, biases, K, n, k);
    return BO_OK;
}

int bo_q2t_dequant(const uint32_t *wcodes, const uint16_t *scales, int64_t N, int64_t K,
                   int64_t n0, int64_t n1, double *W)
{
    if (!shape_ok(0, N, K) || n0 < 0 || n1 > N || n0 > n1) return BO_ERR_SHAPE;
    for (int64_t n = n0; n < n1; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int t;
            if (q2t_trit(wcodes, K, n, k, &t)) return BO_ERR_CODE;
            W[(n - n0) * K + k] = (double)t * bo_f16_to_f64(scales[n * (K / 128) + k / 128]);
        }
    return BO_OK;
}

int bo_t5_dequant(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                  int64_t n0, int64_t n1, double *W)
{
    if (!shape_ok(0, N, K) || n0 < 0 || n1 > N || n0 > n1) return BO_ERR_SHAPE;
    for (int64_t n = n0; n < n1; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int t;
            if (t5_trit(codes, K, n, k, &t)) return BO_ERR_CODE;
            W[(n - n0) * K + k] = t * bo_f16_to_f64(scales[n * (K / 128) + k / 128]);
        }
    return BO_OK;
}

/* The selected (m, n) entries of y = x W^T and of a = |x| |W|^T.
 * m_idx / n_idx list the rows of x and of W to evaluate (NULL: all of them, in order);
 * y and a are [m_cnt][n_cnt] row-major. */
/* form: 0 binary, 1 ternary, 2 affine 1-bit (biases used only there), 3 base-3 ternary */
static int matmul(int form, const void *words, const uint16_t *scales, const uint16_t *biases,
                  const uint16_t *x, int64_t M, int64_t N, int64_t K,
                  const int64_t *m_idx, int64_t m_cnt, const int64_t *n_idx, int64_t n_cnt,
                  double *y, double *a)
{
    if (!shape_ok(M, N, K)) return BO_ERR_SHAPE;
    if (!m_idx) m_cnt = M;
    if (!n_idx) n_cnt = N;
    for (int64_t i = 0; i < m_cnt; ++i)
        if (m_idx && (m_idx[i] < 0 || m_idx[i] >= M)) return BO_ERR_SHAPE;
    for (int64_t j = 0; j < n_cnt; ++j)
        if (n_idx && (n_idx[j] < 0 || n_idx[j] >= N)) return BO_ERR_SHAPE;

    double *wrow = (double *)malloc((size_t)(K ? K : 1) * sizeof(double));
    if (!wrow) return BO_ERR_NOMEM;
    int rc = BO_OK;
    for (int64_t j = 0; j < n_cnt && rc == BO_OK; ++j) {
        const int64_t n = n_idx ? n_idx[j] : j;
        rc = form == 1 ? bo_q2t_dequant(words, scales, N, K, n, n + 1, wrow)
           : form == 2 ? bo_q1a_dequant(words, scales, biases, N, K, n, n + 1, wrow)
           : form == 3 ? bo_t5_dequant(words, scales, N, K, n, n + 1, wrow)
                       : bo_q1_dequant(words, scales, N, K, n, n + 1, wrow);
        for (int64_t i = 0; i < m_cnt && rc == BO_OK; ++i) {
            const int64_t m = m_idx ? m_idx[i] : i;
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = wrow[k] * bo_f16_to_f64(x[m * K + k]);
                acc += p;
                mag += fabs(p);
            }
            y[i * n_cnt + j] = acc;
            if (a) a[i * n_cnt + j] = mag;
        }
    }
    free(wrow);
    return rc;
}

int bo_q1_matmul(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x,
                 int64_t M, int64_t N, int64_t K,
                 const int64_t *m_idx, int64_t m_cnt, const int64_t *n_idx, int64_t n_cnt,
                 double *y, double *a)
{
    return matmul(0, wbits, scales, NULL, x, M, N, K, m_idx, m_cnt, n_idx, n_cnt, y, a);
}

int bo_q1a_matmul(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases, const uint16_t *x,
                  int64_t M, int64_t N, int64_t K,
                  const int64_t *m_idx, int64_t m_cnt, const int64_t *n_idx, int64_t n_cnt,
                  double *y, double *a)
{
    return matmul(2, wbits, scales, biases, x, M, N, K, m_idx, m_cnt, n_idx, n_cnt, y, a);
}

int bo_t5_matmul(const uint8_t *codes, const uint16_t *scales, const uint16_t *x,
                 int64_t M, int64_t N, int64_t K,
                 const int64_t *m_idx, int64_t m_cnt, const int64_t *n_idx, int64_t n_cnt,
                 double *y, double *a)
{
    return matmul(3, codes, scales, NULL, x, M, N, K, m_idx, m_cnt, n_idx, n_cnt, y, a);
}

int bo_q2t_matmul(const uint32_t *wcodes, const uint16_t *scales, const uint16_t *x,
                  int64_t M, int64_t N, int64_t K,
                  const int64_t *m_idx, int64_t m_cnt, const int64_t *n_idx, int64_t n_cnt,
                  double *y, double *a)
{
    return matmul(1, wcodes, scales, NULL, x, M, N, K, m_idx, m_cnt, n_idx, n_cnt, y, a);
}

/* ---- exact fixed-point cross-check ------------------------------------------------------- */

/* A finite binary16 value as integer significand F and exponent E: value = F * 2^E, E >= -24. */
static int f16_split(uint16_t h, int64_t *F, int *E)
{
    const int e = (h >> 10) & 0x1F;
    const int f = h & 0x3FF;
    if (e == 31) return BO_ERR_NONFINITE;
    if (e == 0) { *F = f; *E = -24; }
    else { *F = 1024 + f; *E = e - 25; }
    if (h & 0x8000) *F = -*F;
    return BO_OK;
}

/* y_exact[i][j] = round_to_double( sum_k t(n,k) * s(n,k/128) * x(m,k) ), computed with
 * 128-bit integers in units of 2^-48 (exact for K < 2^40).  For binary weights t = +-1. */
static int exact(int ternary, const uint32_t *words, const uint16_t *scales, const uint16_t *x,
                 int64_t M, int64_t N, int64_t K,
                 const int64_t *m_idx, int64_t m_cnt, const int64_t *n_idx, int64_t n_cnt, double *y)
{
    if (!shape_ok(M, N, K)) return BO_ERR_SHAPE;
    if (!m_idx) m_cnt = M;
    if (!n_idx) n_cnt = N;
    for (int64_t j = 0; j < n_cnt; ++j) {
        const int64_t n = n_idx ? n_idx[j] : j;
        if (n < 0 || n >= N) return BO_ERR_SHAPE;
        for (int64_t i = 0; i < m_cnt; ++i) {
            const int64_t m = m_idx ? m_idx[i] : i;
            if (m < 0 || m >= M) return BO_ERR_SHAPE;
            __int128 acc = 0;
            for (int64_t k = 0; k < K; ++k) {
                int t;
                if (ternary) {
                    if (q2t_trit(words, K, n, k, &t)) return BO_ERR_CODE;
                } else {
                    t = ((words[n * (K / 32) + k / 32] >> (k % 32)) & 1u) ? 1 : -1;
                }
                int64_t Fs, Fx; int Es, Ex;
                if (f16_split(scales[n * (K / 128) + k / 128], &Fs, &Es)) return BO_ERR_NONFINITE;
                if (f16_split(x[m * K + k], &Fx, &Ex)) return BO_ERR_NONFINITE;
                /* Es + Ex >= -48, so the product is a whole number of 2^-48 units */
                acc += (__int128)(t * Fs * Fx) * ((__int128)1 << (Es + Ex + 48));
            }
            y[i * n_cnt + j] = ldexp((double)acc, -48);   /* one rounding, to nearest */
        }
    }
    return BO_OK;
}

int bo_q1_exact(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x,
                int64_t M, int64_t N, int64_t K,
                const int64_t *m_idx, int64_t m_cnt, const int64_t *n_idx, int64_t n_cnt, double *y)
{
    return exact(0, wbits, scales, x, M, N, K, m_idx, m_cnt, n_idx, n_cnt, y);
}

int bo_q2t_exact(const uint32_t *wcodes, const uint16_t *scales, const uint16_t *x,
                 int64_t M, int64_t N, int64_t K,
                 const int64_t *m_idx, int64_t m_cnt, const int64_t *n_idx, int64_t n_cnt, double *y)
{
    return exact(1, wcodes, scales, x, M, N, K, m_idx, m_cnt, n_idx, n_cnt, y);
}
