// capi.hip -- the C ABI of libbonsai: host-side validation, launches, and the host
// pack/unpack functions that make the storage layout executable.  Declarations and the
// normative layout are in include/bonsai.h.
#include <limits.h>

#include <hip/hip_ext.h>

#include "../../include/bonsai.h"
#include "launch.h"

namespace bonsai {
namespace {

__global__ void fill_zero_kernel(float *y, int64_t count)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) y[i] = 0.f;
}

thread_local const char *g_last_device_error = "none";
thread_local hipEvent_t g_time_start = nullptr, g_time_stop = nullptr;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared argument checks of the GPU entry points.  max_m < 0: no upper bound on M.
bonsai_status check_gpu_args(const void *w, const void *s, const void *x, const float *y,
                             int64_t M, int64_t N, int64_t K, int64_t max_m)
{
    if (M < 0 || N < 0 || K < 0 || (max_m >= 0 && M > max_m)) return BONSAI_ERR_SHAPE;
    if (K % 128 != 0 || K > BONSAI_MAX_K || N > (1 << 30) || M > (1 << 30)) return BONSAI_ERR_SHAPE;
    if (M == 0 || N == 0) return BONSAI_OK;
    if (!y) return BONSAI_ERR_NULL;
    if (K == 0) return aligned16(y) ? BONSAI_OK : BONSAI_ERR_ALIGN;
    if (!w || !s || !x) return BONSAI_ERR_NULL;
    if (!aligned16(w) || !aligned16(s) || !aligned16(x) || !aligned16(y)) return BONSAI_ERR_ALIGN;
    return BONSAI_OK;
}

// 2 s in binary16, exactly (an exponent step, or a shift of a subnormal's fraction, which
// carries into the exponent by itself); false when 2 s is not finite or s is inf / NaN
bool f16_twice(uint16_t s, uint16_t *out)
{
    const uint16_t sign = s & 0x8000u, mag = s & 0x7FFFu;
    const unsigned e = mag >> 10;
    if (e >= 30) return false;
    *out = (uint16_t)(sign | (e == 0 ? mag << 1 : mag + 0x400u));
    return true;
}

// A refused launch: keep its name for bonsai_last_device_error and clear the runtime's
// last-error state, so that the caller's next, unrelated HIP call does not report it again.
bonsai_status device_status(hipError_t e)
{
    if (e == hipSuccess) return BONSAI_OK;
    g_last_device_error = hipGetErrorName(e);
    (void)hipGetLastError();
    return BONSAI_ERR_DEVICE;
}

template <typename Launch>
bonsai_status run(const void *w, const void *s, const void *x, float *y, int64_t M, int64_t N,
                  int64_t K, int64_t max_m, void *stream, Launch launch)
{
    const bonsai_status st = check_gpu_args(w, s, x, y, M, N, K, max_m);
    if (st != BONSAI_OK || M == 0 || N == 0) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const hipError_t e = K == 0 ? launch_fill_zero(y, M * N, hs)
                                : launch((int)M, (int)N, (int)K, hs);
    return device_status(e);
}

}  // namespace

hipError_t launch_kernel(const void *fn, dim3 grid, dim3 block, void **args, size_t lds, hipStream_t stream)
{
    hipEvent_t start = g_time_start, stop = g_time_stop;
    g_time_start = g_time_stop = nullptr;
    if (!start && !stop) return hipLaunchKernel(fn, grid, block, args, lds, stream);
    return hipExtLaunchKernel(fn, grid, block, args, lds, stream, start, stop, 0);
}

hipError_t launch_fill_zero(float *y, int64_t count, hipStream_t stream)
{
    const int64_t blocks = (count + 255) / 256;
    void *args[] = {&y, &count};
    return launch_kernel(reinterpret_cast<const void *>(&fill_zero_kernel),
                           dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), args, 0, stream);
}

}  // namespace bonsai

using namespace bonsai;

extern "C" {

bonsai_status bonsai_q1_gemv(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x,
                             float *y, int64_t M, int64_t N, int64_t K, void *hip_stream)
{
    return run(wbits, scales, x, y, M, N, K, BONSAI_GEMV_MAX_M, hip_stream,
               [&](int m, int n, int k, hipStream_t st) { return launch_q1_gemv(wbits, scales, x, y, m, n, k, st); });
}

bonsai_status bonsai_q1_gemm(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x,
                             float *y, int64_t M, int64_t N, int64_t K, void *hip_stream)
{
    return run(wbits, scales, x, y, M, N, K, -1, hip_stream,
               [&](int m, int n, int k, hipStream_t st) { return launch_q1_gemm(wbits, scales, x, y, m, n, k, st); });
}

bonsai_status bonsai_q2t_gemv(const uint32_t *wcodes, const uint16_t *scales, const uint16_t *x,
                              float *y, int64_t M, int64_t N, int64_t K, void *hip_stream)
{
    return run(wcodes, scales, x, y, M, N, K, BONSAI_GEMV_MAX_M, hip_stream,
               [&](int m, int n, int k, hipStream_t st) { return launch_q2t_gemv(wcodes, scales, x, y, m, n, k, st); });
}

bonsai_status bonsai_q2t_gemm(const uint32_t *wcodes, const uint16_t *scales, const uint16_t *x,
                              float *y, int64_t M, int64_t N, int64_t K, void *hip_stream)
{
    return run(wcodes, scales, x, y, M, N, K, -1, hip_stream,
               [&](int m, int n, int k, hipStream_t st) { return launch_q2t_gemm(wcodes, scales, x, y, m, n, k, st); });
}

bonsai_status bonsai_q1a_matmul(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases,
                                const uint16_t *x, float *y, int64_t M, int64_t N, int64_t K, void *hip_stream)
{
    if (M > 0 && N > 0 && K > 0 && K % 128 == 0 && K <= BONSAI_MAX_K && N <= (1 << 30) && M <= (1 << 30)) {
        if (!biases) return BONSAI_ERR_NULL;
        if (!aligned16(biases)) return BONSAI_ERR_ALIGN;
    }
    return run(wbits, scales, x, y, M, N, K, -1, hip_stream, [&](int m, int n, int k, hipStream_t st) {
        return launch_q1a_matmul(wbits, scales, biases, x, y, m, n, k, st);
    });
}

bonsai_status bonsai_t5_matmul(const uint8_t *codes, const uint16_t *scales, const uint16_t *x,
                               float *y, int64_t M, int64_t N, int64_t K, void *hip_stream)
{
    return run(codes, scales, x, y, M, N, K, -1, hip_stream,
               [&](int m, int n, int k, hipStream_t st) { return launch_t5_matmul(codes, scales, x, y, m, n, k, st); });
}

bonsai_status bonsai_t5_pack(const int8_t *trits, int64_t N, int64_t K, uint8_t *codes)
{
    if (N < 0 || K < 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!trits || !codes) return BONSAI_ERR_NULL;
    const int64_t sb = (K + 159) / 160;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < sb; ++b)
            for (int c = 0; c < 32; ++c) {
                unsigned v = 0, place = 1;
                for (int i = 0; i < 5; ++i, place *= 3) {
                    const int64_t k = 160 * b + c + 32 * i;
                    if (k >= K) continue;
                    const int8_t t = trits[n * K + k];
                    if (t < -1 || t > 1) return BONSAI_ERR_VALUE;
                    v += (unsigned)(t < 0 ? 2 : t) * place;
                }
                codes[n * 32 * sb + 32 * b + c] = (uint8_t)v;
            }
    return BONSAI_OK;
}

bonsai_status bonsai_t5_unpack(const uint8_t *codes, int64_t N, int64_t K, int8_t *trits)
{
    if (N < 0 || K < 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!trits || !codes) return BONSAI_ERR_NULL;
    const int64_t sb = (K + 159) / 160;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < sb; ++b)
            for (int c = 0; c < 32; ++c) {
                unsigned v = codes[n * 32 * sb + 32 * b + c];
                if (v >= 243) return BONSAI_ERR_CODE;
                for (int i = 0; i < 5; ++i, v /= 3) {
                    const int64_t k = 160 * b + c + 32 * i;
                    const int d = (int)(v % 3);
                    if (k >= K) {
                        if (d != 0) return BONSAI_ERR_CODE;      // padding must hold zero weights
                        continue;
                    }
                    trits[n * K + k] = (int8_t)(d == 2 ? -1 : d);
                }
            }
    return BONSAI_OK;
}

bonsai_status bonsai_q2t_to_t5(const uint32_t *wcodes, int64_t N, int64_t K, uint8_t *codes)
{
    if (N < 0 || K < 0 || K % 16 != 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!wcodes || !codes) return BONSAI_ERR_NULL;
    const int64_t sb = (K + 159) / 160;
    for (int64_t n = 0; n < N; ++n) {
        const uint32_t *row = wcodes + n * (K / 16);
        for (int64_t b = 0; b < sb; ++b)
            for (int c = 0; c < 32; ++c) {
                unsigned v = 0, place = 1;
                for (int i = 0; i < 5; ++i, place *= 3) {
                    const int64_t k = 160 * b + c + 32 * i;
                    if (k >= K) continue;
                    const unsigned f = (row[k / 16] >> (2 * (k % 16))) & 3u;
                    if (f == 2) return BONSAI_ERR_CODE;
                    v += (f == 0 ? 0u : f == 1 ? 1u : 2u) * place;   // digit = w mod 3
                }
                codes[n * 32 * sb + 32 * b + c] = (uint8_t)v;
            }
    }
    return BONSAI_OK;
}

bonsai_status bonsai_t5_to_q2t(const uint8_t *codes, int64_t N, int64_t K, uint32_t *wcodes)
{
    if (N < 0 || K < 0 || K % 16 != 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!wcodes || !codes) return BONSAI_ERR_NULL;
    const int64_t sb = (K + 159) / 160;
    for (int64_t n = 0; n < N; ++n) {
        uint32_t *row = wcodes + n * (K / 16);
        for (int64_t w = 0; w < K / 16; ++w) row[w] = 0;
        for (int64_t b = 0; b < sb; ++b)
            for (int c = 0; c < 32; ++c) {
                unsigned v = codes[n * 32 * sb + 32 * b + c];
                if (v >= 243) return BONSAI_ERR_CODE;
                for (int i = 0; i < 5; ++i, v /= 3) {
                    const int64_t k = 160 * b + c + 32 * i;
                    const unsigned d = v % 3;
                    if (k >= K) {
                        if (d != 0) return BONSAI_ERR_CODE;      // padding must hold zero weights
                        continue;
                    }
                    row[k / 16] |= (d == 0 ? 0u : d == 1 ? 1u : 3u) << (2 * (k % 16));
                }
            }
    }
    return BONSAI_OK;
}

bonsai_status bonsai_q1_to_affine(const uint16_t *scales, int64_t n_groups, uint16_t *mlx_scales,
                                  uint16_t *mlx_biases)
{
    if (n_groups < 0) return BONSAI_ERR_SHAPE;
    if (n_groups == 0) return BONSAI_OK;
    if (!scales || !mlx_scales || !mlx_biases) return BONSAI_ERR_NULL;
    for (int64_t g = 0; g < n_groups; ++g) {
        if (!f16_twice(scales[g], &mlx_scales[g])) return BONSAI_ERR_VALUE;
        mlx_biases[g] = (uint16_t)(scales[g] ^ 0x8000u);
    }
    return BONSAI_OK;
}

bonsai_status bonsai_q1_from_affine(const uint16_t *mlx_scales, const uint16_t *mlx_biases, int64_t n_groups,
                                    uint16_t *scales)
{
    if (n_groups < 0) return BONSAI_ERR_SHAPE;
    if (n_groups == 0) return BONSAI_OK;
    if (!scales || !mlx_scales || !mlx_biases) return BONSAI_ERR_NULL;
    for (int64_t g = 0; g < n_groups; ++g) {
        const uint16_t s = (uint16_t)(mlx_biases[g] ^ 0x8000u);
        uint16_t twice;
        if (!f16_twice(s, &twice) || twice != mlx_scales[g]) return BONSAI_ERR_VALUE;
        scales[g] = s;
    }
    return BONSAI_OK;
}

bonsai_status bonsai_q1_embed(const uint32_t *wbits, const uint16_t *scales, const int64_t *ids,
                              uint16_t *out, int64_t n_ids, int64_t V, int64_t K, void *hip_stream)
{
    if (n_ids < 0 || V < 0 || K < 0 || K % 128 != 0 || K > BONSAI_MAX_K || n_ids > (1 << 30) || V > (1 << 30))
        return BONSAI_ERR_SHAPE;
    if (n_ids == 0 || K == 0) return BONSAI_OK;
    if (!ids || !out || (V > 0 && (!wbits || !scales))) return BONSAI_ERR_NULL;
    if (!aligned16(ids) || !aligned16(out) || (V > 0 && (!aligned16(wbits) || !aligned16(scales))))
        return BONSAI_ERR_ALIGN;
    return device_status(launch_q1_embed(wbits, scales, ids, out, n_ids, V, (int)K, static_cast<hipStream_t>(hip_stream)));
}

bonsai_status bonsai_q1_pack(const int8_t *signs, int64_t N, int64_t K, uint32_t *wbits)
{
    if (N < 0 || K < 0 || K % 32 != 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!signs || !wbits) return BONSAI_ERR_NULL;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t w = 0; w < K / 32; ++w) {
            uint32_t word = 0;
            for (int j = 0; j < 32; ++j) {
                const int8_t v = signs[n * K + 32 * w + j];
                if (v != 1 && v != -1) return BONSAI_ERR_VALUE;
                word |= (uint32_t)(v > 0) << j;
            }
            wbits[n * (K / 32) + w] = word;
        }
    return BONSAI_OK;
}

bonsai_status bonsai_q1_unpack(const uint32_t *wbits, int64_t N, int64_t K, int8_t *signs)
{
    if (N < 0 || K < 0 || K % 32 != 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!signs || !wbits) return BONSAI_ERR_NULL;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            signs[n * K + k] = ((wbits[n * (K / 32) + k / 32] >> (k % 32)) & 1u) ? 1 : -1;
    return BONSAI_OK;
}

bonsai_status bonsai_q2t_pack(const int8_t *trits, int64_t N, int64_t K, uint32_t *wcodes)
{
    if (N < 0 || K < 0 || K % 16 != 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!trits || !wcodes) return BONSAI_ERR_NULL;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t w = 0; w < K / 16; ++w) {
            uint32_t word = 0;
            for (int j = 0; j < 16; ++j) {
                const int8_t v = trits[n * K + 16 * w + j];
                uint32_t code;
                if (v == 0) code = 0u;
                else if (v == 1) code = 1u;
                else if (v == -1) code = 3u;
                else return BONSAI_ERR_VALUE;
                word |= code << (2 * j);
            }
            wcodes[n * (K / 16) + w] = word;
        }
    return BONSAI_OK;
}

bonsai_status bonsai_q2t_unpack(const uint32_t *wcodes, int64_t N, int64_t K, int8_t *trits)
{
    if (N < 0 || K < 0 || K % 16 != 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!trits || !wcodes) return BONSAI_ERR_NULL;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const uint32_t code = (wcodes[n * (K / 16) + k / 16] >> (2 * (k % 16))) & 3u;
            if (code == 2u) return BONSAI_ERR_CODE;
            trits[n * K + k] = code == 0u ? 0 : (code == 1u ? 1 : -1);
        }
    return BONSAI_OK;
}

const char *bonsai_last_device_error(void) { return g_last_device_error; }

bonsai_status bonsai_time_next_launch(void *start_event, void *stop_event)
{
    g_time_start = static_cast<hipEvent_t>(start_event);
    g_time_stop = static_cast<hipEvent_t>(stop_event);
    return BONSAI_OK;
}

const char *bonsai_status_str(bonsai_status s)
{
    switch (s) {
    case BONSAI_OK: return "ok";
    case BONSAI_ERR_NULL: return "a required pointer is NULL";
    case BONSAI_ERR_SHAPE: return "M, N or K out of range, or K not a multiple of 128";
    case BONSAI_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case BONSAI_ERR_VALUE: return "input outside the weight alphabet, or not an exact binary-weight scale/bias pair";
    case BONSAI_ERR_CODE: return "reserved ternary code (2-bit field 0b10, base-3 byte above 242 or nonzero padding)";
    case BONSAI_ERR_DEVICE: return "HIP launch failed";
    }
    return "unknown status";
}

}  // extern "C"
