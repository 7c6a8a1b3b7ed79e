// capi.hip -- the C ABI of libbonsai, GPU side: argument validation and launches.  The
// host-only entry points (pack / unpack and the layout conversions) are in host.cpp.
// Declarations and the normative layout are in include/bonsai.h.
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

const char *bonsai_last_device_error(void) { return g_last_device_error; }

bonsai_status bonsai_time_next_launch(void *start_event, void *stop_event)
{
    g_time_start = static_cast<hipEvent_t>(start_event);
    g_time_stop = static_cast<hipEvent_t>(stop_event);
    return BONSAI_OK;
}

}  // extern "C"
