// capi.hip -- the C ABI of libbonsai, GPU side: argument validation and launches.  The
// host-only entry points (pack / unpack and the layout conversions) are in host.cpp.
// Declarations and the normative layout are in include/bonsai.h.
#include <limits.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <utility>

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
// The measurement hook as armed by bonsai_time_next_launch, and as taken by the entry point
// being served (g_call_*): every GPU entry point takes and clears the armed hook on entry, so
// that a call returning early (an argument error, an empty shape) consumes it too.
thread_local hipEvent_t g_time_start = nullptr, g_time_stop = nullptr;
thread_local hipEvent_t g_call_start = nullptr, g_call_stop = nullptr;

// A launch plan in progress on this thread (bonsai_plan): the planned compute-unit count, and
// where the launch goes instead of the device.
struct Plan {
    int cus;
    bool device;        // planning for the current device: its kernels' registers are looked up
    char *buf;
    int64_t len;
    int launches;
};
thread_local Plan *g_plan = nullptr;

// Takes the armed hook for the call now being served (the outermost scope of an entry point
// does; scopes nested inside it leave the taken hook alone).
thread_local bool g_in_call = false;
struct HookScope {
    const bool outer;
    HookScope() : outer(!g_in_call)
    {
        if (!outer) return;
        g_in_call = true;
        g_call_start = g_time_start;
        g_call_stop = g_time_stop;
        g_time_start = g_time_stop = nullptr;
    }
    ~HookScope()
    {
        if (!outer) return;
        g_in_call = false;
        g_call_start = g_call_stop = nullptr;
    }
};

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
    HookScope hook;
    const bonsai_status st = check_gpu_args(w, s, x, y, M, N, K, max_m);
    if (st != BONSAI_OK || M == 0 || N == 0) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const hipError_t e = K == 0 ? launch_fill_zero(y, M * N, hs)
                                : launch((int)M, (int)N, (int)K, hs);
    return device_status(e);
}

// Per-device lookups: compute units, the LDS limit set on a kernel, a kernel's registers.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];
std::mutex g_fn_mutex;
std::map<std::pair<int, const void *>, int> g_fn_lds, g_fn_vgprs;

int current_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    return dev;
}

}  // namespace

int device_cus()
{
    if (g_plan) return g_plan->cus;
    const int dev = current_device();
    if (dev >= kMaxDevices) {
        int n = 0;
        return hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
    }
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    g_cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

bool set_lds_limit(const void *fn, int bytes)
{
    if (g_plan) return true;            // nothing is launched
    const auto key = std::make_pair(current_device(), fn);
    std::lock_guard<std::mutex> lock(g_fn_mutex);
    auto it = g_fn_lds.find(key);
    if (it != g_fn_lds.end() && it->second >= bytes) return true;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess) return false;
    g_fn_lds[key] = bytes;
    return true;
}

int func_vgprs(const void *fn)
{
    if (g_plan && !g_plan->device) return 0;
    const auto key = std::make_pair(current_device(), fn);
    std::lock_guard<std::mutex> lock(g_fn_mutex);
    auto it = g_fn_vgprs.find(key);
    if (it != g_fn_vgprs.end()) return it->second;
    hipFuncAttributes a;
    const int regs = hipFuncGetAttributes(&a, fn) == hipSuccess && a.numRegs > 0 ? a.numRegs : 0;
    g_fn_vgprs[key] = regs;
    return regs;
}

hipError_t launch_kernel(const void *fn, const char *name, dim3 grid, dim3 block, void **args, size_t lds,
                         hipStream_t stream)
{
    if (g_plan) {
        if (g_plan->launches++ == 0 && g_plan->buf && g_plan->len > 0) {
            // a launcher's signature "R ns::f(args) [T = v, ...]" is written as "f[T = v, ...]"
            const char *open = strchr(name, '(');
            while (open && strncmp(open, "(anonymous namespace)", 21) == 0) open = strchr(open + 21, '(');
            const char *start = name;
            if (open) {
                for (const char *c = name; c < open; ++c)
                    if (*c == ':' || *c == ' ') start = c + 1;
            }
            const int base = open ? (int)(open - start) : (int)strlen(name);
            const char *targs = open ? strstr(open, " [") : nullptr;
            snprintf(g_plan->buf, (size_t)g_plan->len, "%.*s%s grid=%u,%u block=%u lds=%zu%s", base, start,
                     targs ? targs + 1 : "", grid.x, grid.y, block.x, lds,
                     g_call_start || g_call_stop ? " timed" : "");
        }
        g_call_start = g_call_stop = nullptr;       // the hook is consumed, as by a launch
        return hipSuccess;
    }
    hipEvent_t start = g_call_start, stop = g_call_stop;
    g_call_start = g_call_stop = nullptr;
    if (!start && !stop) return hipLaunchKernel(fn, grid, block, args, lds, stream);
    return hipExtLaunchKernel(fn, grid, block, args, lds, stream, start, stop, 0);
}

hipError_t launch_fill_zero(float *y, int64_t count, hipStream_t stream)
{
    const int64_t blocks = (count + 255) / 256;
    void *args[] = {&y, &count};
    return launch_kernel(reinterpret_cast<const void *>(&fill_zero_kernel), "fill_zero_kernel",
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
    HookScope hook;
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
    HookScope hook;
    if (n_ids < 0 || V < 0 || K < 0 || K % 128 != 0 || K > BONSAI_MAX_K || n_ids > (1 << 30) || V > (1 << 30))
        return BONSAI_ERR_SHAPE;
    if (n_ids == 0 || K == 0) return BONSAI_OK;
    if (!ids || !out || (V > 0 && (!wbits || !scales))) return BONSAI_ERR_NULL;
    if (!aligned16(ids) || !aligned16(out) || (V > 0 && (!aligned16(wbits) || !aligned16(scales))))
        return BONSAI_ERR_ALIGN;
    return device_status(launch_q1_embed(wbits, scales, ids, out, n_ids, V, (int)K, static_cast<hipStream_t>(hip_stream)));
}

bonsai_status bonsai_probe_stream(void *buf, int64_t bytes, int mode, uint32_t *sink, void *hip_stream)
{
    HookScope hook;
    if (mode < 0 || mode > 2 || bytes <= 0 || bytes % 1024 != 0 || bytes > ((int64_t)1 << 40)) return BONSAI_ERR_SHAPE;
    if (!buf || !sink) return BONSAI_ERR_NULL;
    if (!aligned16(buf) || !aligned16(sink)) return BONSAI_ERR_ALIGN;
    return device_status(launch_probe_stream(buf, bytes, mode, sink, static_cast<hipStream_t>(hip_stream)));
}

bonsai_status bonsai_probe_clock(uint64_t *stamps, int64_t spin_ns, void *hip_stream)
{
    HookScope hook;
    if (spin_ns < 0 || spin_ns > 1000000000) return BONSAI_ERR_SHAPE;
    if (!stamps) return BONSAI_ERR_NULL;
    if (!aligned16(stamps)) return BONSAI_ERR_ALIGN;
    return device_status(launch_probe_clock(stamps, spin_ns, static_cast<hipStream_t>(hip_stream)));
}

bonsai_status bonsai_plan(int op, int64_t M, int64_t N, int64_t K, int cus, char *buf, int64_t len)
{
    if (buf && len > 0) buf[0] = '\0';
    if (op < 0 || op > 6) return BONSAI_ERR_VALUE;
    if (g_plan) return BONSAI_ERR_VALUE;
    // cus <= 0: the current device's count, looked up before the plan starts
    Plan plan{cus > 0 ? cus : device_cus(), cus <= 0, buf, len, 0};
    // stand-in device pointers: never dereferenced, nothing is launched
    const uint32_t *w = reinterpret_cast<const uint32_t *>(uintptr_t{1} << 20);
    const uint16_t *sc = reinterpret_cast<const uint16_t *>(uintptr_t{2} << 20);
    const uint16_t *bi = reinterpret_cast<const uint16_t *>(uintptr_t{3} << 20);
    const uint16_t *x = reinterpret_cast<const uint16_t *>(uintptr_t{4} << 20);
    float *y = reinterpret_cast<float *>(uintptr_t{5} << 20);
    g_plan = &plan;
    bonsai_status st = BONSAI_OK;
    switch (op) {
    case 0: st = bonsai_q1_gemv(w, sc, x, y, M, N, K, nullptr); break;
    case 1: st = bonsai_q1_gemm(w, sc, x, y, M, N, K, nullptr); break;
    case 2: st = bonsai_q2t_gemv(w, sc, x, y, M, N, K, nullptr); break;
    case 3: st = bonsai_q2t_gemm(w, sc, x, y, M, N, K, nullptr); break;
    case 4: st = bonsai_t5_matmul(reinterpret_cast<const uint8_t *>(w), sc, x, y, M, N, K, nullptr); break;
    case 5: st = bonsai_q1a_matmul(w, sc, bi, x, y, M, N, K, nullptr); break;
    default:
        st = bonsai_q1_embed(w, sc, reinterpret_cast<const int64_t *>(bi), reinterpret_cast<uint16_t *>(y), M, N, K,
                             nullptr);
        break;
    }
    g_plan = nullptr;
    if (st == BONSAI_OK && plan.launches == 0 && buf && len > 0) snprintf(buf, (size_t)len, "none");
    return st;
}

const char *bonsai_last_device_error(void) { return g_last_device_error; }

bonsai_status bonsai_time_next_launch(void *start_event, void *stop_event)
{
    g_time_start = static_cast<hipEvent_t>(start_event);
    g_time_stop = static_cast<hipEvent_t>(stop_event);
    return BONSAI_OK;
}

}  // extern "C"
