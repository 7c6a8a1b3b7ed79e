// probe.hip -- measurement probes: what the machine's HBM delivers to a plain stream, and the
// shader clock.  Decode is the bandwidth-bound phase ("1-bit Bonsai 27B" model card,
// cross-platform throughput), so the decode kernels are judged against the read rate a kernel
// that does nothing but read reaches on the same chip, through the same two load paths the
// kernels use: 16-byte vector loads into registers, and direct global->LDS copies.
#include "device.h"
#include "launch.h"

namespace bonsai {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glb_void_t;

constexpr int kProbeThreads = 512;      // 8 waves per workgroup, one workgroup per CU
constexpr int kProbeUnroll = 8;         // 16-byte loads in flight per lane (vector loads)
constexpr int kProbeRing = 4;           // 1 KB copies per wave in its LDS ring (3 in flight)

// Each wave folds what it read into one word (so no load is dead) and stores it: one store
// per wave.  Lane l of wave w reads the 16-byte cells l + 64 (w + W j), j = 0, 1, ... of the
// buffer, kProbeUnroll of them in flight (non-temporal: the data is used once).
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4 *__restrict__ p, int64_t n16,
                                                                   uint32_t *__restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride * kProbeUnroll) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int64_t j = i + u * stride;
            v[u] = j < n16 ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) sink[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = acc;
}

// The same bytes by direct global->LDS copies: wave w copies the 1 KB chunks w, w + W, ... into
// a ring of kProbeRing slots of its own, kProbeRing - 1 copies in flight; a chunk's slot is
// reused once the copy kProbeRing - 1 behind it has landed.  At the end each wave folds the
// last chunk it holds into its word.
__global__ __launch_bounds__(kProbeThreads) void probe_lds_kernel(const u32x4 *__restrict__ p, int64_t n16,
                                                                  uint32_t *__restrict__ sink)
{
    extern __shared__ u32x4 lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    char *const ring = reinterpret_cast<char *>(lds) + wave * kProbeRing * 1024;
    const int64_t waves = (int64_t)gridDim.x * nw;
    const int64_t chunks = n16 / 64;
    int k = 0;
    for (int64_t c = (int64_t)blockIdx.x * nw + wave; c < chunks; c += waves, ++k) {
        __builtin_amdgcn_global_load_lds((glb_void_t *)(p + c * 64 + lane), (lds_void_t *)(ring + (k % kProbeRing) * 1024),
                                         16, 0, 0);
        if (k >= kProbeRing - 1) vm_wait<kProbeRing - 1>();
    }
    vm_wait<0>();
    uint32_t acc = 0;
    if (k > 0) {
        const u32x4 v = reinterpret_cast<const u32x4 *>(ring + ((k - 1) % kProbeRing) * 1024)[lane];
        acc = v[0] ^ v[1] ^ v[2] ^ v[3];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
    if (lane == 0) sink[blockIdx.x * nw + wave] = acc;
}

// Writes zeros over the buffer, 16 bytes per lane per store.
__global__ __launch_bounds__(kProbeThreads) void probe_write_kernel(u32x4 *__restrict__ p, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, p + i);
}

// One wave: the shader clock counter and the 100 MHz real-time counter at the start, a wait of
// spin_ns of real time (bounded by the caller's check), the two counters again.
__global__ __launch_bounds__(64) void probe_clock_kernel(uint64_t *__restrict__ stamps, int64_t spin_ticks)
{
    const uint64_t m0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    uint64_t r1 = r0;
    while (r1 - r0 < (uint64_t)spin_ticks) {
        __builtin_amdgcn_s_sleep(2);
        r1 = __builtin_amdgcn_s_memrealtime();
    }
    const uint64_t m1 = __builtin_amdgcn_s_memtime();
    r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        stamps[0] = m0;
        stamps[1] = r0;
        stamps[2] = m1;
        stamps[3] = r1;
    }
}

}  // namespace

// mode 0: read by 16-byte vector loads; 1: read by direct global->LDS copies; 2: write zeros.
// One workgroup of 8 waves per CU; the sink takes one word per wave.
hipError_t launch_probe_stream(void *buf, int64_t bytes, int mode, uint32_t *sink, hipStream_t stream)
{
    const int cus = device_cus();
    const int grid = cus < 2048 ? cus : 2048;
    int64_t n16 = bytes / 16;
    if (mode == 0) {
        const u32x4 *p = static_cast<const u32x4 *>(buf);
        void *args[] = {&p, &n16, &sink};
        return launch_kernel(reinterpret_cast<const void *>(&probe_read_kernel), "probe_read_kernel", dim3(grid),
                             dim3(kProbeThreads), args, 0, stream);
    }
    if (mode == 1) {
        const size_t lds = (size_t)(kProbeThreads / 64) * kProbeRing * 1024;
        const u32x4 *p = static_cast<const u32x4 *>(buf);
        void *args[] = {&p, &n16, &sink};
        return launch_kernel(reinterpret_cast<const void *>(&probe_lds_kernel), "probe_lds_kernel", dim3(grid),
                             dim3(kProbeThreads), args, lds, stream);
    }
    u32x4 *p = static_cast<u32x4 *>(buf);
    void *args[] = {&p, &n16};
    return launch_kernel(reinterpret_cast<const void *>(&probe_write_kernel), "probe_write_kernel", dim3(grid),
                         dim3(kProbeThreads), args, 0, stream);
}

hipError_t launch_probe_clock(uint64_t *stamps, int64_t spin_ns, hipStream_t stream)
{
    int64_t ticks = (spin_ns + 9) / 10;             // the real-time counter runs at 100 MHz
    void *args[] = {&stamps, &ticks};
    return launch_kernel(reinterpret_cast<const void *>(&probe_clock_kernel), "probe_clock_kernel", dim3(1), dim3(64),
                         args, 0, stream);
}

}  // namespace bonsai
