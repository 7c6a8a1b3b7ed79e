// q2t_gemv.hip -- ternary g128 decode GEMV on 2-bit codes (gfx950), M <= 8.
//
// Weights are {-1, 0, +1} x FP16 group scale ("Ternary Bonsai 27B" article, ternary format),
// held in 2 bits per weight as the current release does (same article, limitations).  Field
// value 0 -> 0, 1 -> +1, 3 -> -1.
//
// Same work split as the binary GEMV: lane <-> row, K-slices across the waves of a workgroup,
// x wave-uniform in SGPRs, partials summed in LDS in a fixed order.
//
// Code expansion (exact).  Shifting a word left by 14-2j puts field j on bits 14..15 and field
// j+8 on bits 30..31; masking with 0xC000C000 leaves binary16 bit patterns whose sign bit is
// the field's high bit and whose exponent MSB is its low bit: 01 -> +2.0, 11 -> -2.0, 00 -> +0
// (10, reserved, would give -0).  v_dot2_f32_f16 multiplies the pair exactly with
// (x[16w+j], x[16w+8+j]); the factor 2 is folded into the group scale as s/2.
#include "device.h"
#include "launch.h"

namespace bonsai {
namespace {

constexpr int kGroupsPerBatch = 2;

template <int M>
__global__ __launch_bounds__(1024) void q2t_gemv_kernel(const uint32_t *__restrict__ wcodes,
                                                        const uint16_t *__restrict__ scales,
                                                        const uint16_t *__restrict__ x,
                                                        float *__restrict__ y, int N, int K, int gps)
{
    extern __shared__ float red[];
    const int lane = threadIdx.x & 63;
    const int slice = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nslices = blockDim.x >> 6;
    const int G = K >> 7;
    const int row = blockIdx.x * 64 + lane;
    const int r = row < N ? row : N - 1;
    const int g0 = slice * gps;
    const int g1 = min(G, g0 + gps);

    const uint4 *wrow = reinterpret_cast<const uint4 *>(wcodes + (size_t)r * (K >> 4));
    const uint16_t *srow = scales + (size_t)r * G;
    const uint32_t *xd = reinterpret_cast<const uint32_t *>(x);

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;

    for (int gb = g0; gb < g1; gb += kGroupsPerBatch) {
        uint4 q[kGroupsPerBatch][2];
        float s[kGroupsPerBatch];
#pragma unroll
        for (int u = 0; u < kGroupsPerBatch; ++u) {
            const int g = min(gb + u, g1 - 1);
            q[u][0] = wrow[2 * g];
            q[u][1] = wrow[2 * g + 1];
            s[u] = 0.5f * f16_bits_to_f32(srow[g]);
        }
#pragma unroll
        for (int u = 0; u < kGroupsPerBatch; ++u) {
            const int g = gb + u;
            if (g >= g1) break;
            const uint32_t words[8] = {q[u][0].x, q[u][0].y, q[u][0].z, q[u][0].w,
                                       q[u][1].x, q[u][1].y, q[u][1].z, q[u][1].w};
            float part[M];
#pragma unroll
            for (int m = 0; m < M; ++m) part[m] = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint32_t e[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) e[j] = (words[i] << (14 - 2 * j)) & 0xC000C000u;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    // x[16i .. 16i+15] of group g of row m, as 8 dwords
                    const uint32_t *xw = xd + (size_t)m * (K >> 1) + (size_t)g * 64 + i * 8;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint32_t a = xw[j >> 1], b = xw[4 + (j >> 1)];
                        part[m] = dot2(e[j], (j & 1) ? pack_hi(a, b) : pack_lo(a, b), part[m]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < M; ++m) acc[m] = fmaf(s[u], part[m], acc[m]);
        }
    }

    if (nslices == 1) {
        if (row < N)
#pragma unroll
            for (int m = 0; m < M; ++m) y[(size_t)m * N + row] = acc[m];
        return;
    }
#pragma unroll
    for (int m = 0; m < M; ++m) red[(slice * M + m) * 64 + lane] = acc[m];
    __syncthreads();
    if (slice == 0 && row < N) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float t = red[m * 64 + lane];
            for (int sl = 1; sl < nslices; ++sl) t += red[(sl * M + m) * 64 + lane];
            y[(size_t)m * N + row] = t;
        }
    }
}

template <int M>
hipError_t launch_m(const uint32_t *wcodes, const uint16_t *scales, const uint16_t *x, float *y,
                    int N, int K, hipStream_t stream)
{
    const int G = K / 128;
    const int tiles = (N + 63) / 64;
    int slices = 1;
    if (tiles < 2048) slices = min(16, min(G, (2048 + tiles - 1) / tiles));
    const int gps = (G + slices - 1) / slices;
    slices = (G + gps - 1) / gps;
    const size_t lds = slices > 1 ? (size_t)slices * M * 64 * sizeof(float) : 0;
    void *args[] = {&wcodes, &scales, &x, &y, &N, &K, (void *)&gps};
    return launch_kernel(reinterpret_cast<const void *>(&q2t_gemv_kernel<M>), dim3(tiles), dim3(64 * slices), args,
                           lds, stream);
}

}  // namespace

hipError_t launch_q2t_gemv(const uint32_t *wcodes, const uint16_t *scales, const uint16_t *x, float *y,
                           int M, int N, int K, hipStream_t stream)
{
    switch (M) {
    case 1: return launch_m<1>(wcodes, scales, x, y, N, K, stream);
    case 2: return launch_m<2>(wcodes, scales, x, y, N, K, stream);
    case 3: return launch_m<3>(wcodes, scales, x, y, N, K, stream);
    case 4: return launch_m<4>(wcodes, scales, x, y, N, K, stream);
    case 5: return launch_m<5>(wcodes, scales, x, y, N, K, stream);
    case 6: return launch_m<6>(wcodes, scales, x, y, N, K, stream);
    case 7: return launch_m<7>(wcodes, scales, x, y, N, K, stream);
    case 8: return launch_m<8>(wcodes, scales, x, y, N, K, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace bonsai
