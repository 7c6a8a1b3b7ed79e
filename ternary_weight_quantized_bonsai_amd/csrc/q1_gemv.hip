// q1_gemv.hip -- binary g128 decode GEMV on gfx950:  y[m][n] = sum_k W[n][k] x[m][k],  M <= 8.
//
// The matmul runs straight on the packed sign words ("1-bit Bonsai 27B" model card: the
// weights are used packed and never expanded back to FP16; the CUDA kernel unpacks the sign
// codes inside the matmul and applies the group scales).  Decode is the memory-bound phase
// (model card, cross-platform throughput), so the kernel is built around streaming the
// 1.125 bits/weight once from HBM.
//
// Work split.  Lane <-> weight row: each lane of a wave owns one of 64 consecutive rows and
// walks a contiguous slice of its row's groups; the waves of a workgroup take the K-slices
// of the same 64 rows and their partial sums meet in LDS in a fixed order (deterministic).
// Because every lane of a wave is at the same k at the same time, x is wave-uniform and is
// read through the scalar cache into SGPRs: it costs no VGPRs and no vector bandwidth.
//
// Sign expansion (exact).  For bit pair (j, j+16) of a word, shifting the word left by 15-j
// puts the two bits on the binary16 sign positions 15 and 31; and-or with 1.0|1.0 then gives
// the half pair (+-1, +-1) (bit 1 -> -1.0, bit 0 -> +1.0), which v_dot2_f32_f16 multiplies
// exactly with the x pair (x[32w+j], x[32w+16+j]) into an fp32 partial.  Once per 128-weight
// group the partial is multiplied by -s (the minus undoes the flipped polarity).
#include "device.h"
#include "launch.h"

namespace bonsai {
namespace {

constexpr int kGroupsPerBatch = 4;   // loads issued together before the batch is consumed

template <int M>
__global__ __launch_bounds__(1024) void q1_gemv_kernel(const uint32_t *__restrict__ wbits,
                                                       const uint16_t *__restrict__ scales,
                                                       const uint16_t *__restrict__ x,
                                                       float *__restrict__ y, int N, int K, int gps)
{
    extern __shared__ float red[];                      // [slices][M][64] partial sums
    const int lane = threadIdx.x & 63;
    const int slice = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nslices = blockDim.x >> 6;
    const int G = K >> 7;
    const int row = blockIdx.x * 64 + lane;
    const int r = row < N ? row : N - 1;               // tail lanes read a valid row, store nothing
    const int g0 = slice * gps;
    const int g1 = min(G, g0 + gps);

    const uint4 *wrow = reinterpret_cast<const uint4 *>(wbits + (size_t)r * (K >> 5));
    const uint16_t *srow = scales + (size_t)r * G;
    const uint32_t *xd = reinterpret_cast<const uint32_t *>(x);

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;

    for (int gb = g0; gb < g1; gb += kGroupsPerBatch) {
        uint4 q[kGroupsPerBatch];
        float s[kGroupsPerBatch];
#pragma unroll
        for (int u = 0; u < kGroupsPerBatch; ++u) {
            const int g = min(gb + u, g1 - 1);
            q[u] = wrow[g];
            s[u] = f16_bits_to_f32(srow[g]);
        }
#pragma unroll
        for (int u = 0; u < kGroupsPerBatch; ++u) {
            const int g = gb + u;
            if (g >= g1) break;
            const uint32_t words[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
            float part[M];
#pragma unroll
            for (int m = 0; m < M; ++m) part[m] = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t e[16];
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    e[j] = ((words[i] << (15 - j)) & 0x80008000u) | 0x3C003C00u;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    // x[32i .. 32i+31] of group g of row m, as 16 dwords of half pairs
                    const uint32_t *xw = xd + (size_t)m * (K >> 1) + (size_t)g * 64 + i * 16;
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const uint32_t a = xw[j >> 1], b = xw[8 + (j >> 1)];
                        part[m] = dot2(e[j], (j & 1) ? pack_hi(a, b) : pack_lo(a, b), part[m]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < M; ++m) acc[m] = fmaf(-s[u], part[m], acc[m]);
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
hipError_t launch_m(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x, float *y,
                    int N, int K, hipStream_t stream)
{
    const int G = K / 128;
    const int tiles = (N + 63) / 64;
    // Enough waves to cover the chip (1024 SIMDs) at least twice: split K across the waves
    // of a workgroup when there are few row tiles.
    int slices = 1;
    if (tiles < 2048) slices = min(16, min(G, (2048 + tiles - 1) / tiles));
    const int gps = (G + slices - 1) / slices;
    slices = (G + gps - 1) / gps;
    const size_t lds = slices > 1 ? (size_t)slices * M * 64 * sizeof(float) : 0;
    void *args[] = {&wbits, &scales, &x, &y, &N, &K, (void *)&gps};
    return launch_kernel(reinterpret_cast<const void *>(&q1_gemv_kernel<M>), dim3(tiles), dim3(64 * slices), args,
                           lds, stream);
}

}  // namespace

hipError_t launch_q1_gemv(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x, float *y,
                          int M, int N, int K, hipStream_t stream)
{
    switch (M) {
    case 1: return launch_m<1>(wbits, scales, x, y, N, K, stream);
    case 2: return launch_m<2>(wbits, scales, x, y, N, K, stream);
    case 3: return launch_m<3>(wbits, scales, x, y, N, K, stream);
    case 4: return launch_m<4>(wbits, scales, x, y, N, K, stream);
    case 5: return launch_m<5>(wbits, scales, x, y, N, K, stream);
    case 6: return launch_m<6>(wbits, scales, x, y, N, K, stream);
    case 7: return launch_m<7>(wbits, scales, x, y, N, K, stream);
    case 8: return launch_m<8>(wbits, scales, x, y, N, K, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace bonsai
