// q1_gemm.hip -- binary g128 prefill GEMM on gfx950 MFMA:  y[M][N] = x[M][K] W^T.
//
// Prefill is the compute-bound phase ("1-bit Bonsai 27B" model card, cross-platform
// throughput: pp512), so the contraction runs on the matrix cores (v_mfma_f32_16x16x32_f16,
// fp16 in, fp32 accumulate).  The weights reach the MFMA B operand straight from the packed
// sign words: each lane expands its bits to binary16 +-s in registers (exact: -s is s with
// the sign bit flipped), so the group scale is folded into the operand and one accumulator
// set runs across all groups.  No FP16 copy of W is ever written anywhere.
//
// k interleave.  An MFMA lane holds 8 k-values of its operand.  The sign expansion pairs bit
// j with bit j+16 of a word (one shift puts both on the binary16 sign positions), so within
// each 32-wide K-step the MFMA's k order is (0,16,1,17,...,15,31).  The X tile is written to
// LDS in the same interleaved order, so A and B agree on every k and the sum is unchanged.
//
// Tiling: 128 x 128 output tile per workgroup of 4 waves (2 x 2), each wave 64 x 64 as a
// 4 x 4 grid of 16 x 16 MFMA tiles; K advances 32 per step through a double-buffered LDS
// X tile.
#include <limits.h>

#include "device.h"
#include "launch.h"

namespace bonsai {
namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int XS_STRIDE = 20;                  // dwords per LDS row (16 used + 4 pad)

__global__ __launch_bounds__(256) void q1_gemm_kernel(const uint32_t *__restrict__ wbits,
                                                      const uint16_t *__restrict__ scales,
                                                      const uint16_t *__restrict__ x,
                                                      float *__restrict__ y, int M, int N, int K)
{
    __shared__ uint32_t xs[2][BM * XS_STRIDE];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_n = (N + BN - 1) / BN;
    const int m0 = (blockIdx.x / tiles_n) * BM, n0 = (blockIdx.x % tiles_n) * BN;
    const int G = K >> 7, W = K >> 5;
    const int KT = K / BK;

    // X staging: thread -> (tile row tid/2, j-half tid&1 covering j = 8h .. 8h+7 of the step)
    const int xr = tid >> 1, xh = tid & 1;
    const bool xlive = (m0 + xr) < M;
    const uint16_t *xrow = x + (size_t)(xlive ? m0 + xr : 0) * K;

    // B: lane (n = lane & 15, q = lane >> 4) of N-block nb
    const int q = lane >> 4;
    int nrow[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) nrow[nb] = min(n0 + wn * 64 + nb * 16 + (lane & 15), N - 1);

    float4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = (float4_t){0.f, 0.f, 0.f, 0.f};

    auto stage = [&](int kt, int buf) {
        uint4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
        if (xlive) {
            lo = *reinterpret_cast<const uint4 *>(xrow + kt * BK + 8 * xh);
            hi = *reinterpret_cast<const uint4 *>(xrow + kt * BK + 16 + 8 * xh);
        }
        uint4 d0, d1;   // dword j' = (x[8h+j'], x[16+8h+j'])
        d0.x = pack_lo(lo.x, hi.x); d0.y = pack_hi(lo.x, hi.x);
        d0.z = pack_lo(lo.y, hi.y); d0.w = pack_hi(lo.y, hi.y);
        d1.x = pack_lo(lo.z, hi.z); d1.y = pack_hi(lo.z, hi.z);
        d1.z = pack_lo(lo.w, hi.w); d1.w = pack_hi(lo.w, hi.w);
        uint4 *dst = reinterpret_cast<uint4 *>(&xs[buf][xr * XS_STRIDE + 8 * xh]);
        dst[0] = d0;
        dst[1] = d1;
    };

    stage(0, 0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) stage(kt + 1, buf ^ 1);

        // B fragments: dword i = (bit 4q+i, bit 16+4q+i) of the row's word, as +-s
        half8_t bf[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const uint32_t wd = wbits[(size_t)nrow[nb] * W + kt];
            const uint32_t sb = scales[(size_t)nrow[nb] * G + (kt >> 2)];
            const uint32_t c = (sb | (sb << 16)) ^ 0x80008000u;     // (-s, -s)
            uint32_t e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) e[i] = ((wd << (15 - 4 * q - i)) & 0x80008000u) ^ c;
            bf[nb] = __builtin_bit_cast(half8_t, (uint4){e[0], e[1], e[2], e[3]});
        }
        // A fragments from LDS: row m = lane & 15 of M-block mb, dwords 4q .. 4q+3
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const uint4 av = *reinterpret_cast<const uint4 *>(
                &xs[buf][(wm * 64 + mb * 16 + (lane & 15)) * XS_STRIDE + 4 * q]);
            const half8_t af = __builtin_bit_cast(half8_t, av);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[nb], acc[mb][nb], 0, 0, 0);
        }
        __syncthreads();
    }

    // C tile layout: lane holds rows 4*(lane>>4) + i, column lane & 15
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int col = n0 + wn * 64 + nb * 16 + (lane & 15);
            if (col >= N) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rowm = m0 + wm * 64 + mb * 16 + 4 * (lane >> 4) + i;
                if (rowm < M) y[(size_t)rowm * N + col] = acc[mb][nb][i];
            }
        }
}

}  // namespace

hipError_t launch_q1_gemm(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x, float *y,
                          int M, int N, int K, hipStream_t stream)
{
    const int64_t tiles = (int64_t)((N + BN - 1) / BN) * ((M + BM - 1) / BM);
    if (tiles > INT_MAX) return hipErrorInvalidValue;
    void *args[] = {&wbits, &scales, &x, &y, &M, &N, &K};
    return launch_kernel(reinterpret_cast<const void *>(&q1_gemm_kernel), dim3((unsigned)tiles), dim3(256),
                           args, 0, stream);
}

}  // namespace bonsai
