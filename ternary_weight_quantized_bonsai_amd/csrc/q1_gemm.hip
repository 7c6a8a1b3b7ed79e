// q1_gemm.hip -- binary g128 prefill GEMM on gfx950 MFMA:  y[M][N] = x[M][K] W^T.
//
// Prefill is the compute-bound phase ("1-bit Bonsai 27B" model card, cross-platform
// throughput: pp512), so the contraction runs on the matrix cores (v_mfma_f32_32x32x16_f16,
// fp16 in, fp32 accumulate).  The weights reach the MFMA B operand straight from the packed
// sign words: each lane expands its bits to binary16 +-s in registers (exact: -s is s with the
// sign bit flipped), so the group scale is folded into the operand and one accumulator set
// runs across all groups.  No FP16 copy of W is written anywhere.
//
// Tiling.  A workgroup of 4 waves computes a 128 (M) x 256 (N) tile; wave w owns columns
// 64w .. 64w+63 of it, all 128 rows, as 4 x 2 MFMA tiles of 32 x 32.  K advances 64 at a
// time.  The X tile (128 rows x 128 B) is staged in LDS by direct global->LDS loads, double
// buffered, with the 16-byte chunk c of row r stored at 128 r + 16 (c ^ ((r >> 1) & 7)) so
// the MFMA A-operand reads (32 rows, one 16-byte chunk each) are free of bank conflicts.
// Each lane reads its two columns' sign words straight into registers.
//
// Sign expansion in natural k order.  An MFMA lane holds 8 consecutive k of its operand as 4
// half pairs (k, k+1).  Merging a word with itself shifted (u = bits 0..15 | bits 1..16 in the
// high half, u2 likewise for bits 16..31) places bits k and k+1 at positions q and 16+q, so
// one shift puts both on the binary16 sign bits and an and-xor with (-s, -s) yields (+-s, +-s).
#include <limits.h>

#include <type_traits>

#include "device.h"
#include "launch.h"

namespace bonsai {
namespace {

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int XTILE = BM * BK * 2;               // 16 KB per buffer

typedef float float16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glb_void_t;

// 4 dwords (k = p .. p+7 of a 16-k half-word) of +-s from the merged word v, whose bits q and
// 16+q hold k = q and q+1 of that half-word; c = (-s, -s).
__device__ __forceinline__ half8_t expand8(uint32_t v, int p, uint32_t c)
{
    u32x4 e;
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = ((v << (15 - (p + 2 * i))) & 0x80008000u) ^ c;
    return __builtin_bit_cast(half8_t, e);
}

constexpr int NS = 4;                            // pipeline depth (X tiles in LDS, B words in registers)

__global__ __launch_bounds__(256) void q1_gemm_kernel(const uint32_t *__restrict__ wbits,
                                                      const uint16_t *__restrict__ scales,
                                                      const uint16_t *__restrict__ x,
                                                      float *__restrict__ y, int M, int N, int K)
{
    __shared__ __attribute__((aligned(16))) char xs[NS * XTILE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tiles_n = (N + BN - 1) / BN;
    const int m0 = (blockIdx.x / tiles_n) * BM, n0 = (blockIdx.x % tiles_n) * BN;
    const int G = K >> 7, W = K >> 5;
    const int KT = K / BK;

    // X staging: this wave issues instructions 4 wave .. 4 wave + 3 of the tile's 16
    // (8 rows x 128 B each): lane -> row 8i + lane/8, chunk (lane%8) ^ ((row >> 1) & 7)
    const u32x4 *xg = reinterpret_cast<const u32x4 *>(x);           // row m, chunk c at m * (K/8) + c
    size_t xsrc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 8 * (4 * wave + j) + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        xsrc[j] = (size_t)min(m0 + r, M - 1) * (K >> 3) + c;
    }

    // B: this lane's columns n0 + 64 wave + (lane % 32) + 32 t, t = 0, 1; its k-block lane / 32
    const int q = lane >> 5;
    int ncol[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) ncol[t] = min(n0 + 64 * wave + (lane & 31) + 32 * t, N - 1);
    const uint2 *wrow[2] = {reinterpret_cast<const uint2 *>(wbits + (size_t)ncol[0] * W),
                            reinterpret_cast<const uint2 *>(wbits + (size_t)ncol[1] * W)};
    const uint16_t *srow[2] = {scales + (size_t)ncol[0] * G, scales + (size_t)ncol[1] * G};

    float16_t acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

    // One pipeline stage = 8 VMEM instructions per wave: 4 X DMAs, 2 B word pairs, 2 scales.
    uint2 wd[NS][2];
    uint32_t sb[NS][2];
    auto issue = [&](int kt, auto slot_c) {
        constexpr int slot = decltype(slot_c)::value;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_global_load_lds((glb_void_t *)(xg + xsrc[j] + kt * (BK / 8)),
                                             (lds_void_t *)(xs + slot * XTILE + (4 * wave + j) * 1024), 16, 0, 0);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            wd[slot][t] = wrow[t][kt];
            sb[slot][t] = srow[t][kt >> 1];
        }
    };

    auto compute = [&](auto slot_c) {
        constexpr int slot = decltype(slot_c)::value;
        const char *xb = xs + slot * XTILE;
        uint32_t cs[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) cs[t] = (sb[slot][t] | (sb[slot][t] << 16)) ^ 0x80008000u;   // (-s, -s)
        half8_t af[2][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int r = 32 * mt + (lane & 31);
            af[0][mt] = *reinterpret_cast<const half8_t *>(xb + 128 * r + 16 * (q ^ ((r >> 1) & 7)));
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {                // k16 steps: word s/2, half s%2
            if (s + 1 < 4) {                         // next k16 step's A fragments
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int r = 32 * mt + (lane & 31);
                    const int c = 2 * (s + 1) + q;
                    af[(s + 1) & 1][mt] = *reinterpret_cast<const half8_t *>(xb + 128 * r + 16 * (c ^ ((r >> 1) & 7)));
                }
            }
            half8_t bf[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint32_t w = (s >> 1) ? wd[slot][t].y : wd[slot][t].x;
                const uint32_t hi = 0xFFFF0000u;
                const uint32_t v = (s & 1) ? (((w >> 1) & hi) | (((w >> 16) | (w << 16)) & ~hi))
                                           : (((w << 15) & hi) | (w & ~hi));
                bf[t] = expand8(v, 8 * q, cs[t]);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    acc[mt][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[s & 1][mt], bf[t], acc[mt][t], 0, 0, 0);
        }
    };

    // Step kt: wait for stage kt (later stages may stay in flight), barrier (all waves' DMAs
    // landed, all waves done with the slot about to be refilled), refill, compute.
    auto step = [&](int kt, auto slot_c) {
        constexpr int slot = decltype(slot_c)::value;
        const int ahead = min(NS - 2, KT - 1 - kt);  // stages issued after stage kt
        // s_waitcnt fields: vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8]
        if (ahead >= 2) __builtin_amdgcn_s_waitcnt(0x4F70);        // vmcnt(16)
        else if (ahead == 1) __builtin_amdgcn_s_waitcnt(0x0F78);   // vmcnt(8)
        else __builtin_amdgcn_s_waitcnt(0x0F70);                   // vmcnt(0)
        // Workgroup barrier without the release fence __syncthreads() implies (which would
        // drain every in-flight stage); the clobber keeps LDS accesses on their side of it.
        asm volatile("s_barrier" ::: "memory");
        if (kt + NS - 1 < KT) issue(kt + NS - 1, std::integral_constant<int, (slot + NS - 1) % NS>{});
        compute(slot_c);
    };

#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
        if (i < KT) {
            if (i == 0) issue(0, std::integral_constant<int, 0>{});
            if (i == 1) issue(1, std::integral_constant<int, 1>{});
            if (i == 2) issue(2, std::integral_constant<int, 2>{});
        }
    for (int kt = 0; kt < KT; kt += NS) {
        step(kt, std::integral_constant<int, 0>{});
        if (kt + 1 < KT) step(kt + 1, std::integral_constant<int, 1>{});
        if (kt + 2 < KT) step(kt + 2, std::integral_constant<int, 2>{});
        if (kt + 3 < KT) step(kt + 3, std::integral_constant<int, 3>{});
    }

    // D layout (32 x 32): lane holds column lane % 32, rows 8 (i / 4) + 4 (lane / 32) + i % 4
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int col = n0 + 64 * wave + 32 * t + (lane & 31);
            if (col >= N) continue;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int rowm = m0 + 32 * mt + 8 * (i >> 2) + 4 * q + (i & 3);
                if (rowm < M) y[(size_t)rowm * N + col] = acc[mt][t][i];
            }
        }
}

}  // namespace

hipError_t launch_q1_gemm(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x, float *y,
                          int M, int N, int K, hipStream_t stream)
{
    const int64_t tiles = (int64_t)((N + BN - 1) / BN) * ((M + BM - 1) / BM);
    if (tiles > INT_MAX || K % BK != 0) return hipErrorInvalidValue;
    void *args[] = {&wbits, &scales, &x, &y, &M, &N, &K};
    return launch_kernel(reinterpret_cast<const void *>(&q1_gemm_kernel), dim3((unsigned)tiles), dim3(256),
                         args, 0, stream);
}

}  // namespace bonsai
