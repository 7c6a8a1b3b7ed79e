// q1_gemv.hip -- binary g128 decode GEMV on gfx950 for one row of x:  y[n] = sum_k W[n][k] x[k].
//
// The matmul runs straight on the packed sign words ("1-bit Bonsai 27B" model card: the
// weights are used packed and never expanded back to FP16; the CUDA kernel unpacks the sign
// codes inside the matmul and applies the group scales).  Decode is the memory-bound phase
// (model card, cross-platform throughput), so the kernels are organised around streaming the
// 1.125 bits/weight from HBM once, with as few VALU operations per weight as possible: the
// signs of four weights index a table of the 16 signed sums of their x values.
//
// Work split.  A workgroup owns 64 consecutive weight rows (lane r of every wave <-> row r);
// its waves take disjoint K-slices (whole groups) of those rows and meet in LDS at the end,
// summed in a fixed order.  Weight bytes reach LDS by direct global->LDS loads of whole lines.
// Two to eight rows of x (M = 2..8) go to the matrix-core GEMV instead (gemv_mfma.hip).
#include "device.h"
#include "launch.h"

namespace bonsai {
namespace {

// ---- M = 1: nibble lookup tables ------------------------------------------------------------
//
// For every 4-wide chunk c of a group, a 16-entry fp32 table holds T_c[v] = sum_{j<4} +-x_{4c+j}
// with the sign of term j given by bit j of v (bit 1 -> +x, bit 0 -> -x).  A row's 128 sign
// bits of the group are then 32 nibbles, and the group's signed sum is sum_c T_c[nibble_c]:
// one LDS read and one add per 4 weights, about 0.6 VALU operations per weight in all.  The
// 32 tables of a group (2 KB) are built by the wave itself (two 16-byte LDS writes per lane).
//
// Addressing: with l = w << 2 and h = w >> 2, the low / high nibble of byte k of w, times 4, is
// one SDWA and of byte k of l / h with 0x3C, written into byte 0 of an address register whose
// bits 8..31 hold the (256-aligned) table base.  Chunk c's table is 16 consecutive floats at
// byte offset 64*c (the read's immediate offset), so the 16 possible addresses of a lookup lie
// in 16 distinct LDS banks: lookups never conflict, equal nibbles broadcast.
//
// Weight tile: 8 groups (128 B) of each of the wave's 64 rows arrive through direct
// global->LDS loads, 8 rows x 128 B per instruction (fully used lines).  The 16-byte cell of
// (row r, group u) of a batch sits at 128*r + 16*(u ^ ((r >> 1) & 7)): the swizzle keeps a
// wave's row-wise reads of one column free of bank conflicts.

// r[7:0] = 4 * nibble (byte KB of v masked with 0x3C); r[31:8] keep the LUT base (256-aligned).
template <int KB>
__device__ __forceinline__ void nib_addr(uint32_t &r, uint32_t v, uint32_t mask_3c)
{
    if constexpr (KB == 0)
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:BYTE_0" : "+v"(r) : "s"(mask_3c), "v"(v));
    else if constexpr (KB == 1)
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:BYTE_1" : "+v"(r) : "s"(mask_3c), "v"(v));
    else if constexpr (KB == 2)
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:BYTE_2" : "+v"(r) : "s"(mask_3c), "v"(v));
    else
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:BYTE_3" : "+v"(r) : "s"(mask_3c), "v"(v));
}

typedef __attribute__((address_space(3))) float lds_f32_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glb_void_t;

// float at LDS byte address addr + imm (imm becomes the instruction's offset field)
__device__ __forceinline__ float lds_f32(uint32_t addr, int imm)
{
    return reinterpret_cast<const lds_f32_t *>(static_cast<uintptr_t>(addr))[imm / 4];
}

// The 8 table addresses of one word (chunks 8i .. 8i+7 of the group); r[] keep the base.
__device__ __forceinline__ void word_addrs(uint32_t w, uint32_t r[8], uint32_t mask_3c)
{
    const uint32_t l = w << 2, h = w >> 2;
    nib_addr<0>(r[0], l, mask_3c); nib_addr<0>(r[1], h, mask_3c);
    nib_addr<1>(r[2], l, mask_3c); nib_addr<1>(r[3], h, mask_3c);
    nib_addr<2>(r[4], l, mask_3c); nib_addr<2>(r[5], h, mask_3c);
    nib_addr<3>(r[6], l, mask_3c); nib_addr<3>(r[7], h, mask_3c);
}

constexpr int kLutBatch = 8;                        // groups per weight tile (128 B per row)
constexpr int kLutTileBytes = 64 * kLutBatch * 16;  // 8 KB
constexpr int kLutBytes = 32 * 16 * 4;              // 2 KB of tables per group

__global__ __launch_bounds__(384) void q1_gemv_lut_kernel(const uint32_t *__restrict__ wbits,
                                                          const uint16_t *__restrict__ scales,
                                                          const uint16_t *__restrict__ x,
                                                          float *__restrict__ y, int N, int K, int gps)
{
    constexpr int B = kLutBatch;
    extern __shared__ u32x4 lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int G = K >> 7;
    const int row0 = blockIdx.x * 64;
    const int row = row0 + lane;
    const int g0 = wave * gps;
    const int g1 = min(G, g0 + gps);

    char *wl = reinterpret_cast<char *>(lds) + wave * (kLutTileBytes + kLutBytes);
    char *tile = wl;
    char *lut = wl + kLutTileBytes;
    const u32x4 *wg = reinterpret_cast<const u32x4 *>(wbits);      // (row n, group g) at n * G + g
    const uint16_t *srow = scales + (size_t)min(row, N - 1) * G;
    const bool vec_scales = (G & 7) == 0;       // batches then start at multiples of 8 groups
    const uint32_t mask_3c = __builtin_amdgcn_readfirstlane(0x3Cu);
    const uint32_t lut_addr = (uint32_t)(uintptr_t)((lds_char_t *)lut);
    uint32_t raddr[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) raddr[j] = lut_addr;

    // table build: this lane writes entries 4*bt .. 4*bt+3 of chunks bc and bc + 16
    const int bc = lane >> 2, bt = lane & 3;
    const float sg2 = (bt & 1) ? 1.f : -1.f, sg3 = (bt & 2) ? 1.f : -1.f;
    uint2 xq0 = *reinterpret_cast<const uint2 *>(x + (size_t)g0 * 128 + 4 * bc);
    uint2 xq1 = *reinterpret_cast<const uint2 *>(x + (size_t)g0 * 128 + 4 * (bc + 16));

    // tile load: instruction i fetches row 8i + lane/8, group (lane%8) ^ ((row >> 1) & 7)
    float sc[B];
    auto issue = [&](int gb) {
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int r = 8 * i + (lane >> 3);
            const int gg = min(gb + ((lane & 7) ^ ((r >> 1) & 7)), g1 - 1);
            const int rr = min(row0 + r, N - 1);
            __builtin_amdgcn_global_load_lds((glb_void_t *)(wg + (size_t)rr * G + gg),
                                             (lds_void_t *)(tile + i * 1024), 16, 0, 0);
        }
        if (vec_scales) {
            // the batch's 8 scales of this row in one 16-byte load (K % 1024 == 0 keeps every
            // row's scales and every batch start 16-byte aligned)
            const u32x4 v = *reinterpret_cast<const u32x4 *>(srow + gb);
#pragma unroll
            for (int u = 0; u < B; ++u) sc[u] = f16_bits_to_f32((uint16_t)(v[u >> 1] >> (16 * (u & 1))));
        } else {
#pragma unroll
            for (int u = 0; u < B; ++u) sc[u] = f16_bits_to_f32(srow[min(gb + u, g1 - 1)]);
        }
    };

    float acc = 0.f;
    issue(g0);
    for (int gb = g0; gb < g1; gb += B) {
        __builtin_amdgcn_s_waitcnt(0x0F70);             // vmcnt(0): tile and scales of this batch
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int g = gb + u;
            if (g >= g1) break;
            // build the 32 tables of group g, then fetch the next group's x
            const uint2 xc[2] = {xq0, xq1};
            if (g + 1 < g1) {
                xq0 = *reinterpret_cast<const uint2 *>(x + (size_t)(g + 1) * 128 + 4 * bc);
                xq1 = *reinterpret_cast<const uint2 *>(x + (size_t)(g + 1) * 128 + 4 * (bc + 16));
            }
#pragma unroll
            for (int hq = 0; hq < 2; ++hq) {
                const half2_t p01 = as_half2(xc[hq].x), p23 = as_half2(xc[hq].y);
                const float x0 = (float)p01[0], x1 = (float)p01[1];
                const float base = fmaf(sg3, (float)p23[1], fmaf(sg2, (float)p23[0], -x0 - x1));
                u32x4 e;
                e[0] = __builtin_bit_cast(uint32_t, base);                                  // v = 4bt
                e[1] = __builtin_bit_cast(uint32_t, fmaf(2.f, x0, base));                  // v = 4bt + 1
                e[2] = __builtin_bit_cast(uint32_t, fmaf(2.f, x1, base));                  // v = 4bt + 2
                e[3] = __builtin_bit_cast(uint32_t, fmaf(2.f, x1, fmaf(2.f, x0, base)));   // v = 4bt + 3
                *reinterpret_cast<u32x4 *>(lut + 64 * (bc + 16 * hq) + 16 * bt) = e;
            }
            // this lane's row: 4 words x 8 nibbles, two words (16 reads) in flight at a time
            const u32x4 q = *reinterpret_cast<const u32x4 *>(tile + 128 * lane + 16 * (u ^ ((lane >> 1) & 7)));
            float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                word_addrs(q[i], &raddr[0], mask_3c);          // in place: only bits 0..7 change
                word_addrs(q[i + 1], &raddr[8], mask_3c);
                float t[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) t[j] = lds_f32(raddr[j], 64 * (8 * i + j));
                a0 += (t[0] + t[1]) + (t[2] + t[3]);
                a1 += (t[4] + t[5]) + (t[6] + t[7]);
                a2 += (t[8] + t[9]) + (t[10] + t[11]);
                a3 += (t[12] + t[13]) + (t[14] + t[15]);
            }
            acc = fmaf(sc[u], (a0 + a1) + (a2 + a3), acc);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);             // lgkmcnt(0): tile reads done before reuse
        if (gb + B < g1) issue(gb + B);
    }

    if (nwaves == 1) {
        if (row < N) y[row] = acc;
        return;
    }
    float *red = reinterpret_cast<float *>(reinterpret_cast<char *>(lds) + nwaves * (kLutTileBytes + kLutBytes));
    red[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave == 0 && row < N) {
        float t = red[lane];
        for (int w = 1; w < nwaves; ++w) t += red[w * 64 + lane];
        y[row] = t;
    }
}

// Small N (at most 256 row tiles, one per CU): one 64-row tile per workgroup and one 4-group
// K-slice per wave, so every wave has a single 4 KB copy and 128 lookups per lane after it
// lands; the waves' partial sums meet in LDS in a fixed order.  A wave builds only its own 4
// groups' tables, all at once (one wait), after its copy and x have arrived.
constexpr int kL4Groups = 4;
constexpr int kL4Tile = 64 * kL4Groups * 16;        // 4 KB: 64 rows x 4 groups
constexpr int kL4Lut = kL4Groups * kLutBytes;       // 8 KB of tables
constexpr int kL4Wave = kL4Tile + kL4Lut + 64 * 4;  // + this wave's partial sums
constexpr int kL4MaxWaves = 13;                     // 13 x 12.25 KB fits the 160 KB of LDS

template <bool VEC_SCALES>
__global__ __launch_bounds__(kL4MaxWaves * 64) void q1_gemv_lut4_kernel(const uint32_t *__restrict__ wbits,
                                                                        const uint16_t *__restrict__ scales,
                                                                        const uint16_t *__restrict__ x,
                                                                        float *__restrict__ y, int N, int K)
{
    extern __shared__ u32x4 lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int G = K >> 7;
    const int g0 = wave * kL4Groups, g1 = min(G, g0 + kL4Groups), gl = g1 - 1;
    const int row = blockIdx.x * 64 + lane;
    char *const tile = reinterpret_cast<char *>(lds) + wave * kL4Wave;
    char *const lut = tile + kL4Tile;
    float *const part = reinterpret_cast<float *>(lut + kL4Lut);

    // tile copy: instruction k covers rows 16 k .. 16 k + 15, 4 lanes per row; the cell of
    // (row r, group u) lands at 64 r + 16 (u ^ ((r >> 2) & 3))
    const u32x4 *wg = reinterpret_cast<const u32x4 *>(wbits);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int r = 16 * k + (lane >> 2);
        const int gg = min(g0 + ((lane & 3) ^ ((r >> 2) & 3)), gl);
        const int rr = min(blockIdx.x * 64 + r, N - 1);
        __builtin_amdgcn_global_load_lds((glb_void_t *)(wg + (size_t)rr * G + gg),
                                         (lds_void_t *)(tile + k * 1024), 16, 0, 0);
    }
    const uint16_t *srow = scales + (size_t)min(row, N - 1) * G;
    uint2 scv;                                      // VEC_SCALES: the 4 scales as loaded
    uint32_t scs[kL4Groups];
    if constexpr (VEC_SCALES) {
        scv = *reinterpret_cast<const uint2 *>(srow + g0);
    } else {
#pragma unroll
        for (int u = 0; u < kL4Groups; ++u) scs[u] = srow[min(g0 + u, gl)];
    }

    // tables: lane builds quads e = lane + 64 k of the wave's 4 groups (group u = e / 128,
    // chunk c, entries 4 bt .. 4 bt + 3), from x loaded all at once
    uint2 xq[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int e = lane + 64 * k;
        xq[k] = *reinterpret_cast<const uint2 *>(x + (size_t)min(g0 + (e >> 7), gl) * 128 + 4 * ((e >> 2) & 31));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int e = lane + 64 * k;
        const int u = e >> 7, c = (e >> 2) & 31, bt = e & 3;
        const half2_t p01 = as_half2(xq[k].x), p23 = as_half2(xq[k].y);
        const float x0 = (float)p01[0], x1 = (float)p01[1];
        const float sg2 = (bt & 1) ? 1.f : -1.f, sg3 = (bt & 2) ? 1.f : -1.f;
        const float base = fmaf(sg3, (float)p23[1], fmaf(sg2, (float)p23[0], -x0 - x1));
        u32x4 ev;
        ev[0] = __builtin_bit_cast(uint32_t, base);                                 // v = 4bt
        ev[1] = __builtin_bit_cast(uint32_t, fmaf(2.f, x0, base));                 // v = 4bt + 1
        ev[2] = __builtin_bit_cast(uint32_t, fmaf(2.f, x1, base));                 // v = 4bt + 2
        ev[3] = __builtin_bit_cast(uint32_t, fmaf(2.f, x1, fmaf(2.f, x0, base)));  // v = 4bt + 3
        *reinterpret_cast<u32x4 *>(lut + u * kLutBytes + 64 * c + 16 * bt) = ev;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);             // vmcnt(0): the tile copy landed
    __builtin_amdgcn_s_waitcnt(0xC07F);             // lgkmcnt(0): this wave's tables are written

    const uint32_t mask_3c = __builtin_amdgcn_readfirstlane(0x3Cu);
    const uint32_t lut_addr = (uint32_t)(uintptr_t)((lds_char_t *)lut);
    uint32_t raddr[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) raddr[j] = lut_addr;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < kL4Groups; ++u) {
        const u32x4 q = *reinterpret_cast<const u32x4 *>(tile + 64 * lane + 16 * (u ^ ((lane >> 2) & 3)));
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            word_addrs(q[i], &raddr[0], mask_3c);
            word_addrs(q[i + 1], &raddr[8], mask_3c);
            float t[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) t[j] = lds_f32(raddr[j], u * kLutBytes + 64 * (8 * i + j));
            a0 += (t[0] + t[1]) + (t[2] + t[3]);
            a1 += (t[4] + t[5]) + (t[6] + t[7]);
            a2 += (t[8] + t[9]) + (t[10] + t[11]);
            a3 += (t[12] + t[13]) + (t[14] + t[15]);
        }
        uint32_t sbits;
        if constexpr (VEC_SCALES) sbits = ((u & 2) ? scv.y : scv.x) >> (16 * (u & 1));
        else sbits = scs[u];
        // groups past K (the last wave's slice may be short) count with scale 0
        const float s = (g0 + u < g1) ? f16_bits_to_f32((uint16_t)sbits) : 0.f;
        acc = fmaf(s, (a0 + a1) + (a2 + a3), acc);
    }
    part[lane] = acc;
    __syncthreads();
    if (wave == 0 && row < N) {
        float t = acc;
        for (int w = 1; w < nwaves; ++w)
            t += reinterpret_cast<const float *>(reinterpret_cast<char *>(lds) + w * kL4Wave + kL4Tile + kL4Lut)[lane];
        y[row] = t;
    }
}

hipError_t launch_lut4(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x, float *y,
                       int N, int K, hipStream_t stream)
{
    const int G = K / 128;
    const int tiles = (N + 63) / 64;
    const int waves = (G + kL4Groups - 1) / kL4Groups;
    const size_t lds = (size_t)waves * kL4Wave;
    const bool vec = (G % kL4Groups) == 0;          // every wave's scales then start 8-byte aligned
    const void *fn = vec ? reinterpret_cast<const void *>(&q1_gemv_lut4_kernel<true>)
                         : reinterpret_cast<const void *>(&q1_gemv_lut4_kernel<false>);
    static const bool attrs_set = [] {
        const int most = kL4MaxWaves * kL4Wave;
        return hipFuncSetAttribute(reinterpret_cast<const void *>(&q1_gemv_lut4_kernel<true>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, most) == hipSuccess &&
               hipFuncSetAttribute(reinterpret_cast<const void *>(&q1_gemv_lut4_kernel<false>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, most) == hipSuccess;
    }();
    if (!attrs_set) return hipErrorInvalidValue;
    void *args[] = {&wbits, &scales, &x, &y, &N, &K};
    return launch_kernel(fn, dim3(tiles), dim3(64 * waves), args, lds, stream);
}

hipError_t launch_lut(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x, float *y,
                      int N, int K, hipStream_t stream)
{
    const int G = K / 128;
    const int tiles = (N + 63) / 64;
    constexpr size_t per_wave = kLutTileBytes + kLutBytes;
    // Split K across the waves of a workgroup only until the grid has a wave per SIMD
    // (1024 SIMDs): the LDS each wave needs makes more, smaller waves a net loss.
    int slices = 1;
    while (slices < 6 && (int64_t)tiles * slices < 1024 && slices * kLutBatch < G) ++slices;
    int gps = (G + slices - 1) / slices;
    gps = ((gps + kLutBatch - 1) / kLutBatch) * kLutBatch;
    slices = (G + gps - 1) / gps;
    const size_t lds = (size_t)slices * per_wave + (slices > 1 ? (size_t)slices * 64 * sizeof(float) : 0);
    void *args[] = {&wbits, &scales, &x, &y, &N, &K, &gps};
    return launch_kernel(reinterpret_cast<const void *>(&q1_gemv_lut_kernel), dim3(tiles), dim3(64 * slices),
                         args, lds, stream);
}

}  // namespace

hipError_t launch_q1_gemv(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x, float *y,
                          int M, int N, int K, hipStream_t stream)
{
    if (M >= 2 && M <= 8) return launch_gemv_mfma(false, wbits, scales, x, y, M, N, K, stream);
    if (M != 1) return hipErrorInvalidValue;
    // one tile per CU at most and the 4-group slices of K fit one workgroup: small-N kernel
    if ((N + 63) / 64 <= 256 && (K / 128 + kL4Groups - 1) / kL4Groups <= kL4MaxWaves)
        return launch_lut4(wbits, scales, x, y, N, K, stream);
    return launch_lut(wbits, scales, x, y, N, K, stream);
}

}  // namespace bonsai
