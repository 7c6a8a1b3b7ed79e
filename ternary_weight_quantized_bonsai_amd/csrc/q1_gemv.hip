// q1_gemv.hip -- binary g128 decode GEMV on gfx950 for one row of x:  y[n] = sum_k W[n][k] x[k].
//
// The matmul runs straight on the packed sign words ("1-bit Bonsai 27B" model card: the
// weights are used packed and never expanded back to FP16; the CUDA kernel unpacks the sign
// codes inside the matmul and applies the group scales).  Decode is the memory-bound phase
// (model card, cross-platform throughput), so the kernels are organised around streaming the
// 1.125 bits/weight from HBM once, with as few VALU operations per weight as possible: the
// signs of four weights index a table of the 16 signed sums of their x values.
//
// Two kernels share the method: one for small N (a row tile per CU, the tile's waves splitting
// K) and a persistent one for large N (tables built once per CU).  Weight bytes reach LDS by
// direct global->LDS loads of whole lines.  K too long for their tables in LDS, and two to eight
// rows of x (M = 2..8), go to the matrix-core GEMV instead (gemv_mfma.hip).
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

constexpr int kLutBytes = 32 * 16 * 4;              // 2 KB of tables per group

// 16-byte LDS store at addr, issued from asm: the compiler cannot tell it apart from the LDS
// the in-flight direct global->LDS copies write, and would otherwise wait for every copy
// (s_waitcnt vmcnt(0)) before the first such store.  Callers order it with explicit waits.
__device__ __forceinline__ void lds_store_b128(uint32_t addr, u32x4 v)
{
    asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// Up to mid N: one tile of ROWS = 64 or 32 rows per workgroup.  A wave owns GPW = GPL * 64 / ROWS
// consecutive groups of the tile's rows: lane l takes row l % ROWS and the GPL groups
// GPL (l / ROWS) .. + GPL - 1 of the wave's.  With GPL = 4 every wave has a single 4 KB tile
// copy and 128 lookups per lane after it lands, whatever ROWS; 32-row tiles spread a small N
// over twice the CUs, at the price of tables for twice the groups per wave.  GPL = 2 (32-row
// tiles) halves each wave's share, so a workgroup has twice the waves and spreads them more
// evenly over the CU's four SIMDs (10 waves go 3-3-2-2, where 5 went 2-1-1-1).  The waves'
// partial sums meet in LDS and are added in a fixed order.
//
// Everything a wave needs reaches its LDS by direct global->LDS copies, issued in this order:
// its x values, the weight tile, the scales.  Copies complete in issue order, so waiting until
// at most the tile's and the scales' copies are outstanding means x has landed: the wave builds
// its tables while the tile is still on its way from HBM.  (Read through the compiler, x would
// wait for every copy: it cannot tell the copies' LDS writes from the table writes, and orders
// loads of mixed kinds by waiting for all of them.)
// AFF: affine 1-bit weights (MLX's form, a scale a and a bias b per group, weight a q + b for
// the bit q; "1-bit Bonsai 27B" model card, "MLX packaging").  With D the group's table sum of
// +-x and X the group's plain sum of x, the group contributes a sum(q x) + b X =
// (a / 2) D + (a / 2 + b) X.  X is the same for every row: each wave adds up its groups' x from
// the quads its lanes already hold (one lane of the four that hold a quad), across the wave.
// GPL: groups per lane (4, or 2 for 32-row tiles: twice the waves, each half the work, so that
// the waves spread more evenly over a CU's four SIMDs).
template <int ROWS, bool AFF = false, int GPL = 4>
struct L4 {
    static constexpr int lpr = 64 / ROWS;               // lanes per row
    static constexpr int gpw = GPL * lpr;               // groups per wave
    static_assert(gpw >= 4 && gpw <= 8, "a wave's x (gpw * 256 B) is staged by whole 1 KB copies");
    static constexpr int tile = ROWS * gpw * 16;        // 4 KB of cells (2 KB at GPL 2)
    static constexpr int lut = gpw * kLutBytes;         // tables; x is staged in the first gpw * 256 B
    static constexpr int scales = ROWS * gpw * 4;       // 1 KB: one dword per (row, group) at most;
                                                        // the wave's partial sums once the lookups end
                                                        // (AFF: the biases follow, laid out alike)
    static constexpr int wave = tile + lut + (AFF ? 2 : 1) * scales;   // 13 / 14 KB (ROWS 64), 21 / 22 (32)
    static constexpr int max_waves = (160 * 1024) / wave;   // 12 / 11 or 7
    static constexpr int rows_per_copy = 1024 / (gpw * 16);  // tile rows per 1 KB copy
    // the 16-byte cell of (row r, group u) sits at gpw * 16 * r + 16 (u ^ swz(r))
    static __device__ __forceinline__ int swz(int r) { return (r / (16 / gpw)) & (gpw - 1); }
};

// Ordering point for the compiler only: no memory access moves across it.
__device__ __forceinline__ void compiler_fence() { asm volatile("" : : : "memory"); }

// Eight 8-byte LDS reads at addr + 128 k (k < 8), after WAIT (an s_waitcnt, or nothing), and
// waited for in the same block.
#define BONSAI_L4_XREAD8(WAIT, Q, ADDR)                                                                \
    asm volatile(WAIT "ds_read_b64 %0, %8\n\tds_read_b64 %1, %8 offset:128\n\t"                        \
                 "ds_read_b64 %2, %8 offset:256\n\tds_read_b64 %3, %8 offset:384\n\t"                  \
                 "ds_read_b64 %4, %8 offset:512\n\tds_read_b64 %5, %8 offset:640\n\t"                  \
                 "ds_read_b64 %6, %8 offset:768\n\tds_read_b64 %7, %8 offset:896\n\t"                  \
                 "s_waitcnt lgkmcnt(0)"                                                                \
                 : "=&v"((Q)[0]), "=&v"((Q)[1]), "=&v"((Q)[2]), "=&v"((Q)[3]), "=&v"((Q)[4]),          \
                   "=&v"((Q)[5]), "=&v"((Q)[6]), "=&v"((Q)[7])                                         \
                 : "v"(ADDR)                                                                           \
                 : "memory")

// PAIRS: G is even, so the scales of groups 2p, 2p + 1 of a row are one aligned dword.
// AFF: affine weights (biases used only then).  GPL: groups per lane (see L4).
template <int ROWS, bool PAIRS, bool AFF, int GPL>
__global__ __launch_bounds__((L4<ROWS, AFF, GPL>::max_waves * 64)) void q1_gemv_lut4_kernel(
    const uint32_t *__restrict__ wbits, const uint16_t *__restrict__ scales, const uint16_t *__restrict__ biases,
    const uint16_t *__restrict__ x, float *__restrict__ y, int N, int K)
{
    using L = L4<ROWS, AFF, GPL>;
    extern __shared__ u32x4 lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int G = K >> 7;
    const int g0 = wave * L::gpw, g1 = min(G, g0 + L::gpw), gl = g1 - 1;
    const int r = lane % ROWS, h = lane / ROWS;             // this lane's row and group block
    const int n0 = blockIdx.x * ROWS;
    char *const tile = reinterpret_cast<char *>(lds) + wave * L::wave;
    char *const lut = tile + L::tile;
    char *const sc = lut + L::lut;
    char *const bc = sc + L::scales;                         // biases (AFF only)
    float *const part = reinterpret_cast<float *>(sc);

    // x: copy j, lane l brings x[128 g0 + 512 j + 8 l .. + 7] to lut + 1 KB j + 16 l (clamped
    // inside x past K)
    const u32x4 *xg = reinterpret_cast<const u32x4 *>(x);
#pragma unroll
    for (int j = 0; j < L::gpw / 4; ++j)
        __builtin_amdgcn_global_load_lds((glb_void_t *)(xg + min(16 * g0 + 64 * j + lane, 16 * G - 1)),
                                         (lds_void_t *)(lut + 1024 * j), 16, 0, 0);
    compiler_fence();
    // tile: copy k covers rows rows_per_copy * k + lane / gpw, one 16-byte cell per lane
    const u32x4 *wg = reinterpret_cast<const u32x4 *>(wbits);
#pragma unroll
    for (int k = 0; k < L::tile / 1024; ++k) {
        const int rr = L::rows_per_copy * k + lane / L::gpw;
        const int gg = min(g0 + ((lane % L::gpw) ^ L::swz(rr)), gl);
        __builtin_amdgcn_global_load_lds((glb_void_t *)(wg + (size_t)min(n0 + rr, N - 1) * G + gg),
                                         (lds_void_t *)(tile + k * 1024), 16, 0, 0);
    }
    // scales: element d = 64 k + lane of copy k is (row d % ROWS, pair d / ROWS) for PAIRS
    // (4 bytes), else (row d % ROWS, group d / ROWS) (2 bytes, the low half of its dword); it
    // lands in the dword at sc + 4 d
    // (AFF: the biases likewise, to bc)
    constexpr int kScaleCopies = (PAIRS ? ROWS * L::gpw / 2 : ROWS * L::gpw) / 64;
#pragma unroll
    for (int which = 0; which < (AFF ? 2 : 1); ++which) {
        const uint16_t *const src = which ? biases : scales;
        char *const dst = which ? bc : sc;
#pragma unroll
        for (int k = 0; k < kScaleCopies; ++k) {
            const int d = 64 * k + lane;
            const size_t rbase = (size_t)min(n0 + d % ROWS, N - 1) * G;
            if constexpr (PAIRS)
                __builtin_amdgcn_global_load_lds((glb_void_t *)(src + rbase + min(g0 + 2 * (d / ROWS), G - 2)),
                                                 (lds_void_t *)(dst + 256 * k), 4, 0, 0);
            else
                __builtin_amdgcn_global_load_lds((glb_void_t *)(src + rbase + min(g0 + d / ROWS, gl)),
                                                 (lds_void_t *)(dst + 256 * k), 2, 0, 0);
        }
    }
    compiler_fence();

    // x quads: quad k of this lane is x[128 g0 + 64 k + 4 (lane / 4) .. + 3], at
    // lut + 128 k + 8 (lane / 4); the first block waits until at most the tile, scale (and
    // bias) copies are in flight
    constexpr int kQuads = 2 * L::gpw;
    uint2 xq[kQuads];
    const uint32_t xa = (uint32_t)(uintptr_t)((lds_char_t *)lut) + 8 * (lane >> 2);
    constexpr int kAfterX = L::tile / 1024 + (AFF ? 2 : 1) * kScaleCopies;   // copies issued after x
    static_assert(kAfterX == 3 || kAfterX == 4 || kAfterX == 6 || kAfterX == 8 || kAfterX == 12);
    if constexpr (kAfterX == 3) BONSAI_L4_XREAD8("s_waitcnt vmcnt(3)\n\t", xq, xa);
    else if constexpr (kAfterX == 4) BONSAI_L4_XREAD8("s_waitcnt vmcnt(4)\n\t", xq, xa);
    else if constexpr (kAfterX == 6) BONSAI_L4_XREAD8("s_waitcnt vmcnt(6)\n\t", xq, xa);
    else if constexpr (kAfterX == 8) BONSAI_L4_XREAD8("s_waitcnt vmcnt(8)\n\t", xq, xa);
    else BONSAI_L4_XREAD8("s_waitcnt vmcnt(12)\n\t", xq, xa);
    if constexpr (kQuads == 16) BONSAI_L4_XREAD8("", xq + 8, xa + 1024);

    // AFF: X of the wave's group u is the sum of quads 2u, 2u + 1 over the 16 values of lane / 4;
    // lanes with lane % 4 == 0 contribute, and a fixed butterfly adds them across the wave.
    // Groups 0..3 and 4..7 are kept apart (xs0, xs1): a select between one array's elements by
    // the lane's h would become a dynamically indexed, scratch-resident array.
    float xs0[4] = {0.f, 0.f, 0.f, 0.f}, xs1[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (AFF) {
#pragma unroll
        for (int u = 0; u < L::gpw; ++u) {
            float t = 0.f;
#pragma unroll
            for (int k = 2 * u; k < 2 * u + 2; ++k) {
                const half2_t p01 = as_half2(xq[k].x), p23 = as_half2(xq[k].y);
                t += ((float)p01[0] + (float)p01[1]) + ((float)p23[0] + (float)p23[1]);
            }
            t = (lane & 3) == 0 ? t : 0.f;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
            if (u < 4) xs0[u] = t;
            else xs1[u & 3] = t;
        }
    }

    // tables: lane builds quads e = lane + 64 k of the wave's groups (group e / 128, chunk
    // (e / 4) % 32, entries 4 bt .. 4 bt + 3); they overwrite the staged x, which this wave
    // alone has read, and whose reads have completed
    const uint32_t lut_lane = (uint32_t)(uintptr_t)((lds_char_t *)lut) + 16 * lane;
#pragma unroll
    for (int k = 0; k < kQuads; ++k) {
        const int bt = lane & 3;                    // quad e = lane + 64 k: bt = e % 4
        const half2_t p01 = as_half2(xq[k].x), p23 = as_half2(xq[k].y);
        const float x0 = (float)p01[0], x1 = (float)p01[1];
        const float sg2 = (bt & 1) ? 1.f : -1.f, sg3 = (bt & 2) ? 1.f : -1.f;
        const float base = fmaf(sg3, (float)p23[1], fmaf(sg2, (float)p23[0], -x0 - x1));
        u32x4 ev;
        ev[0] = __builtin_bit_cast(uint32_t, base);                                 // v = 4bt
        ev[1] = __builtin_bit_cast(uint32_t, fmaf(2.f, x0, base));                 // v = 4bt + 1
        ev[2] = __builtin_bit_cast(uint32_t, fmaf(2.f, x1, base));                 // v = 4bt + 2
        ev[3] = __builtin_bit_cast(uint32_t, fmaf(2.f, x1, fmaf(2.f, x0, base)));  // v = 4bt + 3
        // quad e sits at lut + (e / 128) * 2 KB + 64 ((e / 4) % 32) + 16 (e % 4) = lut + 16 lane + 1 KB * k
        lds_store_b128(lut_lane + 1024 * k, ev);
    }
    vm_wait<0>();                                   // the tile and the scales landed
    lgkm_wait0();                                   // this wave's tables are written

    // this lane's scales (and biases) (row r, groups GPL h .. GPL h + GPL - 1 of the wave's),
    // before the lookups
    constexpr int kSw = PAIRS ? GPL / 2 : GPL;
    uint32_t sw[kSw], bw[AFF ? kSw : 1];
#pragma unroll
    for (int k = 0; k < kSw; ++k) {
        const int off = 4 * (kSw * h + k) * ROWS + 4 * r;
        sw[k] = *reinterpret_cast<const uint32_t *>(sc + off);
        if constexpr (AFF) bw[k] = *reinterpret_cast<const uint32_t *>(bc + off);
    }

    const uint32_t mask_3c = __builtin_amdgcn_readfirstlane(0x3Cu);
    // the tables of this lane's GPL groups start at lut + GPL * 2 KB * h (256-aligned)
    const uint32_t lut_addr = (uint32_t)(uintptr_t)((lds_char_t *)lut) + GPL * kLutBytes * h;
    uint32_t raddr[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) raddr[j] = lut_addr;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < GPL; ++u) {
        const int ug = GPL * h + u;                 // group of the wave's slice
        const u32x4 q = *reinterpret_cast<const u32x4 *>(tile + L::gpw * 16 * r + 16 * (ug ^ L::swz(r)));
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
        const uint16_t sbits = (uint16_t)(PAIRS ? sw[u >> 1] >> (16 * (u & 1)) : sw[u]);
        // groups past K (the last wave's slice may be short) count with scale 0
        const bool live = g0 + ug < g1;
        if constexpr (AFF) {
            const uint16_t bbits = (uint16_t)(PAIRS ? bw[u >> 1] >> (16 * (u & 1)) : bw[u]);
            const float ha = live ? 0.5f * f16_bits_to_f32(sbits) : 0.f;          // a / 2
            const float hb = live ? ha + f16_bits_to_f32(bbits) : 0.f;           // a / 2 + b
            // X of this lane's group GPL h + u of the wave's
            float xu;
            if constexpr (L::gpw == 8) xu = h ? xs1[u] : xs0[u];
            else if constexpr (GPL == 4) xu = xs0[u];
            else xu = h ? xs0[2 + u] : xs0[u];
            acc = fmaf(ha, (a0 + a1) + (a2 + a3), acc);
            acc = fmaf(hb, xu, acc);
        } else {
            const float s = live ? f16_bits_to_f32(sbits) : 0.f;
            acc = fmaf(s, (a0 + a1) + (a2 + a3), acc);
        }
    }
    part[lane] = acc;                               // the scales were read before the lookups
    __syncthreads();
    if (wave == 0 && lane < ROWS && n0 + lane < N) {
        float t = 0.f;
        for (int w = 0; w < nwaves; ++w) {
            const float *pw = reinterpret_cast<const float *>(reinterpret_cast<char *>(lds) + w * L::wave + L::tile + L::lut);
#pragma unroll
            for (int hh = 0; hh < L::lpr; ++hh) t += pw[hh * ROWS + lane];
        }
        y[n0 + lane] = t;
    }
}

template <int ROWS, bool AFF, int GPL = 4>
hipError_t launch_lut4(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases, const uint16_t *x,
                       float *y, int N, int K, hipStream_t stream)
{
    using L = L4<ROWS, AFF, GPL>;
    const int G = K / 128;
    const int tiles = (N + ROWS - 1) / ROWS;
    const int waves = (G + L::gpw - 1) / L::gpw;
    const size_t lds = (size_t)waves * L::wave;
    const bool pairs = (G % 2) == 0;                // a row's scale pairs are then dword aligned
    const void *fn = pairs ? reinterpret_cast<const void *>(&q1_gemv_lut4_kernel<ROWS, true, AFF, GPL>)
                           : reinterpret_cast<const void *>(&q1_gemv_lut4_kernel<ROWS, false, AFF, GPL>);
    if (!set_lds_limit(fn, L::max_waves * L::wave)) return hipErrorInvalidValue;
    void *args[] = {&wbits, &scales, &biases, &x, &y, &N, &K};
    return launch_kernel(fn, __PRETTY_FUNCTION__, dim3(tiles), dim3(64 * waves), args, lds, stream);
}

// ---- M = 1, large N: persistent workgroups, tables built once ------------------------------
//
// With many row tiles, rebuilding the tables for every tile costs as much VALU work as the
// lookups.  Here one workgroup per CU builds the tables of every group of K once (2 KB per
// group, shared by its waves) and each wave then owns whole 64-row tiles: wave gw of the W
// waves in the grid takes tiles gw, gw + W, ..., and lane r accumulates row r over all of K,
// so no partial sums cross waves (gw numbers the waves wave-major, gw = wave * grid + block,
// so that fewer tiles than waves still spread over every CU).  A tile goes past in batches of 4 groups (64 rows x 64 B of
// sign words and the rows' scales), double buffered in the wave's LDS: the copies of batch
// i + 1 are in flight while batch i is looked up.  Every iteration issues exactly one batch's
// copies (past the wave's last batch, that batch again), so one wait with a fixed count finds
// the older batch landed.
// AFF: affine 1-bit weights, as in the tile kernels: the biases travel with the scales, and X,
// the plain sum of x over each group, is added up once per workgroup while the tables are built
// (held in LDS beside them); a group then contributes (a / 2) D + (a / 2 + b) X.
constexpr int kLPGroups = 4;
constexpr int kLPTile = 64 * kLPGroups * 16;        // 4 KB of cells per batch
constexpr int kLPScales = 64 * kLPGroups * 4;       // 1 KB: one dword per (row, group) at most
constexpr int kLPBuf = kLPTile + kLPScales;         // 5 KB; buffer 1 first stages the wave's x
constexpr int kLPMaxWaves = 8;
constexpr int kLPMaxPer = kLPBuf / 256;             // groups of x one buffer can stage
// buffer bytes (AFF: the biases follow the scales) and the LDS bytes for X of every group
constexpr int lp_buf(bool aff) { return aff ? kLPBuf + kLPScales : kLPBuf; }
constexpr int lp_xsum_bytes(int GT, bool aff) { return aff ? (4 * GT + 15) / 16 * 16 : 0; }

template <bool PAIRS, bool AFF>
__global__ __launch_bounds__(kLPMaxWaves * 64) void q1_gemv_lutp_kernel(const uint32_t *__restrict__ wbits,
                                                                        const uint16_t *__restrict__ scales,
                                                                        const uint16_t *__restrict__ biases,
                                                                        const uint16_t *__restrict__ x,
                                                                        float *__restrict__ y, int N, int K)
{
    constexpr int BUF = lp_buf(AFF);
    extern __shared__ u32x4 lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int G = K >> 7;
    const int nb = (G + kLPGroups - 1) / kLPGroups;         // batches per tile
    const int GT = kLPGroups * nb;                          // groups with tables (past G: scale 0)
    char *const tables = reinterpret_cast<char *>(lds);     // group g at tables + 2 KB g
    float *const xsum = reinterpret_cast<float *>(tables + GT * kLutBytes);   // AFF: X of group g
    char *const bufs = tables + GT * kLutBytes + lp_xsum_bytes(GT, AFF) + wave * (2 * BUF);
    const int tiles = (N + 63) / 64;
    const int W = gridDim.x * nwaves;
    const int gw = wave * gridDim.x + blockIdx.x;
    const int nbat = (gw < tiles ? (tiles - 1 - gw) / W + 1 : 0) * nb;     // this wave's batches
    const u32x4 *wg = reinterpret_cast<const u32x4 *>(wbits);
    constexpr int kCopies = 4 + (PAIRS ? 2 : 4) * (AFF ? 2 : 1);   // copies per batch

    // batch i of this wave (tile i / nb, groups 4 (i % nb) ..) into buffer i % 2
    auto issue = [&](int i) {
        const int ic = min(i, max(nbat - 1, 0));
        const int n0 = (gw + W * (ic / nb)) * 64;           // rows clamp to N - 1 (a wave without tiles too)
        const int g0 = kLPGroups * (ic % nb);
        char *const buf = bufs + (i & 1) * BUF;
        // cells: copy k covers rows 16 k .. 16 k + 15, 4 lanes per row; cell (r, u) at 64 r + 16 (u ^ ((r >> 2) & 3))
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = 16 * k + (lane >> 2);
            const int gg = min(g0 + ((lane & 3) ^ ((r >> 2) & 3)), G - 1);
            __builtin_amdgcn_global_load_lds((glb_void_t *)(wg + (size_t)min(n0 + r, N - 1) * G + gg),
                                             (lds_void_t *)(buf + 1024 * k), 16, 0, 0);
        }
        // scales of row `lane`: PAIRS, copy p brings groups g0 + 2p, g0 + 2p + 1 as the dword at
        // buf + 4 KB + 256 p + 4 lane; else copy u brings group g0 + u as that dword's low half
        // (AFF: the biases likewise, 1 KB further)
        const size_t rbase = (size_t)min(n0 + lane, N - 1) * G;
#pragma unroll
        for (int which = 0; which < (AFF ? 2 : 1); ++which) {
            const uint16_t *const src = which ? biases : scales;
            char *const dst = buf + kLPTile + kLPScales * which;
#pragma unroll
            for (int k = 0; k < (PAIRS ? 2 : 4); ++k) {
                if constexpr (PAIRS)
                    __builtin_amdgcn_global_load_lds((glb_void_t *)(src + rbase + min(g0 + 2 * k, G - 2)),
                                                     (lds_void_t *)(dst + 256 * k), 4, 0, 0);
                else
                    __builtin_amdgcn_global_load_lds((glb_void_t *)(src + rbase + min(g0 + k, G - 1)),
                                                     (lds_void_t *)(dst + 256 * k), 2, 0, 0);
            }
        }
    };

    // tables: this wave builds groups [ga, gb) from their x, staged in its buffer 1: copy j,
    // lane l brings x[128 ga + 512 j + 8 l .. + 7] (clamped inside x) to buffer 1 + 1 KB j + 16 l
    const int per = (GT + nwaves - 1) / nwaves;             // at most kLPMaxPer (host check)
    const int ga = min(GT, wave * per), gb = min(GT, ga + per);
    char *const xs = bufs + BUF;
    const u32x4 *xg = reinterpret_cast<const u32x4 *>(x);
    for (int j = 0; j < (gb - ga + 3) / 4; ++j)
        __builtin_amdgcn_global_load_lds((glb_void_t *)(xg + min(16 * ga + 64 * j + lane, 16 * G - 1)),
                                         (lds_void_t *)(xs + 1024 * j), 16, 0, 0);
    compiler_fence();
    issue(0);
    compiler_fence();

    // quad k of this lane: group ga + k / 2, chunk 16 (k % 2) + lane / 4, entries 4 bt .. + 3
    // (bt = lane % 4), from x[128 ga + 64 k + 4 (lane / 4) .. + 3] at xs + 128 k + 8 (lane / 4);
    // it goes to tables + 2 KB ga + 1 KB k + 16 lane.  Quads are read 8 at a time, the first
    // eight once at most batch 0's copies are in flight.
    const uint32_t xa = (uint32_t)(uintptr_t)((lds_char_t *)xs) + 8 * (lane >> 2);
    const uint32_t tl = (uint32_t)(uintptr_t)((lds_char_t *)tables) + kLutBytes * ga + 16 * lane;
    const int nq = 2 * (gb - ga);
    for (int kb = 0; kb < nq; kb += 8) {
        uint2 xq[8];
        if (kb == 0) {
            // x landed once at most batch 0's copies are in flight
            if constexpr (kCopies == 6) BONSAI_L4_XREAD8("s_waitcnt vmcnt(6)\n\t", xq, xa);
            else if constexpr (kCopies == 8) BONSAI_L4_XREAD8("s_waitcnt vmcnt(8)\n\t", xq, xa);
            else BONSAI_L4_XREAD8("s_waitcnt vmcnt(12)\n\t", xq, xa);
        } else {
            BONSAI_L4_XREAD8("", xq, xa + 128 * kb);
        }
        const int bt = lane & 3;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (kb + k >= nq) break;
            const half2_t p01 = as_half2(xq[k].x), p23 = as_half2(xq[k].y);
            const float x0 = (float)p01[0], x1 = (float)p01[1];
            const float sg2 = (bt & 1) ? 1.f : -1.f, sg3 = (bt & 2) ? 1.f : -1.f;
            const float base = fmaf(sg3, (float)p23[1], fmaf(sg2, (float)p23[0], -x0 - x1));
            u32x4 ev;
            ev[0] = __builtin_bit_cast(uint32_t, base);                                 // v = 4bt
            ev[1] = __builtin_bit_cast(uint32_t, fmaf(2.f, x0, base));                 // v = 4bt + 1
            ev[2] = __builtin_bit_cast(uint32_t, fmaf(2.f, x1, base));                 // v = 4bt + 2
            ev[3] = __builtin_bit_cast(uint32_t, fmaf(2.f, x1, fmaf(2.f, x0, base)));  // v = 4bt + 3
            lds_store_b128(tl + 1024 * (kb + k), ev);
        }
        if constexpr (AFF) {
            // X of groups ga + (kb + k) / 2 (quads k, k + 1): one lane of the four that hold a
            // quad contributes, and a fixed butterfly adds across the wave
#pragma unroll
            for (int k = 0; k < 8; k += 2) {
                if (kb + k >= nq) break;
                float t = 0.f;
#pragma unroll
                for (int kk = k; kk < k + 2; ++kk) {
                    const half2_t p01 = as_half2(xq[kk].x), p23 = as_half2(xq[kk].y);
                    t += ((float)p01[0] + (float)p01[1]) + ((float)p23[0] + (float)p23[1]);
                }
                t = (lane & 3) == 0 ? t : 0.f;
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
                if (lane == 0) xsum[ga + (kb + k) / 2] = t;
            }
        }
    }
    issue(1);                                       // buffer 1: its staged x has been read
    lgkm_wait0();                                   // this wave's tables are written ...
    asm volatile("s_barrier" : : : "memory");       // ... and every wave's

    const uint32_t mask_3c = __builtin_amdgcn_readfirstlane(0x3Cu);
    const uint32_t tbase = (uint32_t)(uintptr_t)((lds_char_t *)tables);
    float acc = 0.f;
    int b = 0, t = gw;                              // batch of the tile, tile
    for (int i = 0; i < nbat; ++i) {
        vm_wait<kCopies>();                         // batch i landed; batch i + 1 may be in flight
        const char *buf = bufs + (i & 1) * BUF;
        uint32_t sw[PAIRS ? 2 : 4], bw[AFF ? (PAIRS ? 2 : 4) : 1];
#pragma unroll
        for (int k = 0; k < (PAIRS ? 2 : 4); ++k) {
            sw[k] = *reinterpret_cast<const uint32_t *>(buf + kLPTile + 256 * k + 4 * lane);
            if constexpr (AFF) bw[k] = *reinterpret_cast<const uint32_t *>(buf + kLPTile + kLPScales + 256 * k + 4 * lane);
        }
        // tables of groups 4 b .. 4 b + 3 start at tbase + 8 KB b (256-aligned)
        uint32_t raddr[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) raddr[j] = tbase + 4 * kLutBytes * b;
#pragma unroll
        for (int u = 0; u < kLPGroups; ++u) {
            const u32x4 q = *reinterpret_cast<const u32x4 *>(buf + 64 * lane + 16 * (u ^ ((lane >> 2) & 3)));
            float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
            for (int i2 = 0; i2 < 4; i2 += 2) {
                word_addrs(q[i2], &raddr[0], mask_3c);
                word_addrs(q[i2 + 1], &raddr[8], mask_3c);
                float tv[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) tv[j] = lds_f32(raddr[j], u * kLutBytes + 64 * (8 * i2 + j));
                a0 += (tv[0] + tv[1]) + (tv[2] + tv[3]);
                a1 += (tv[4] + tv[5]) + (tv[6] + tv[7]);
                a2 += (tv[8] + tv[9]) + (tv[10] + tv[11]);
                a3 += (tv[12] + tv[13]) + (tv[14] + tv[15]);
            }
            const uint16_t sbits = (uint16_t)(PAIRS ? sw[u >> 1] >> (16 * (u & 1)) : sw[u]);
            const bool live = kLPGroups * b + u < G;
            if constexpr (AFF) {
                const uint16_t bbits = (uint16_t)(PAIRS ? bw[u >> 1] >> (16 * (u & 1)) : bw[u]);
                const float ha = live ? 0.5f * f16_bits_to_f32(sbits) : 0.f;          // a / 2
                const float hb = live ? ha + f16_bits_to_f32(bbits) : 0.f;           // a / 2 + b
                acc = fmaf(ha, (a0 + a1) + (a2 + a3), acc);
                acc = fmaf(hb, xsum[kLPGroups * b + u], acc);
            } else {
                const float s = live ? f16_bits_to_f32(sbits) : 0.f;
                acc = fmaf(s, (a0 + a1) + (a2 + a3), acc);
            }
        }
        if (++b == nb) {                            // the tile is complete
            const int row = 64 * t + lane;
            if (row < N) y[row] = acc;
            acc = 0.f;
            b = 0;
            t += W;
        }
        lgkm_wait0();                               // this buffer's reads are done before it refills
        issue(i + 2);
    }
    vm_wait<0>();                                   // no copy into LDS outlives the wave
}

template <bool AFF>
size_t lutp_lds(int G, int nwaves)
{
    const int GT = 4 * ((G + 3) / 4);
    return (size_t)kLutBytes * GT + lp_xsum_bytes(GT, AFF) + (size_t)nwaves * 2 * lp_buf(AFF);
}

// Waves per workgroup for the persistent kernel (0: the tables of K do not fit the LDS).
template <bool AFF = false>
int lutp_waves(int G)
{
    const int GT = 4 * ((G + 3) / 4);
    const long room = 160L * 1024 - (long)kLutBytes * GT - lp_xsum_bytes(GT, AFF);
    int nw = room > 0 ? (int)(room / (2 * lp_buf(AFF))) : 0;
    if (nw > kLPMaxWaves) nw = kLPMaxWaves;
    if (nw < 4 || (GT + nw - 1) / nw > lp_buf(AFF) / 256) return 0;
    return nw;
}

template <bool AFF = false>
hipError_t launch_lutp(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases, const uint16_t *x,
                       float *y, int N, int K, int nwaves, hipStream_t stream)
{
    const int G = K / 128;
    const int tiles = (N + 63) / 64;
    const int grid = min(device_cus(), (tiles + nwaves - 1) / nwaves);
    const size_t lds = lutp_lds<AFF>(G, nwaves);
    const bool pairs = (G % 2) == 0;
    const void *fn = pairs ? reinterpret_cast<const void *>(&q1_gemv_lutp_kernel<true, AFF>)
                           : reinterpret_cast<const void *>(&q1_gemv_lutp_kernel<false, AFF>);
    if (!set_lds_limit(fn, kLdsPerCu)) return hipErrorInvalidValue;
    void *args[] = {&wbits, &scales, &biases, &x, &y, &N, &K};
    return launch_kernel(fn, __PRETTY_FUNCTION__, dim3(grid), dim3(64 * nwaves), args, lds, stream);
}

#undef BONSAI_L4_XREAD8

}  // namespace

// Affine 1-bit weights, one row of x, on the table kernels: the binary routes of
// launch_q1_gemv, with the persistent kernel only where K is long (below).
bool q1a_lut_fits(int N, int K)
{
    const int G = K / 128;
    const bool fits32 = (G + L4<32, true, 2>::gpw - 1) / L4<32, true, 2>::gpw <= L4<32, true, 2>::max_waves ||
                        (G + L4<32, true>::gpw - 1) / L4<32, true>::gpw <= L4<32, true>::max_waves;
    const bool fits64 = (G + L4<64, true>::gpw - 1) / L4<64, true>::gpw <= L4<64, true>::max_waves;
    // 64-row tiles at any N (they beat the matrix-core kernel at every N timed), and the
    // persistent kernel, whose tables fit a little further in K
    return (fits32 && ((int64_t)N + 31) / 32 <= device_cus()) || fits64 || lutp_waves<true>(G) != 0;
}

hipError_t launch_q1a_lut(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases, const uint16_t *x,
                          float *y, int N, int K, hipStream_t stream)
{
    // as the binary route: byte tables for many rows, 32-row tiles while one round of the CUs
    // holds them, with two groups per lane where their waves fit, then 64-row tiles
    const int G = K / 128;
    const int cus = device_cus();
    if ((int64_t)N >= 600LL * cus && G >= 16 && lut8a_fits(N, K))
        return launch_lut8a(wbits, scales, biases, x, y, N, K, stream);
    const bool one_round32 = ((int64_t)N + 31) / 32 <= cus;
    using A2 = L4<32, true, 2>;
    if (one_round32 && (G + A2::gpw - 1) / A2::gpw <= A2::max_waves)
        return launch_lut4<32, true, 2>(wbits, scales, biases, x, y, N, K, stream);
    const bool fits32 = (G + L4<32, true>::gpw - 1) / L4<32, true>::gpw <= L4<32, true>::max_waves;
    if (fits32 && one_round32) return launch_lut4<32, true>(wbits, scales, biases, x, y, N, K, stream);
    if (!q1a_lut_fits(N, K)) return hipErrorInvalidValue;
    // past six rounds of 64-row tiles the persistent kernel, except for short K at moderate N
    // (timed: K = 5120, N = 248320: 65 us against 90 for the tiles; K = 2560 and 3072 at
    // N = 100003 ... 248320: 18-39 us against 24-65; K = 1152 and 2048: the tiles lead by about
    // 1 us up to N = 160000 and trail by 2.5 us at 248320)
    const int64_t tiles64 = ((int64_t)N + 63) / 64;
    const bool persist = tiles64 > 6 * cus && (G >= 20 || tiles64 > 12 * cus);
    const bool fits64 = (G + L4<64, true>::gpw - 1) / L4<64, true>::gpw <= L4<64, true>::max_waves;
    if (fits64 && !persist)
        return launch_lut4<64, true>(wbits, scales, biases, x, y, N, K, stream);
    if (const int nw = lutp_waves<true>(G)) return launch_lutp<true>(wbits, scales, biases, x, y, N, K, nw, stream);
    return launch_lut4<64, true>(wbits, scales, biases, x, y, N, K, stream);
}

hipError_t launch_q1_gemv(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x, float *y,
                          int M, int N, int K, hipStream_t stream)
{
    if (M >= 2 && M <= 8) return launch_gemv_mfma(false, wbits, scales, x, y, M, N, K, stream);
    if (M != 1) return hipErrorInvalidValue;
    // The route follows measurements at K = 5120 (N = 1024 ... 248320) and K = 13824:
    // - 32-row tiles while one round of the CUs holds them (twice the CUs of 64-row tiles), with
    //   two groups per lane where the waves fit (10 waves instead of 5 at K = 5120, 5120 x 5120:
    //   4.4 us instead of 5.3);
    // - 64-row tiles (one workgroup per CU, about 5 us a round) up to six rounds;
    // - beyond, the persistent kernel: about 15 us up front for the tables of all of K on every
    //   CU, then about 0.15 ns a row, so it overtakes near 100k rows.  Shorter K fits two or
    //   more tiles' workgroups on a CU and builds fewer tables per tile, so there the tiles keep
    //   the lead further: with K/128 < 28 they won at every N timed up to 200k rows (K = 1152 ...
    //   3072: by 1 to 3.5 us), and below 16 up to 248320 as well;
    // - K too long for any of their tables in LDS: the matrix-core kernel, which measured 9.6 us
    //   against 15.7 for a table-lookup kernel that stages K in batches (N = 5120, K = 13824).
    const int G = K / 128;
    using L32 = L4<32, false, 2>;
    const bool fits32 = (G + L32::gpw - 1) / L32::gpw <= L32::max_waves;
    const bool fits64 = (G + L4<64>::gpw - 1) / L4<64>::gpw <= L4<64>::max_waves;
    const int64_t tiles64 = ((int64_t)N + 63) / 64;
    const int cus = device_cus();
    // - many rows (the LM head): byte tables, rebuilt per 1024 k on every CU, which halve the
    //   lookups of the nibble tables (K = 5120: 248320 rows in 36 us against 51 us; they tie
    //   near 131072 rows, below which the rebuilds cost more than the lookups they save)
    if ((int64_t)N >= 600LL * cus && G >= 16 && lut8_fits(N, K)) return launch_lut8(wbits, scales, x, y, N, K, stream);
    if (fits32 && ((int64_t)N + 31) / 32 <= cus) return launch_lut4<32, false, 2>(wbits, scales, nullptr, x, y, N, K, stream);
    const bool persist = tiles64 > 6 * cus && (G >= 28 || (G >= 16 && tiles64 > 14 * cus));
    if (fits64 && !persist) return launch_lut4<64, false>(wbits, scales, nullptr, x, y, N, K, stream);
    if (const int nw = lutp_waves(G)) return launch_lutp(wbits, scales, nullptr, x, y, N, K, nw, stream);
    if (fits64) return launch_lut4<64, false>(wbits, scales, nullptr, x, y, N, K, stream);
    return launch_gemv_mfma(false, wbits, scales, x, y, M, N, K, stream);
}

}  // namespace bonsai
