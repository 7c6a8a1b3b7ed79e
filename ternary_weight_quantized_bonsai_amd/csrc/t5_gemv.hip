// t5_gemv.hip -- small-M matmul on base-3 ternary weights (five trits per byte), matrix cores.
//
// Ternary weights ({-1, 0, +1} x the FP16 group scale; "Ternary Bonsai 27B" article, ternary
// format) need log2(3) bits each; the article's limitations section notes that the current
// release stores them in 2 bits and that native-density storage is still to come.  This
// library's base-3 layout gets within 1 % of that bound: a row is a run of 32-byte superblocks
// of 160 weights, and byte c of a superblock holds the weights k = c + 32 i (i = 0..4) as the
// base-3 number sum_i d_i 3^i with d = w mod 3.  That is 1.6 bits per weight, 1.725 with the
// scales, against 2.125 for the 2-bit codes.
//
// Why this order.  v_mfma_f32_16x16x32_f16 takes 32 k per instruction; a lane (row i = lane %
// 16, quarter q = lane / 16) supplies 8 of them.  With digit i of byte c standing for k = c +
// 32 i, digit i of bytes 8q .. 8q + 7 of a superblock are exactly k = 32 i + 8q .. 32 i + 8q + 7:
// one MFMA per digit, and the lane's B operand is 8 consecutive halves of x, one 16-byte LDS
// read with no repacking.
//
// Decoding.  A 256-entry table in LDS maps a byte to its five digits, each as the high byte of
// the binary16 it becomes: 0x00 (0), 0x40 (+2) or 0xC0 (-2), digits 0..3 in the entry's first
// dword and digit 4 in its second.  One v_perm_b32 then builds the operand pair of bytes 2m and
// 2m + 1 for digit i, (0x00, digit byte, 0x00, digit byte), exactly; the factor 2 comes off once
// at the end.  Bytes 243..255 are reserved: the table maps them to zero weights, and results on
// them are unspecified.  The table is a static LDS array, so its address is a constant the
// compiler folds into the reads, and a lookup's address (8 times byte k of a word) is one SDWA
// shift.  The table reads land on random banks; that conflict cost is what this decode adds over
// the 2-bit codes' shift-and-mask.
//
// Work split (as the small-M kernel for the other layouts).  A workgroup owns 16 RT weight rows
// and one block of 16 rows of x; its waves take slices of 640 k (four superblocks, five groups):
// the slice's codes, scales and x arrive by direct global->LDS copies, each 32-k block's MFMAs
// chain within their group of 128 k and the group scale is applied to the sums once per group;
// the waves' partial sums meet in LDS and are added in a fixed order.
#include <limits.h>

#include "device.h"
#include "launch.h"

namespace bonsai {
namespace {

typedef float float4_v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glb_void_t;

constexpr int kT5SbPerSlice = 4;                     // superblocks of 160 k per slice
constexpr int kT5GroupsPerSlice = 5;                 // groups of 128 k per slice (640 k)
constexpr int kT5SliceBytes = 32 * kT5SbPerSlice;    // code bytes per row and slice
constexpr int kT5XStride = 2 * 640 + 16;             // LDS bytes per row of x (640 k + pad)
constexpr int kT5LutBytes = 256 * 8;
// Waves per workgroup: at most 16 (WIDE), which caps a wave at 128 VGPRs, or 8.  The 32-row
// tile takes about 160 VGPRs: the 8-wave build keeps them all, the 16-wave build fits in 128
// (no spill) and lets a CU hold two 8-wave workgroups by registers.
constexpr int t5_max_waves(bool wide) { return wide ? 16 : 8; }

constexpr int t5_scale_bytes(int rt) { return (5 * 16 * rt + 63) / 64 * 256; }

typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) const unsigned long long lds_u64_t;

// the 8-byte table entry at LDS byte address a
__device__ __forceinline__ uint2 lut_entry(uint32_t a)
{
    const unsigned long long v = *reinterpret_cast<lds_u64_t *>((uintptr_t)a);
    return uint2{(uint32_t)v, (uint32_t)(v >> 32)};
}

// 8 * (byte KB of v): the byte offset of its 8-byte table entry, one SDWA shift
template <int KB>
__device__ __forceinline__ uint32_t entry_offset(uint32_t v, uint32_t three)
{
    uint32_t r;
    if constexpr (KB == 0)
        asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "s"(three), "v"(v));
    else if constexpr (KB == 1)
        asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "s"(three), "v"(v));
    else if constexpr (KB == 2)
        asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "s"(three), "v"(v));
    else
        asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "s"(three), "v"(v));
    return r;
}

// LDS bytes of one wave: codes, scales and the M rows of x
constexpr int t5_wave_bytes(int rt, int m) { return 16 * rt * kT5SliceBytes + t5_scale_bytes(rt) + m * kT5XStride; }

template <int RT, bool WIDE>
__global__ __launch_bounds__(t5_max_waves(WIDE) * 64) void t5_gemv_kernel(const uint8_t *__restrict__ codes,
                                                                  const uint16_t *__restrict__ scales,
                                                                  const uint16_t *__restrict__ x,
                                                                  float *__restrict__ y, int M, int N, int K)
{
    constexpr int R = 16 * RT;
    constexpr int TILE = R * kT5SliceBytes;
    constexpr int SCB = t5_scale_bytes(RT);
    // the byte table is a static LDS array: its address is then a constant the compiler folds
    // into the table reads, so a lookup is one SDWA shift; the rest of LDS is dynamic
    __shared__ uint2 lut[256];
    extern __shared__ u32x4 lds[];
    x += (size_t)16 * blockIdx.y * K;
    y += (size_t)16 * blockIdx.y * N;
    M = min(16, M - 16 * (int)blockIdx.y);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int G = K >> 7;
    const int SB = (K + 159) / 160;                   // superblocks per row
    const int units = 2 * SB;                         // 16-byte units per row
    const int ns = (SB + kT5SbPerSlice - 1) / kT5SbPerSlice;
    const int n0 = blockIdx.x * R;
    const int wbytes = t5_wave_bytes(RT, M);
    char *const mine = reinterpret_cast<char *>(lds) + wave * wbytes;
    char *const tile = mine;
    char *const sc = mine + TILE;
    char *const xs = sc + SCB;
    float *const red = reinterpret_cast<float *>(reinterpret_cast<char *>(lds) + nw * wbytes);
    const int q = lane >> 4, i16 = lane & 15;
    const u32x4 *xg = reinterpret_cast<const u32x4 *>(x);
    const int xunits = K >> 3;                        // 16-byte units per row of x

    // the byte -> digits table: digit i of v as byte i (0..3 of .x, 4 of .y) 0x00, 0x40 or 0xC0
    for (int v = threadIdx.x; v < 256; v += blockDim.x) {
        uint32_t b[2] = {0u, 0u};
        if (v < 243) {
            int r = v;
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const int d = r % 3;
                r /= 3;
                b[i >> 2] |= (d == 0 ? 0x00u : d == 1 ? 0x40u : 0xC0u) << (8 * (i & 3));
            }
        }
        lut[v] = uint2{b[0], b[1]};
    }
    __syncthreads();

    float4_v acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t] = float4_v{0.f, 0.f, 0.f, 0.f};
    const float4_v zero4 = float4_v{0.f, 0.f, 0.f, 0.f};
    const uint32_t lut_base = (uint32_t)(uintptr_t)((lds_char_t *)lut);
    const uint32_t three = __builtin_amdgcn_readfirstlane(3u);

    for (int s = wave; s < ns; s += nw) {
        const int g0 = kT5GroupsPerSlice * s;
        // codes: copy k covers rows 8 k + lane / 8; the 16-byte unit c of row r lands in slot
        // c ^ (r & 7) of the row's 128 bytes (clamped inside the row: past-K groups count 0)
#pragma unroll
        for (int k = 0; k < TILE / 1024; ++k) {
            const int r = 8 * k + (lane >> 3);
            const int c = (lane & 7) ^ (r & 7);
            const int unit = min(2 * kT5SbPerSlice * s + c, units - 1);
            __builtin_amdgcn_global_load_lds(
                (glb_void_t *)(codes + (size_t)min(n0 + r, N - 1) * (32 * SB) + 16 * unit),
                (lds_void_t *)(tile + k * 1024), 16, 0, 0);
        }
        // scales: entry e = 5 r + u (row r, group u of the slice) is the low half of the dword
        // at sc + 4 e (one 2-byte copy per entry)
#pragma unroll
        for (int k = 0; k < SCB / 256; ++k) {
            const int e = 64 * k + lane, r = min(e / 5, R - 1), u = e % 5;
            __builtin_amdgcn_global_load_lds(
                (glb_void_t *)(scales + (size_t)min(n0 + r, N - 1) * G + min(g0 + u, G - 1)),
                (lds_void_t *)(sc + 256 * k), 2, 0, 0);
        }
        // x: row m, k = 640 s .. 640 s + 639 (80 units; clamped inside K)
        for (int m = 0; m < M; ++m) {
            const u32x4 *row = xg + (size_t)m * xunits;
            __builtin_amdgcn_global_load_lds((glb_void_t *)(row + min(80 * s + lane, xunits - 1)),
                                             (lds_void_t *)(xs + m * kT5XStride), 16, 0, 0);
            if (lane < 16)
                __builtin_amdgcn_global_load_lds((glb_void_t *)(row + min(80 * s + 64 + lane, xunits - 1)),
                                                 (lds_void_t *)(xs + m * kT5XStride + 1024), 16, 0, 0);
        }
        vm_wait<0>();                                     // this wave's slice landed
        if (g0 + kT5GroupsPerSlice > G) {
            // groups past K (last slice only) hold clamped copies: their scales become zero
            for (int e = lane; e < 5 * R; e += 64)
                if (g0 + e % 5 >= G) *reinterpret_cast<uint16_t *>(sc + 4 * e) = 0;
        }

        const char *xrow = xs + min(i16, M - 1) * kT5XStride;   // row i16 of x (M - 1 past M)
        float4_v d[RT];
#pragma unroll
        for (int sb = 0; sb < kT5SbPerSlice; ++sb) {
            // this lane's 8 bytes (8q .. 8q + 7) of superblock sb in each row tile, decoded
            uint2 lv[RT][8];
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                const int r = 16 * t + i16;
                const int slot = (2 * sb + (q >> 1)) ^ (r & 7);
                const uint2 b8 = *reinterpret_cast<const uint2 *>(tile + kT5SliceBytes * r + 16 * slot + 8 * (q & 1));
                lv[t][0] = lut_entry(lut_base + entry_offset<0>(b8.x, three));
                lv[t][1] = lut_entry(lut_base + entry_offset<1>(b8.x, three));
                lv[t][2] = lut_entry(lut_base + entry_offset<2>(b8.x, three));
                lv[t][3] = lut_entry(lut_base + entry_offset<3>(b8.x, three));
                lv[t][4] = lut_entry(lut_base + entry_offset<0>(b8.y, three));
                lv[t][5] = lut_entry(lut_base + entry_offset<1>(b8.y, three));
                lv[t][6] = lut_entry(lut_base + entry_offset<2>(b8.y, three));
                lv[t][7] = lut_entry(lut_base + entry_offset<3>(b8.y, three));
            }
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const int blk = 5 * sb + i;                   // 32-k block of the slice
                const int u = blk >> 2;                       // its group in the slice
                const u32x4 bv = *reinterpret_cast<const u32x4 *>(xrow + 64 * blk + 16 * q);
                const half8_t bf = __builtin_bit_cast(half8_t, bv);
                // (0x00, byte i' of the first source, 0x00, byte i' of the second)
                const uint32_t sel = 0x000C000Cu | ((uint32_t)(i & 3) << 8) | ((uint32_t)(4 + (i & 3)) << 24);
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    u32x4 av;
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        av[m] = i < 4 ? __builtin_amdgcn_perm(lv[t][2 * m + 1].x, lv[t][2 * m].x, sel)
                                      : __builtin_amdgcn_perm(lv[t][2 * m + 1].y, lv[t][2 * m].y, sel);
                    d[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), bf,
                                                                  (blk & 3) == 0 ? zero4 : d[t], 0, 0, 0);
                }
                if ((blk & 3) == 3) {
                    // group u complete: D rows 16 t + 4 q + r take their scale
#pragma unroll
                    for (int t = 0; t < RT; ++t)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int row = 16 * t + 4 * q + r;
                            const uint16_t sv = *reinterpret_cast<const uint16_t *>(sc + 4 * (5 * row + u));
                            acc[t][r] = fmaf(f16_bits_to_f32(sv), d[t][r], acc[t][r]);
                        }
                }
            }
        }
        lgkm_wait0();                                     // LDS reads done before the next slice's copies
    }

    // D rows 16 t + 4 q + r, column i16: the wave's partial sums into red[wave][column][row]
    if (i16 < M) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[(wave * M + i16) * R + 16 * t + 4 * q + r] = 0.5f * acc[t][r];
    }
    __syncthreads();
    for (int o = threadIdx.x; o < M * R; o += blockDim.x) {
        const int m = o / R, row = o % R;
        float v = 0.f;
        for (int w = 0; w < nw; ++w) v += red[(w * M + m) * R + row];
        if (n0 + row < N) y[(size_t)m * N + n0 + row] = v;
    }
}

// waves of a workgroup: one per slice, at most 16 and as many as the LDS holds
int t5_waves(int rt, bool wide, int M, int K)
{
    const int ns = ((K + 159) / 160 + kT5SbPerSlice - 1) / kT5SbPerSlice;
    const int per_wave = t5_wave_bytes(rt, M) + M * 16 * rt * 4;
    int nw = ns < t5_max_waves(wide) ? ns : t5_max_waves(wide);
    if (nw > (kLdsPerCu - kT5LutBytes) / per_wave) nw = (kLdsPerCu - kT5LutBytes) / per_wave;
    return nw;
}

size_t t5_lds(int rt, int mb, int nw)
{
    return (size_t)kT5LutBytes + (size_t)nw * t5_wave_bytes(rt, mb) + (size_t)nw * mb * 16 * rt * 4;
}

// waves of t5_gemv_kernel<RT, WIDE> that one CU holds by registers
template <int RT, bool WIDE>
int t5_reg_waves_per_cu()
{
    return reg_waves_per_cu(func_vgprs(reinterpret_cast<const void *>(&t5_gemv_kernel<RT, WIDE>)));
}

template <int RT, bool WIDE>
hipError_t t5_launch_rt(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                        int M, int N, int K, hipStream_t stream)
{
    const int mb = M < 16 ? M : 16;
    const int nw = t5_waves(RT, WIDE, mb, K);
    if (nw < 1) return hipErrorInvalidValue;
    const int64_t blocks = ((int64_t)N + 16 * RT - 1) / (16 * RT);
    const int64_t yblocks = ((int64_t)M + 15) / 16;
    if (blocks > INT_MAX || yblocks > 65535) return hipErrorInvalidValue;
    // dynamic LDS: everything but the static 2 KB byte table
    const void *fn = reinterpret_cast<const void *>(&t5_gemv_kernel<RT, WIDE>);
    if (!set_lds_limit(fn, kLdsPerCu - kT5LutBytes)) return hipErrorInvalidValue;
    void *args[] = {&codes, &scales, &x, &y, &M, &N, &K};
    return launch_kernel(fn, __PRETTY_FUNCTION__, dim3((unsigned)blocks, (unsigned)yblocks), dim3(64 * nw), args,
                         t5_lds(RT, mb, nw) - kT5LutBytes, stream);
}

}  // namespace

// Any M >= 1 (16 rows of x per column block).  Three builds: 16-row tiles (up to 16 waves), 32-row
// tiles with up to 8 waves (163 VGPRs), 32-row tiles with up to 16 waves (held to 128 VGPRs, two
// workgroups per CU).  The launch takes the build whose grid needs the fewest rounds of the
// device's CUs (256 on MI355X), given what the LDS and the registers of a CU hold; on a tie, in the
// order that measured fastest: for one row of x the 16-row tile first (more workgroups in flight),
// for more rows the 8-wave 32-row build first (x, held once per wave, fills the LDS).
hipError_t launch_t5_matmul(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                            int M, int N, int K, hipStream_t stream)
{
    if (M < 1) return hipErrorInvalidValue;
    const int kCus = device_cus();
    const int mb = M < 16 ? M : 16;
    auto rounds = [&](int rt, bool wide, int reg_waves) -> int64_t {
        const int nw = t5_waves(rt, wide, mb, K);
        if (nw < 1) return INT64_MAX;
        int64_t per_cu = kLdsPerCu / (int64_t)t5_lds(rt, mb, nw);
        if (per_cu > reg_waves / nw) per_cu = reg_waves / nw;
        if (per_cu < 1) return INT64_MAX;
        const int64_t blocks = (((int64_t)N + 16 * rt - 1) / (16 * rt)) * (((int64_t)M + 15) / 16);
        return (blocks + per_cu * kCus - 1) / (per_cu * kCus);
    };
    const int64_t r1 = rounds(1, true, t5_reg_waves_per_cu<1, true>());
    const int64_t r2n = rounds(2, false, t5_reg_waves_per_cu<2, false>());
    const int64_t r2s = rounds(2, true, t5_reg_waves_per_cu<2, true>());
    if (M == 1) {
        if (r1 <= r2n && r1 <= r2s) return t5_launch_rt<1, true>(codes, scales, x, y, M, N, K, stream);
        if (r2n <= r2s) return t5_launch_rt<2, false>(codes, scales, x, y, M, N, K, stream);
        return t5_launch_rt<2, true>(codes, scales, x, y, M, N, K, stream);
    }
    if (r2n <= r2s && r2n <= r1) return t5_launch_rt<2, false>(codes, scales, x, y, M, N, K, stream);
    if (r2s <= r1) return t5_launch_rt<2, true>(codes, scales, x, y, M, N, K, stream);
    return t5_launch_rt<1, true>(codes, scales, x, y, M, N, K, stream);
}

}  // namespace bonsai
