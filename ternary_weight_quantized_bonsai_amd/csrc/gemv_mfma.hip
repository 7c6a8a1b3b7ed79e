// gemv_mfma.hip -- small-M GEMV on the matrix cores: ternary M = 1..8 and binary M = 2..8.
//
// y[m][n] = sum_k W[n][k] x[m][k] for a handful of rows of x.  The weight rows play the MFMA
// row dimension and x the (zero-padded) 16-wide column dimension of v_mfma_f32_16x16x32_f16,
// so one instruction consumes 16 weight rows x 32 k and the expansion of the packed codes to
// binary16 costs about one VALU op per weight; the matrix core does the multiply-adds that
// would otherwise cost M VALU ops per weight.
//
// Operands.  An MFMA lane (row i = lane % 16, quarter q = lane / 16) holds 8 halves of A and
// of B for the same 8 k of a 32-k block.  Which 8 k is a free choice as long as A and B agree,
// so each quarter takes k whose codes sit 16 bits apart in a word; one shift and one mask then
// put a pair of them onto the two binary16 halves:
//   binary  word = the 32 k of the block: quarter q takes bits 4q+i and 4q+i+16 (i = 0..3);
//           ((w << (15 - 4q - i)) & 0x80008000) ^ 0xBC00BC00 is the pair (+-1, +-1), bit 1 -> +1.
//   ternary the block is two words of 16 codes: pair i of quarter q is fields j = 2q + (i % 2)
//           and j + 8 of word i / 2; (w << (14 - 2j)) & 0xC000C000 reads codes 00, 01, 11 as
//           0, +2, -2 (the exponent MSB is the code's low bit, the sign its high bit).
//   affine  binary words again, but the operand is the bit itself, q 2^-7 (binary16 0x2000 or 0):
//           rotate the word so that bit 4q+i lands on bit 13, mask with 0x20002000.
// B holds x at the same k.  Column j of D depends on column j of B alone, so the lanes of the
// columns past M read row M - 1 again (a broadcast) and those columns are never stored.
// The group scale multiplies each group's four chained MFMAs afterwards, one mixed-precision
// FMA per output straight from the binary16 scale, so the operands stay exact small integers
// and every product is exact; the ternary factor 2 comes off the sums once at the end.
//
// Affine weights (MLX's 1-bit form: a scale a and a bias b per group, weight a q + b for the bit
// q; "1-bit Bonsai 27B" model card, "MLX packaging") split each group's sum into a times the
// q-weighted sum D and b times the plain sum X of x over the group.  X does not depend on the
// weight row: each lane adds up its quarter's 32 halves of the group with v_dot2 against (1, 1)
// on the B operand it already holds, and two lane exchanges (quarters 16 and 32 lanes apart)
// complete the column's sum.  The operand's 2^-7 comes off at the end with the bias term scaled
// to match: acc = sum_g a_g D_g + b_g X_g 2^-7, y = 128 acc.
//
// Rows of x beyond 16 take more column blocks: blockIdx.y selects rows 16 y .. 16 y + 15 of x
// and of the output, so a skinny product (a few dozen rows of x, as in checking several draft
// tokens at once) runs as that many 16-column passes over the same weight tiles.
//
// Work split.  A workgroup owns R = 16 RT weight rows; its waves take slices of K of SG = 4 or
// 2 groups.  Each slice's codes (R rows x SG groups), scales and x (M rows x 128 SG k) are
// copied straight into the wave's LDS (direct global->LDS loads, whole lines), the wave's
// partial sums of the R x M outputs meet the other waves' in LDS and are added in a fixed order.
#include <limits.h>

#include <type_traits>

#include "device.h"
#include "launch.h"

namespace bonsai {
namespace {

typedef float float4_v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glb_void_t;

constexpr int kSmMaxWaves = 16;

// SG: groups per K-slice, 4 or 2.  Two-group slices give twice the waves for the same K, which
// spread more evenly over a CU's four SIMDs when four-group slices would leave them uneven.
template <bool TERN, int SG>
struct SmLayout {
    // (affine weights use the binary layout; their biases take a second scale-sized region)
    static constexpr int cell = TERN ? 32 : 16;           // bytes per (row, group)
    static constexpr int row_bytes = SG * cell;            // bytes per row and slice
    static constexpr int lanes_per_row = row_bytes / 16;
    static constexpr int rows_per_copy = 64 / lanes_per_row;
    // LDS bytes per row of x (128 SG k): the pad puts the x rows a lane quarter reads on
    // distinct banks (4 dwords apart for the one-dword ternary reads, 8 for the two-dword
    // binary ones)
    static constexpr int xstride = 256 * SG + (TERN ? 16 : 32);
    // the 16-byte unit c of row r sits at row_bytes r + 16 (c ^ swz(r)): rows 256 B apart (the
    // same banks) hold their units in different places
    static __device__ __forceinline__ int swz(int r) { return (r / (256 / row_bytes)) & (lanes_per_row - 1); }
    static constexpr int scale_bytes = 64 * SG * 4;       // room for one dword per (row, group), 64 rows
};

// LDS bytes of one wave: codes, scales (and biases) and the M rows of x
template <bool TERN, bool AFF, int SG>
constexpr int sm_wave_bytes(int rt, int m)
{
    using L = SmLayout<TERN, SG>;
    return 16 * rt * L::row_bytes + (AFF ? 2 : 1) * L::scale_bytes + m * L::xstride;
}

// four row tiles per wave need more than the 128 VGPRs that 16 waves per workgroup leave
constexpr int sm_max_waves(int rt) { return rt >= 4 ? 12 : kSmMaxWaves; }

// PAIRS: the group count is even, so a row's scales of groups 2p, 2p + 1 are one aligned dword.
// AFF: affine 1-bit weights (binary words, scales and biases); biases is unused otherwise.
template <bool TERN, bool AFF, int RT, bool PAIRS, int SG>
__global__ __launch_bounds__(sm_max_waves(RT) * 64) void gemv_mfma_kernel(const uint32_t *__restrict__ codes,
                                                                     const uint16_t *__restrict__ scales,
                                                                     const uint16_t *__restrict__ biases,
                                                                     const uint16_t *__restrict__ x,
                                                                     float *__restrict__ y, int M, int N, int K)
{
    static_assert(!(TERN && AFF), "affine weights are binary words");
    static_assert(SG == 4 || SG == 2, "four- or two-group slices");
    using L = SmLayout<TERN, SG>;
    constexpr int R = 16 * RT;
    constexpr int TILE = R * L::row_bytes;
    extern __shared__ u32x4 lds[];
    // this workgroup's block of 16 rows of x and y
    x += (size_t)16 * blockIdx.y * K;
    y += (size_t)16 * blockIdx.y * N;
    M = min(16, M - 16 * (int)blockIdx.y);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int G = K >> 7;
    const int ns = (G + SG - 1) / SG;                     // slices of K
    const int n0 = blockIdx.x * R;
    const int wbytes = sm_wave_bytes<TERN, AFF, SG>(RT, M);
    char *const mine = reinterpret_cast<char *>(lds) + wave * wbytes;
    char *const tile = mine;
    char *const sc = mine + TILE;
    char *const bc = sc + L::scale_bytes;                 // biases (affine only), laid out as sc
    char *const xs = sc + (AFF ? 2 : 1) * L::scale_bytes;
    float *const red = reinterpret_cast<float *>(reinterpret_cast<char *>(lds) + nw * wbytes);
    const int q = lane >> 4, i16 = lane & 15;
    const int units = G * (L::cell / 16);                  // 16-byte units per weight row
    const u32x4 *cg = reinterpret_cast<const u32x4 *>(codes);
    const u32x4 *xg = reinterpret_cast<const u32x4 *>(x);

    float4_v acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t] = float4_v{0.f, 0.f, 0.f, 0.f};
    const float4_v zero4 = float4_v{0.f, 0.f, 0.f, 0.f};

    for (int s = wave; s < ns; s += nw) {
        const int g0 = s * SG;
        const int g1 = min(G, g0 + SG), gl = g1 - 1;
        // codes: copy k covers rows rows_per_copy * k + lane / lanes_per_row (a tile under 1 KB,
        // binary 16 rows of two groups, takes the first lanes of one copy); the 16-byte chunk c
        // of row r lands at row_bytes * r + 16 (c ^ swz(r))
#pragma unroll
        for (int k = 0; k < (TILE + 1023) / 1024; ++k) {
            if (1024 * k + 16 * lane < TILE) {
                const int r = L::rows_per_copy * k + lane / L::lanes_per_row;
                const int c = (lane % L::lanes_per_row) ^ L::swz(r);
                const int unit = min(g0 * (L::cell / 16) + c, units - 1);
                __builtin_amdgcn_global_load_lds((glb_void_t *)(cg + (size_t)min(n0 + r, N - 1) * units + unit),
                                                 (lds_void_t *)(tile + k * 1024), 16, 0, 0);
            }
        }
        // scales: SW dwords per row; the scale of (row r, group u) is half u % 2 of the dword at
        // sc + 4 (SW r + u / 2) (PAIRS, SW = SG / 2: one 4-byte copy per row and pair of groups),
        // or the low half of the dword at sc + 4 (SW r + u) (SW = SG: one 2-byte copy per row and
        // group)
        constexpr int SW = PAIRS ? SG / 2 : SG;
#pragma unroll
        for (int which = 0; which < (AFF ? 2 : 1); ++which) {
            const uint16_t *const src = which ? biases : scales;
            char *const dst = which ? bc : sc;
            if constexpr (PAIRS) {
#pragma unroll
                for (int k = 0; k < (SW * R + 63) / 64; ++k) {
                    const int e = 64 * k + lane, r = min(e / SW, R - 1), p = e % SW;
                    __builtin_amdgcn_global_load_lds((glb_void_t *)(src + (size_t)min(n0 + r, N - 1) * G + min(g0 + 2 * p, G - 2)),
                                                     (lds_void_t *)(dst + 256 * k), 4, 0, 0);
                }
            } else {
#pragma unroll
                for (int k = 0; k < (SW * R + 63) / 64; ++k) {
                    const int e = 64 * k + lane, r = min(e / SW, R - 1), u = e % SW;
                    __builtin_amdgcn_global_load_lds((glb_void_t *)(src + (size_t)min(n0 + r, N - 1) * G + min(g0 + u, gl)),
                                                     (lds_void_t *)(dst + 256 * k), 2, 0, 0);
                }
            }
        }
        // x: row m, k = 128 g0 .. 128 g0 + 128 SG - 1 (clamped inside K; past-K groups count 0)
        if (lane < 16 * SG) {
            for (int m = 0; m < M; ++m)
                __builtin_amdgcn_global_load_lds((glb_void_t *)(xg + (size_t)m * (K >> 3) + min(16 * g0 + lane, (K >> 3) - 1)),
                                                 (lds_void_t *)(xs + m * L::xstride), 16, 0, 0);
        }
        vm_wait<0>();                                     // this wave's slice landed
        if (g1 - g0 < SG) {
            // groups past K (last slice only) hold clamped copies: their scales (and biases)
            // become zero
            for (int e = lane; e < R * SG; e += 64) {
                const int r = e / SG, u = e % SG;
                const int off = PAIRS ? 4 * SW * r + 2 * u : 4 * SW * r + 4 * u;
                if (g0 + u >= g1) {
                    *reinterpret_cast<uint16_t *>(sc + off) = 0;
                    if constexpr (AFF) *reinterpret_cast<uint16_t *>(bc + off) = 0;
                }
            }
        }
        // the scales of this lane's D rows 16 t + 4 q + r, all SG groups: the binary16 of group u
        // is half u % 2 of sp[t][r][u / 2] (PAIRS) or the low half of sp[t][r][u]
        constexpr int NB = AFF ? 2 : 1;
        uint32_t sp[NB][RT][4][SW];                       // [0] scales, [1] biases
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * t + 4 * q + r;
                    const char *const base = b ? bc : sc;
                    if constexpr (SW == 4) {
                        const u32x4 v = *reinterpret_cast<const u32x4 *>(base + 16 * row);
#pragma unroll
                        for (int e = 0; e < 4; ++e) sp[b][t][r][e] = v[e];
                    } else if constexpr (SW == 2) {
                        const uint2 v = *reinterpret_cast<const uint2 *>(base + 8 * row);
                        sp[b][t][r][0] = v.x;
                        sp[b][t][r][1] = v.y;
                    } else {
                        sp[b][t][r][0] = *reinterpret_cast<const uint32_t *>(base + 4 * row);
                    }
                }
        float xq[SG];                                     // affine: this quarter's part of X per group

#pragma unroll
        for (int u = 0; u < SG; ++u) {
            // this lane's weight rows: 16 t + i16, one cell each
            uint32_t wd[RT][L::cell / 4];
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                const int r = 16 * t + i16;
                const int sw = L::swz(r);
#pragma unroll
                for (int h = 0; h < L::cell / 16; ++h) {
                    const int c = (L::cell / 16) * u + h;
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(tile + L::row_bytes * r + 16 * (c ^ sw));
#pragma unroll
                    for (int e = 0; e < 4; ++e) wd[t][4 * h + e] = v[e];
                }
            }
            float4_v d[RT];
            const char *xrow = xs + min(i16, M - 1) * L::xstride;   // row i16 of x (M - 1 past M)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                // B: this quarter's 8 k of block kb, in the order of the A pairs
                u32x4 bv;
                if constexpr (TERN) {
                    const int k0 = 128 * u + 32 * kb + 2 * q;
                    const uint32_t a0 = *reinterpret_cast<const uint32_t *>(xrow + 2 * k0);
                    const uint32_t a1 = *reinterpret_cast<const uint32_t *>(xrow + 2 * (k0 + 8));
                    const uint32_t a2 = *reinterpret_cast<const uint32_t *>(xrow + 2 * (k0 + 16));
                    const uint32_t a3 = *reinterpret_cast<const uint32_t *>(xrow + 2 * (k0 + 24));
                    bv[0] = pack_lo(a0, a1);
                    bv[1] = pack_hi(a0, a1);
                    bv[2] = pack_lo(a2, a3);
                    bv[3] = pack_hi(a2, a3);
                } else {
                    const int k0 = 128 * u + 32 * kb + 4 * q;
                    const uint2 xa = *reinterpret_cast<const uint2 *>(xrow + 2 * k0);
                    const uint2 xb = *reinterpret_cast<const uint2 *>(xrow + 2 * (k0 + 16));
                    bv[0] = pack_lo(xa.x, xb.x);
                    bv[1] = pack_hi(xa.x, xb.x);
                    bv[2] = pack_lo(xa.y, xb.y);
                    bv[3] = pack_hi(xa.y, xb.y);
                }
                const half8_t bf = __builtin_bit_cast(half8_t, bv);
                if constexpr (AFF) {
                    const half2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
                    float xs4 = kb == 0 ? 0.f : xq[u];
#pragma unroll
                    for (int e = 0; e < 4; ++e) xs4 = __builtin_amdgcn_fdot2(as_half2(bv[e]), one2, xs4, false);
                    xq[u] = xs4;
                }
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    u32x4 av;
                    if constexpr (AFF) {
                        const uint32_t w = wd[t][kb];
#pragma unroll
                        for (int i = 0; i < 4; ++i)   // rotate bit 4q + i (and 16 above it) onto bit 13
                            av[i] = __builtin_amdgcn_alignbit(w, w, (uint32_t)(4 * q + i + 19)) & 0x20002000u;
                    } else if constexpr (TERN) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t w = wd[t][2 * kb + (i >> 1)];
                            av[i] = (w << (14 - 4 * q - 2 * (i & 1))) & 0xC000C000u;
                        }
                    } else {
                        const uint32_t w = wd[t][kb];
#pragma unroll
                        for (int i = 0; i < 4; ++i) av[i] = ((w << (15 - 4 * q - i)) & 0x80008000u) ^ 0xBC00BC00u;
                    }
                    const half8_t af = __builtin_bit_cast(half8_t, av);
                    d[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, kb == 0 ? zero4 : d[t], 0, 0, 0);
                }
            }
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const half2_t h = as_half2(sp[0][t][r][PAIRS ? u >> 1 : u]);
                    acc[t][r] = fmaf((float)h[PAIRS ? u & 1 : 0], d[t][r], acc[t][r]);
                }
        }
        if constexpr (AFF) {
            // the bias term: X of column i16 is the sum of the four quarters' parts
#pragma unroll
            for (int u = 0; u < SG; ++u) {
                float xg = xq[u] + __shfl_xor(xq[u], 16);
                xg = (xg + __shfl_xor(xg, 32)) * 0x1p-7f;
#pragma unroll
                for (int t = 0; t < RT; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const half2_t h = as_half2(sp[NB - 1][t][r][PAIRS ? u >> 1 : u]);
                        acc[t][r] = fmaf((float)h[PAIRS ? u & 1 : 0], xg, acc[t][r]);
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
            for (int r = 0; r < 4; ++r) red[(wave * M + i16) * R + 16 * t + 4 * q + r] = TERN ? 0.5f * acc[t][r] : AFF ? 128.f * acc[t][r] : acc[t][r];
    }
    __syncthreads();
    for (int o = threadIdx.x; o < M * R; o += blockDim.x) {
        const int m = o / R, row = o % R;
        float v = 0.f;
        for (int w = 0; w < nw; ++w) v += red[(w * M + m) * R + row];
        if (n0 + row < N) y[(size_t)m * N + n0 + row] = v;
    }
}


// waves of a workgroup: one per slice of K, at most 16 and as many as the LDS holds
template <bool TERN, bool AFF, int SG>
int sm_waves(int rt, int M, int K)
{
    const int ns = (K / 128 + SG - 1) / SG;
    const int per_wave = sm_wave_bytes<TERN, AFF, SG>(rt, M) + M * 16 * rt * 4;
    int nw = ns < sm_max_waves(rt) ? ns : sm_max_waves(rt);
    if (nw > kLdsPerCu / per_wave) nw = kLdsPerCu / per_wave;
    return nw;
}

template <bool TERN, bool AFF, int RT, int SG>
hipError_t launch_rt(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases, const uint16_t *x,
                     float *y, int M, int N, int K, hipStream_t stream)
{
    const int mb = M < 16 ? M : 16;                 // rows of x per workgroup
    const int nw = sm_waves<TERN, AFF, SG>(RT, mb, K);
    if (nw < 1) return hipErrorInvalidValue;
    const size_t lds = (size_t)nw * sm_wave_bytes<TERN, AFF, SG>(RT, mb) + (size_t)nw * mb * 16 * RT * 4;
    const int64_t blocks = ((int64_t)N + 16 * RT - 1) / (16 * RT);
    const int64_t yblocks = ((int64_t)M + 15) / 16;
    if (blocks > INT_MAX || yblocks > 65535) return hipErrorInvalidValue;
    const void *fn = (K / 128) % 2 == 0 ? reinterpret_cast<const void *>(&gemv_mfma_kernel<TERN, AFF, RT, true, SG>)
                                        : reinterpret_cast<const void *>(&gemv_mfma_kernel<TERN, AFF, RT, false, SG>);
    if (!set_lds_limit(fn, kLdsPerCu)) return hipErrorInvalidValue;
    void *args[] = {&codes, &scales, &biases, &x, &y, &M, &N, &K};
    return launch_kernel(fn, __PRETTY_FUNCTION__, dim3((unsigned)blocks, (unsigned)yblocks), dim3(64 * nw), args, lds,
                         stream);
}

// waves of gemv_mfma_kernel<TERN, AFF, RT, PAIRS, SG> that one CU holds by registers
template <bool TERN, bool AFF, int RT, bool PAIRS, int SG>
int sm_reg_waves_per_cu()
{
    return reg_waves_per_cu(func_vgprs(reinterpret_cast<const void *>(&gemv_mfma_kernel<TERN, AFF, RT, PAIRS, SG>)));
}

template <bool TERN, bool AFF, int RT, int SG>
int sm_reg_waves(bool pairs)
{
    return pairs ? sm_reg_waves_per_cu<TERN, AFF, RT, true, SG>() : sm_reg_waves_per_cu<TERN, AFF, RT, false, SG>();
}

template <bool TERN, bool AFF, int SG>
struct SmChoice {
    int rt, simd;                                 // tile, groups on the busiest SIMD
    int64_t rounds, rows;
};

// groups that the busiest SIMD of a workgroup computes: wave w runs on SIMD w % 4 and takes
// slices w, w + nw, ... of the ns slices of SG groups
inline int sm_simd_groups(int nw, int ns, int sg)
{
    int most = 0;
    for (int s = 0; s < 4; ++s) {
        int n = 0;
        for (int w = s; w < nw; w += 4) n += (ns - w + nw - 1) / nw;
        most = n > most ? n : most;
    }
    return sg * most;
}

// The row tile (16, 32 or 64 rows) for slices of SG groups: the one whose grid needs the fewest
// rounds of the device's CUs (256 on MI355X), given what the LDS and the registers of a CU hold;
// among those, the one that leaves the busiest CU the fewest weight rows (workgroups per CU,
// rounded up, times the tile), then the larger tile (its x copies and reduction serve more rows).
template <bool TERN, bool AFF, int SG>
SmChoice<TERN, AFF, SG> sm_choose(int M, int N, int K)
{
    const int kCus = device_cus();
    const int mb = M < 16 ? M : 16;
    const bool pairs = (K / 128) % 2 == 0;
    using C = SmChoice<TERN, AFF, SG>;
    auto cost = [&](int rt, int reg_waves) -> C {
        const int nw = sm_waves<TERN, AFF, SG>(rt, mb, K);
        if (nw < 1) return {rt, 0, INT64_MAX, INT64_MAX};
        const int simd = sm_simd_groups(nw, (K / 128 + SG - 1) / SG, SG);
        const int64_t lds = (int64_t)nw * sm_wave_bytes<TERN, AFF, SG>(rt, mb) + (int64_t)nw * mb * 16 * rt * 4;
        int64_t per_cu = kLdsPerCu / lds;
        if (per_cu > reg_waves / nw) per_cu = reg_waves / nw;
        if (per_cu < 1) return {rt, 0, INT64_MAX, INT64_MAX};
        const int64_t blocks = (((int64_t)N + 16 * rt - 1) / (16 * rt)) * (((int64_t)M + 15) / 16);
        return {rt, simd, (blocks + per_cu * kCus - 1) / (per_cu * kCus), (blocks + kCus - 1) / kCus * 16 * rt};
    };
    auto better = [](const C &a, const C &b) {   // a strictly better than b, ties to b
        return a.rounds < b.rounds || (a.rounds == b.rounds && a.rows < b.rows);
    };
    const C c1 = cost(1, sm_reg_waves<TERN, AFF, 1, SG>(pairs));
    const C c2 = cost(2, sm_reg_waves<TERN, AFF, 2, SG>(pairs));
    // the affine kernel keeps scales and biases in registers: no four-tile variant
    C best = {4, 0, INT64_MAX, INT64_MAX};
    if constexpr (!AFF) best = cost(4, sm_reg_waves<TERN, AFF, 4, SG>(pairs));
    if (better(c2, best)) best = c2;
    if (better(c1, best)) best = c1;
    return best;
}

template <bool TERN, bool AFF, int SG>
hipError_t launch_choice(const SmChoice<TERN, AFF, SG> &c, const uint32_t *codes, const uint16_t *scales,
                         const uint16_t *biases, const uint16_t *x, float *y, int M, int N, int K,
                         hipStream_t stream)
{
    if (c.rounds == INT64_MAX) return hipErrorInvalidValue;
    if (c.rt == 1) return launch_rt<TERN, AFF, 1, SG>(codes, scales, biases, x, y, M, N, K, stream);
    if (c.rt == 2) return launch_rt<TERN, AFF, 2, SG>(codes, scales, biases, x, y, M, N, K, stream);
    if constexpr (AFF) return hipErrorInvalidValue;
    else return launch_rt<TERN, AFF, 4, SG>(codes, scales, biases, x, y, M, N, K, stream);
}

template <bool TERN, bool AFF = false>
hipError_t launch_sm(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases, const uint16_t *x,
                     float *y, int M, int N, int K, hipStream_t stream)
{
    // Every wave loads its slice at once and then computes, so a second round of workgroups on
    // a CU pays the load latency again: the best tile for four-group and for two-group slices,
    // then the one of the two with fewer rounds, then fewer rows on the busiest CU, then fewer
    // groups on the busiest SIMD (two-group slices spread a short K over more waves), then four
    // groups (half the slice iterations, each with its waits and scale reads).
    const auto c4 = sm_choose<TERN, AFF, 4>(M, N, K);
    const auto c2 = sm_choose<TERN, AFF, 2>(M, N, K);
    const bool two = c2.rounds < c4.rounds ||
                     (c2.rounds == c4.rounds && (c2.rows < c4.rows || (c2.rows == c4.rows && c2.simd < c4.simd)));
    return two ? launch_choice(c2, codes, scales, biases, x, y, M, N, K, stream)
               : launch_choice(c4, codes, scales, biases, x, y, M, N, K, stream);
}

}  // namespace

// Any M >= 1 (16 rows of x per column block).
hipError_t launch_gemv_mfma(bool ternary, const uint32_t *codes, const uint16_t *scales, const uint16_t *x,
                            float *y, int M, int N, int K, hipStream_t stream)
{
    if (M < 1) return hipErrorInvalidValue;
    return ternary ? launch_sm<true>(codes, scales, nullptr, x, y, M, N, K, stream)
                   : launch_sm<false>(codes, scales, nullptr, x, y, M, N, K, stream);
}

// Affine 1-bit weights (MLX's scale-and-bias form of the binary words), any M >= 1.
hipError_t launch_q1a_matmul(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases,
                             const uint16_t *x, float *y, int M, int N, int K, hipStream_t stream)
{
    if (M < 1) return hipErrorInvalidValue;
    if (M == 1 && q1a_lut_fits(N, K)) return launch_q1a_lut(wbits, scales, biases, x, y, N, K, stream);
    return launch_sm<false, true>(wbits, scales, biases, x, y, M, N, K, stream);
}

// Ternary weights ("Ternary Bonsai 27B" article, ternary format: {-1, 0, +1} times the FP16
// group scale, two bits per weight in the current release) take this kernel for every M.
hipError_t launch_q2t_gemv(const uint32_t *wcodes, const uint16_t *scales, const uint16_t *x, float *y,
                           int M, int N, int K, hipStream_t stream)
{
    if (M < 1 || M > 8) return hipErrorInvalidValue;
    return launch_sm<true>(wcodes, scales, nullptr, x, y, M, N, K, stream);
}

}  // namespace bonsai
