// q1_lut8.hip -- binary g128 GEMV for one row of x over many weight rows (the LM head):
// y[n] = sum_k W[n][k] x[k] straight from the packed sign words ("1-bit Bonsai 27B" model card,
// "Weight representation: Binary g128": bit 1 -> +s, bit 0 -> -s, one FP16 scale per 128
// consecutive weights; its highlights count the LM head among the binary weights).
//
// Decode streams the weights once and is bound by memory bandwidth (model card, cross-platform
// throughput), so what matters is that the arithmetic per weight stays well under what HBM
// delivers.  Here a byte of sign bits, 8 weights, indexes a 256-entry table of the signed sums
// of their 8 x values: one LDS read and one add per 8 weights, and one v_perm_b32 that forms the
// table address from the byte.  With nibble tables (the tile kernels of q1_gemv.hip) it is one
// read, one add and one address operation per 4 weights.
//
// Byte tables are 1 KB each, so one CU holds those of 1024 k (one "slice", 128 tables, 128 KB):
// every CU walks all the slices of its rows, rebuilding the tables between slices, and keeps
// each lane's partial sums in registers across the slices, so no partial sum leaves the CU and
// the result does not depend on how rows are spread over CUs.
//
// LDS banks.  The 32 lanes of a half-wave read in one pass only if they fall on 32 distinct
// banks (or share an address).  The lanes hold different rows, so a table shared by them would
// be read at 32 random entries.  Instead the 32 lanes always read 32 different tables, and each
// table lives in one bank.  Lane l holds row l / 8 of an 8-row unit and group p = l % 8 of the
// slice: the 16-byte cell of four sign words of that (row, group), loaded straight into its
// registers.  At step j it looks up the four bytes of word j, and lookup m of the step takes byte
// i = (m + l / 8) % 4.  The table of byte i of word d = 4 p + j of the slice (its 8 weights) holds
// entry e at byte offset
//     (i >> 1) * 64 KB + e * 256 + (i & 1) * 128 + 4 (4 p + (j + i) % 4),
// i.e. in bank 4 p + (j + m + l / 8) % 4: over a half-wave (p = 0..7, (l / 8) % 4 = 0..3) the 32
// banks of a lookup are distinct.  The address is one v_perm_b32 of the word with a per-lane
// source holding the bank's offset and the 64 KB half, under a per-lane byte selector.
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace bonsai {
namespace {

typedef __attribute__((address_space(3))) float lds_f32_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;

constexpr int kL8SliceK = 1024;             // k per slice: 128 B of sign bits per row, 8 groups
constexpr int kL8Tables = 128 * 1024;       // 128 tables of 256 fp32 entries
constexpr int kL8MaxK = (160 * 1024 - kL8Tables) / 2;   // x (binary16) is staged after the tables
constexpr int kL8MaxKAff = 16128;           // affine: and X of every group after x (2K + K/32 bytes)

// LDS float at byte address a (the kernel's dynamic LDS starts at 0: it has no static LDS).
__device__ __forceinline__ float lds_f32(uint32_t a)
{
    return *reinterpret_cast<const lds_f32_t *>(static_cast<uintptr_t>(a));
}

// Entries I .. END - 1 of this wave's share of a table: entry base + I is lo[I % 16] + hi[I / 16],
// at byte address tb + 256 I.
template <int I, int END>
__device__ __forceinline__ void store_entries(uint32_t tb, const float (&lo)[16], const float *hi)
{
    if constexpr (I < END) {
        *reinterpret_cast<lds_f32_t *>(static_cast<uintptr_t>(tb + 256 * I)) = lo[I % 16] + hi[I / 16];
        store_entries<I + 1, END>(tb, lo, hi);
    }
}

// Compile-time loop: f(IC<I>{}) for I = BEGIN .. END - 1.
template <int I>
struct IC {
    static constexpr int value = I;
};
template <int I, int END, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < END) {
        f(IC<I>{});
        static_for<I + 1, END>(f);
    }
}

// Sum over the 8 lanes 8 r .. 8 r + 7 (every lane gets it): swaps within pairs and within quads,
// then each lane of a half-row of 8 adds the lane at its mirror position -- data-parallel
// moves between lanes (DPP), in a fixed order.
__device__ __forceinline__ float sum8(float v)
{
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    return v;
}

// W waves; PD units in flight per wave (their cells in registers); at most UMAX units per wave (a
// multiple of PD, so a unit's registers are fixed at compile time; the launch gives every
// workgroup at most W UMAX units); the scales of SQ slices of every unit in registers at a time.
//
// AFF: MLX's affine form ("prism-ml/Bonsai-27B-mlx-1bit", MLX packaging): weight a q + b for
// the bit q, a scale a and a bias b (binary16, [N][K/128] each) per group.  With D the table sum
// of +-x over a group and X its plain sum of x, the group adds (a/2) D + (a/2 + b) X.  X of every
// group is summed once per workgroup into LDS after x; the second term does not depend on the
// bits, so each round's biases are read like the scales and folded into the partial sums at
// once, and only the scales stay in registers.
template <int W, int PD, int UMAX, int SQ, bool AFF>
__global__ __launch_bounds__(W * 64) void q1_gemv_lut8_kernel(const uint32_t *__restrict__ wbits,
                                                              const uint16_t *__restrict__ scales,
                                                              const uint16_t *__restrict__ biases,
                                                              const uint16_t *__restrict__ x,
                                                              float *__restrict__ y, int N, int K)
{
    static_assert(UMAX % PD == 0, "a unit's registers are fixed at compile time");
    static_assert(W == 4 || W == 8 || W == 16, "every wave builds an equal share of one half's tables");
    constexpr int EPW = 512 / W;                        // entries of its half's tables each wave builds
    constexpr int NH = EPW / 16;                        // their high nibbles
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = K >> 7;
    const int S = (K + kL8SliceK - 1) / kL8SliceK;      // slices

    // this workgroup's units (8 rows each) and this wave's share: units ub0 + wave + W t
    const int U = (N + 7) / 8;
    const int ub0 = (int)((int64_t)U * blockIdx.x / gridDim.x);
    const int ub1 = (int)((int64_t)U * (blockIdx.x + 1) / gridDim.x);
    const int nw = ub1 - ub0 > wave ? (ub1 - ub0 - wave + W - 1) / W : 0;     // units of this wave

    const int r = lane >> 3, p = lane & 7;              // row of the unit, group of the slice
    const int rq = r & 3;

    // First row of the wave's t-th unit.  The last unit of the matrix starts at row N - 8 when N
    // is not a multiple of 8 (its first rows repeat the unit before, and are written twice with
    // the same value).  A unit slot past the wave's own units still issues every load (so the
    // waits the compiler places stay exact) and is computed but not stored: its scales are the
    // wave's first unit's, and its cells are read from x, which the cache holds (a lane offset
    // is below K bytes, x spans 2K).
    auto unit_row0 = [&](int t) { return min(8 * (ub0 + wave + W * (t < nw ? t : 0)), N - 8); };

    // Unit (s, t) -- slice s, t-th unit: the lane's cell, at the unit's wave-uniform base plus the
    // lane's offset voff of the slice (the group clamped inside a short last slice).
    const char *ubase[UMAX];
#pragma unroll
    for (int t = 0; t < UMAX; ++t)
        ubase[t] = t < nw ? reinterpret_cast<const char *>(wbits) + 16 * (size_t)unit_row0(t) * G
                          : reinterpret_cast<const char *>(x);
    auto load_cell = [&](int t, uint32_t voff, u32x4 &cell) {
        cell = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ubase[t] + voff));
    };
    auto lane_voff = [&](int s) { return 16u * (uint32_t)(r * G + 8 * s + min(p, G - 8 * s - 1)); };
    const char *xb = reinterpret_cast<const char *>(x);

    // Scales (or biases: arr) of slices s0 .. s0 + SQ - 1 of every unit of the wave: lane (r, p)
    // takes that of group 8 s + p of row r (clamped to the row's last group past K), two slices to
    // a register.  A row's 80 bytes of scales (K = 5120) are read together rather than 16 bytes
    // per slice, one slice's worth of the weights apart: between slices the cache would have to
    // hold them while the weights stream.  load_scales issues the loads of units t0 .. t1 - 1,
    // pack_scales pairs them once they are in.
    constexpr int SQ2 = (SQ + 1) / 2;
    auto load_scales = [&](const uint16_t *arr, int s0, int t0, int t1, uint32_t (&raw)[UMAX][SQ]) {
        uint32_t so[SQ];
#pragma unroll
        for (int q = 0; q < SQ; ++q) so[q] = 2u * (uint32_t)(r * G + min(8 * (s0 + q) + p, G - 1));
#pragma unroll
        for (int t = t0; t < t1; ++t) {
            const char *sb = reinterpret_cast<const char *>(arr) + 2 * (size_t)unit_row0(t) * G;
#pragma unroll
            for (int q = 0; q < SQ; ++q) raw[t][q] = *reinterpret_cast<const uint16_t *>(sb + so[q]);
        }
    };
    auto pack_scales = [&](int t0, int t1, const uint32_t (&raw)[UMAX][SQ], uint32_t (&sc)[UMAX][SQ2]) {
#pragma unroll
        for (int t = t0; t < t1; ++t)
#pragma unroll
            for (int q2 = 0; q2 < SQ2; ++q2)
                sc[t][q2] = 2 * q2 + 1 < SQ ? __builtin_amdgcn_perm(raw[t][2 * q2 + 1], raw[t][2 * q2], 0x05040100u)
                                            : raw[t][2 * q2];
    };

    // Tables of slice s: wave w writes entries EPW (w / 2) .. EPW (w / 2) + EPW - 1 of the 64
    // tables of the 64 KB half h = w % 2, one 256-byte row of table columns per entry.  Lane c
    // holds column c of the row: byte i = 2 h + c / 32 of word d = 4 (b / 4) + ((b % 4) - i) % 4,
    // b = c % 32, whose 8 weights are k = 1024 s + 8 (4 d + i) ..; x read clamped inside x past K
    // (such tables belong to groups past K, which count with weight 0).
    const int bh = wave & 1, bq = wave >> 1;
    auto load_x = [&](int s) -> u32x4 {
        const int i = 2 * bh + (lane >> 5), b = lane & 31;
        const int d = 4 * (b >> 2) + (((b & 3) - i) & 3);
        return *reinterpret_cast<const lds_u32x4_t *>(static_cast<uintptr_t>(kL8Tables + 16 * min(128 * s + 4 * d + i, K / 8 - 1)));
    };
    auto build = [&](const u32x4 xv) {
        float xs[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const half2_t pr = as_half2(xv[j]);
            xs[2 * j] = (float)pr[0];
            xs[2 * j + 1] = (float)pr[1];
        }
        // lo[v] = sum_{j<4} (bit j of v ? +x_j : -x_j); hi likewise over x_4..x_7 for the NH high
        // nibbles NH (w / 2) .. NH (w / 2) + NH - 1 of this wave's entries
        float lo[16];
        lo[0] = -((xs[0] + xs[1]) + (xs[2] + xs[3]));
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float tx = 2.f * xs[b];
#pragma unroll
            for (int v = 0; v < (1 << b); ++v) lo[v | (1 << b)] = lo[v] + tx;
        }
        float hi[NH];
#pragma unroll
        for (int hb = 0; hb < NH; ++hb) {
            const int v = NH * bq + hb;
            const float s4 = (v & 1) ? xs[4] : -xs[4], s5 = (v & 2) ? xs[5] : -xs[5];
            const float s6 = (v & 4) ? xs[6] : -xs[6], s7 = (v & 8) ? xs[7] : -xs[7];
            hi[hb] = (s4 + s5) + (s6 + s7);
        }
        store_entries<0, EPW>(bh * 65536 + 256 * (EPW * bq) + 4 * lane, lo, hi);
    };

    // Per-lane lookup constants.  Lookup m takes byte i = (m + rq) % 4 of the word: its selector
    // puts byte 0 of the source (the column offset), byte i of the word (the entry), byte 2 of
    // the source (the 64 KB half) and a zero byte; the source of (step j, lookup m) holds
    // 4 (4 p + (j + i) % 4) + 128 (i & 1) in byte 0 and i >> 1 in byte 2.  (v_perm_b32 selector
    // bytes 0..3 pick bytes of the second operand, 4..7 of the first, 12 gives 0.)
    uint32_t sel[4], src[16];
    u32x4 cell[PD];
    uint32_t raw[UMAX][SQ], sc[UMAX][SQ2];
    float acc[UMAX];
#pragma unroll
    for (int tt = 0; tt < UMAX; ++tt) acc[tt] = 0.f;
    constexpr uint32_t kXsum = kL8Tables;                // + 2K: X of group g at + 4 g (AFF)
    // AFF: add (a/2 + b) X of the lane's groups in slices s0 .. s0 + SQ - 1 (those inside K) to
    // the partial sums of units t0 .. t1 - 1, from the paired scales and the biases in raw
    auto add_bias_terms = [&](int s0, int t0, int t1, const uint32_t (&raw)[UMAX][SQ]) {
#pragma unroll
        for (int q = 0; q < SQ; ++q) {
            const int g = 8 * (s0 + q) + p;             // past K: X = 0 (adds zeros)
            const float xl = lds_f32(kXsum + 2 * K + 4 * min(g, G - 1));
            const float xg = g < G ? xl : 0.f;
#pragma unroll
            for (int t = t0; t < t1; ++t) {
                // a/2 + b as one mixed-precision FMA on the two halves (no fp32 copy of a
                // that the compiler could keep for the slices)
                const float c2 = fmaf(f16_bits_to_f32((uint16_t)(sc[t][q / 2] >> (16 * (q % 2)))), 0.5f,
                                      f16_bits_to_f32((uint16_t)raw[t][q]));
                acc[t] = fmaf(c2, xg, acc[t]);
            }
        }
    };
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int i = (m + rq) & 3;
        sel[m] = 0x0C020000u | ((uint32_t)(4 + i) << 8);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            src[4 * j + m] = (uint32_t)(4 * (4 * p + ((j + i) & 3)) + 128 * (i & 1)) | ((uint32_t)(i >> 1) << 16);
    }

    // x to LDS (after the tables) and the first slice's tables, with the first SQ slices' scales
    // and the first PD units in flight (the loads go out in that order: x, scales, cells, so the
    // first lookups need not wait for every cell of the first slice; 0.3 us less than cells
    // first); the scales are paired once the tables are built.
    {
        constexpr int XR = (kL8MaxK / 8 + W * 64 - 1) / (W * 64);     // 16-byte pieces of x per thread
        const u32x4 *xg = reinterpret_cast<const u32x4 *>(x);
        u32x4 xr[XR];
#pragma unroll
        for (int it = 0; it < XR; ++it) {
            const int c = threadIdx.x + it * W * 64;
            if (c < K / 8) xr[it] = xg[c];
        }
        load_scales(scales, 0, 0, UMAX, raw);
        const uint32_t voff = lane_voff(0);
#pragma unroll
        for (int t = 0; t < PD; ++t) load_cell(t, voff, cell[t]);
#pragma unroll
        for (int it = 0; it < XR; ++it) {
            const int c = threadIdx.x + it * W * 64;
            if (c < K / 8) *reinterpret_cast<lds_u32x4_t *>(static_cast<uintptr_t>(kL8Tables + 16 * c)) = xr[it];
        }
    }
    __syncthreads();
    if constexpr (AFF) {
        // X of group g: wave g mod W adds the group's 128 x, two per lane, then across the wave
        // in a fixed butterfly; lane 0 writes it after x (read once the tables are built)
        for (int g = wave; g < G; g += W) {
            const half2_t pr = as_half2(*reinterpret_cast<const __attribute__((address_space(3))) uint32_t *>(
                static_cast<uintptr_t>(kL8Tables + 256 * g + 4 * lane)));
            float v = (float)pr[0] + (float)pr[1];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
            if (lane == 0) *reinterpret_cast<lds_f32_t *>(static_cast<uintptr_t>(kXsum + 2 * K + 4 * g)) = v;
        }
    }
    build(load_x(0));
    __syncthreads();
    pack_scales(0, UMAX, raw, sc);
    if constexpr (AFF) {                                // the biases, once the scales are paired,
        load_scales(biases, 0, 0, UMAX / 2, raw);       // half the units at a time
        add_bias_terms(0, 0, UMAX / 2, raw);
        load_scales(biases, 0, UMAX / 2, UMAX, raw);
        add_bias_terms(0, UMAX / 2, UMAX, raw);
    }
    for (int s0 = 0; s0 < S; s0 += SQ) {
        if (s0 > 0) {                                   // K > 1024 SQ: the next SQ slices' scales
            load_scales(scales, s0, 0, UMAX / 2, raw);  // (and biases), half the units at a time
            pack_scales(0, UMAX / 2, raw, sc);
            load_scales(scales, s0, UMAX / 2, UMAX, raw);
            pack_scales(UMAX / 2, UMAX, raw, sc);
            if constexpr (AFF) {
                load_scales(biases, s0, 0, UMAX / 2, raw);
                add_bias_terms(s0, 0, UMAX / 2, raw);
                load_scales(biases, s0, UMAX / 2, UMAX, raw);
                add_bias_terms(s0, UMAX / 2, UMAX, raw);
            }
        }
        static_for<0, SQ>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            const int s = s0 + q;
            if (s < S) {
                const bool last = s == S - 1;
                const bool live_group = 8 * s + p < G;  // groups past K (a short last slice) count 0
                const uint32_t voff = lane_voff(s), voffn = lane_voff(last ? s : s + 1);
                static_for<0, UMAX>([&](auto ic) {
                    // Every unit slot is computed (a slot past the wave's units is not stored),
                    // and every slot issues one load: with no branches the compiler's waits count
                    // exactly PD - 1 loads still in flight.
                    constexpr int tt = decltype(ic)::value, b = tt % PD;
                    float tv[16];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int m = 0; m < 4; ++m)
                            tv[4 * j + m] = lds_f32(__builtin_amdgcn_perm(cell[b][j], src[4 * j + m], sel[m]));
                    const float part =
                        (((tv[0] + tv[1]) + (tv[2] + tv[3])) + ((tv[4] + tv[5]) + (tv[6] + tv[7]))) +
                        (((tv[8] + tv[9]) + (tv[10] + tv[11])) + ((tv[12] + tv[13]) + (tv[14] + tv[15])));
                    const uint16_t sbits = (uint16_t)(sc[tt][q / 2] >> (16 * (q % 2)));
                    // AFF: (a/2) D as a (D/2), halving being exact, so the fp16 scale still
                    // feeds the mixed-precision FMA straight from its half of the register
                    const float pv = AFF ? 0.5f * part : part;
                    acc[tt] = live_group ? fmaf(f16_bits_to_f32(sbits), pv, acc[tt]) : acc[tt];
                    // the unit PD ahead into the registers just used; past the last slice a
                    // re-read of x, which the cache holds
                    constexpr int ta = tt + PD;
                    if constexpr (ta < UMAX) {
                        load_cell(ta, voff, cell[b]);
                    } else {
                        const char *bp = last ? xb : ubase[ta - UMAX];
                        cell[b] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(bp + voffn));
                    }
                });
                if (!last) {
                    __syncthreads();                    // every wave is done with these tables
                    build(load_x(s + 1));
                    __syncthreads();
                }
            }
        });
    }
    // add each row's 8 group partials (lanes 8 r .. 8 r + 7) in a fixed order and store; the
    // lane's row is taken afresh from the lane count (mbcnt), which the compiler recomputes here
    // instead of keeping r live through the slices
    const int lane_end = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
#pragma unroll
    for (int tt = 0; tt < UMAX; ++tt) {
        if (tt < nw) {
            const float v = sum8(acc[tt]);
            const int row = min(8 * (ub0 + wave + W * tt), N - 8) + (lane_end >> 3);
            if ((lane_end & 7) == 0) y[row] = v;
        }
    }
}

template <int W, int PD, int UMAX, int SQ, bool AFF>
hipError_t launch_lut8_t(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases, const uint16_t *x,
                         float *y, int N, int K, hipStream_t stream)
{
    if (N < 8 || K > (AFF ? kL8MaxKAff : kL8MaxK)) return hipErrorInvalidValue;
    // one workgroup per CU, or more where a CU's share would exceed W UMAX units
    const int64_t U = ((int64_t)N + 7) / 8;
    const int64_t cus = device_cus();
    const int64_t grid = std::max(std::min(U, cus), (U + W * UMAX - 1) / (W * UMAX));
    const void *fn = reinterpret_cast<const void *>(&q1_gemv_lut8_kernel<W, PD, UMAX, SQ, AFF>);
    const size_t lds = (size_t)kL8Tables + 2 * (size_t)K + (AFF ? 4 * (size_t)(K / 128) : 0);
    if (!set_lds_limit(fn, kLdsPerCu)) return hipErrorInvalidValue;
    void *args[] = {&wbits, &scales, &biases, &x, &y, &N, &K};
    return launch_kernel(fn, __PRETTY_FUNCTION__, dim3((unsigned)grid), dim3(64 * W), args, lds, stream);
}

}  // namespace

bool lut8_fits(int N, int K) { return N >= 8 && K <= kL8MaxK; }
bool lut8a_fits(int N, int K) { return N >= 8 && K <= kL8MaxKAff; }

hipError_t launch_lut8(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x, float *y, int N, int K,
                       hipStream_t stream)
{
    return launch_lut8_t<16, 8, 8, 5, false>(wbits, scales, nullptr, x, y, N, K, stream);
}

hipError_t launch_lut8a(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases, const uint16_t *x,
                        float *y, int N, int K, hipStream_t stream)
{
    return launch_lut8_t<16, 4, 8, 5, true>(wbits, scales, biases, x, y, N, K, stream);
}

}  // namespace bonsai
