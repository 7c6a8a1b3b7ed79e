// gemm_skinny.hip -- y[M][N] = x[M][K] W^T for a few dozen rows of x (16 < M <= 128), binary or
// ternary g128 weights, on the matrix cores.
//
// A pass of the target model over several draft tokens at once ("1-bit Bonsai 27B" model card,
// speculative decoding with the DSpark drafter: a handful of tokens checked per target pass) is
// a product with M in the tens: too many rows of x for the decode kernels, which take 16 of
// them per pass over the weights, and too few to fill the 128 x 256 prefill tiles (N = 13824
// makes 54 of them).  Here every weight is expanded once and serves all rows of x.
//
// Tiling.  A workgroup of 4 waves (one per SIMD) owns 64 weight rows and all rows of x; wave w
// takes a quarter of the groups of K.  Per k16 slice a wave runs MB x 2 v_mfma_f32_32x32x16_f16:
// A = 32 rows of x, B = 32 weight rows expanded from their codes with the group scale folded in
// (the prefill GEMM's operands: +-s for a sign bit, 0 / +-2s for a ternary code), so one
// accumulator set runs across all groups.  The four waves' partial sums meet in LDS and are
// added in a fixed order.
//
// x.  Every workgroup reads all of x, from the cache.  A lane's A operand is 16 bytes of one row
// of x, and the 32 rows of a block lie K apart, so loading it straight into registers touches
// 32 lines per instruction, which the L1 does not keep between slices (timed: 40 us at M = 64
// against 35 for 16-row passes).  Instead each wave copies its rows of x, 64 k at a time, into
// its own LDS ring by direct global->LDS loads of whole lines (chunk c of row m at 16-byte slot
// c ^ (m % 8), so the A reads of 8 lanes fall on distinct banks), and reads the operands from
// there.  The copies are ordered against those reads by waits on the copies themselves, with
// exact counts, since each wave reads only what it copied.
//
// Pipeline.  The A fragments of the next k16 slice are read from LDS and its B fragments
// expanded while the current slice's MFMAs run (one wave per SIMD: nothing else would hide the
// LDS latency); the last slice of a stage waits for the next stage's copies and fetches its
// first operands.
//
// Bound.  The MFMA work is 2 M N K flops; each workgroup also reads all of x (2 M K bytes) from
// the cache.  At M = 64, N = 13824, K = 5120: 9.1 GFLOP and 216 workgroups of 640 KB of x.
#include <algorithm>

#include "device.h"
#include "expand.h"
#include "launch.h"

namespace bonsai {
namespace {

typedef float float16_t __attribute__((ext_vector_type(16)));

template <int I>
struct IC {
    static constexpr int value = I;
};

constexpr int kSkRows = 64;                 // weight rows per workgroup
constexpr int kSkWaves = 4;
// sched_group_barrier masks
constexpr int SG_MFMA = 0x008, SG_VALU = 0x002, SG_DS_READ = 0x100;

// MB: blocks of 32 rows of x (M <= 32 MB).  NB: stages of x (64 k each) in a wave's ring.
template <bool TERN, int MB, int NB>
__global__ __launch_bounds__(kSkWaves * 64) void skinny_gemm_kernel(const uint32_t *__restrict__ codes,
                                                                    const uint16_t *__restrict__ scales,
                                                                    const uint16_t *__restrict__ x,
                                                                    float *__restrict__ y, int M, int N, int K)
{
    static_assert(NB == 2 || NB == 4, "whole groups of stages ahead");
    constexpr int CW = TERN ? 8 : 4;                // code words per (row, group)
    extern __shared__ float red[];                  // the waves' partial sums, for the reduction
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, q = lane >> 5;
    const int G = K >> 7;
    const int n0 = blockIdx.x * kSkRows;
    // this wave's groups
    const int g0 = G * wave / kSkWaves, g1 = G * (wave + 1) / kSkWaves;

    float16_t acc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][t][i] = 0.f;

    // this wave's LDS ring of x stages (64 k of the MB blocks of 32 rows: MB x 4 KB each)
    constexpr int STAGE = MB * 4096;
    const uint32_t ring = (uint32_t)(wave * NB * STAGE);
    typedef __attribute__((address_space(3))) void lds_void_t;
    typedef __attribute__((address_space(1))) const void glb_void_t;
    typedef __attribute__((address_space(3))) half8_t lds_half8_t;
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;
    typedef __attribute__((address_space(3))) uint16_t lds_u16_t;

    // after the x ring, three groups of codes and scales: 64 rows x 16 (ternary 32) bytes of
    // codes and 64 dwords whose low halves hold the scales
    constexpr int GCODES = 64 * 4 * CW, GSLOT = GCODES + 256;
    const uint32_t gring = (uint32_t)(kSkWaves * NB * STAGE + wave * 3 * GSLOT);

    if (g0 < g1) {
        // copy the codes and scales of group g (clamped to the wave's last group, so the copies
        // past it stay in bounds and are simply not used) into group slot r: lane i carries row
        // n0 + i (rows past N repeat row N - 1)
        const int nl = min(n0 + lane, N - 1);
        auto copy_group = [&](int g, int r) {
            const int gg = min(g, g1 - 1);
            const uint32_t slot = gring + (uint32_t)(r * GSLOT);
#pragma unroll
            for (int h = 0; h < CW / 4; ++h)
                __builtin_amdgcn_global_load_lds((glb_void_t *)(codes + ((size_t)nl * G + gg) * CW + 4 * h),
                                                 (lds_void_t *)(uintptr_t)(slot + 1024 * h), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((glb_void_t *)(scales + (size_t)nl * G + gg),
                                             (lds_void_t *)(uintptr_t)(slot + GCODES), 2, 0, 0);
            asm volatile("" : : : "memory");           // the wait counts assume this issue order
        };
        constexpr int GC = CW / 4 + 1;                  // copies per group
        // copy stage st of the wave (k = 128 g0 + 64 st .., clamped to the wave's last stage)
        // into ring slot st % NB: instruction u carries rows 8 u .. 8 u + 7 of the stage (lane:
        // row 8 u + lane / 8, slot lane % 8, which holds chunk (lane % 8) ^ (row % 8))
        const int nst = 2 * (g1 - g0);
        auto copy_stage = [&](int st) {
            const int ss = min(st, nst - 1);
            const int k0 = 128 * g0 + 64 * ss;
            const uint32_t slot = ring + (uint32_t)((st % NB) * STAGE);
#pragma unroll
            for (int u = 0; u < 4 * MB; ++u) {
                const int m = 8 * u + (lane >> 3);
                const int c = (lane & 7) ^ (m & 7);
                const uint16_t *src = x + (size_t)min(m, M - 1) * K + k0 + 8 * c;
                __builtin_amdgcn_global_load_lds((glb_void_t *)src, (lds_void_t *)(uintptr_t)(slot + 1024 * u), 16, 0, 0);
            }
            asm volatile("" : : : "memory");
        };
        // copies in the order the loop keeps: a group's two stages' copies, then the group three
        // ahead (NB / 2 groups of stages ahead)
        copy_group(g0, 0);
        if constexpr (NB == 2) copy_group(g0 + 1, 1);
#pragma unroll
        for (int hh = 0; hh < NB / 2; ++hh) {
            copy_stage(2 * hh);
            copy_stage(2 * hh + 1);
            copy_group(g0 + (NB == 2 ? 2 : hh + 1), NB == 2 ? 2 : hh + 1);
        }

        // Operands of one k16 slice: buffer c holds the current slice's, c ^ 1 the next one's,
        // fetched and expanded under the current slice's MFMAs.
        half8_t af[2][MB], bf[2][2];
        u32x4 cw[2][CW / 4];                            // code words of the group being expanded
        uint32_t cs[2];                                 // its scale pairs
        auto read_codes = [&](int r) {
            const uint32_t gslot = gring + (uint32_t)(r * GSLOT);
            const uint32_t flip = TERN ? 0u : 0x80008000u;     // binary (-s, -s), ternary (s, s)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int row = 32 * t + l32;
#pragma unroll
                for (int hh = 0; hh < CW / 4; ++hh)
                    cw[t][hh] = *reinterpret_cast<const lds_u32x4_t *>((uintptr_t)(gslot + 1024 * hh + 16 * row));
                const uint32_t sv = *reinterpret_cast<const lds_u16_t *>((uintptr_t)(gslot + GCODES + 4 * row));
                cs[t] = (sv | (sv << 16)) ^ flip;
            }
        };
        // A of slice jj (0..3) of stage st, B of slice j (0..7) of the group whose codes are in cw
        auto read_a = [&](int buf, int st, int jj) {
            const uint32_t slot = ring + (uint32_t)((st % NB) * STAGE);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int m = 32 * mb + l32;
                af[buf][mb] = *reinterpret_cast<const lds_half8_t *>(
                    (uintptr_t)(slot + 128 * m + 16 * ((2 * jj + q) ^ (m & 7))));
            }
        };
        auto make_b = [&](int buf, int j) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if constexpr (TERN) bf[buf][t] = expand8_tern(cw[t][j >> 2][j & 3], q, cs[t]);
                else bf[buf][t] = expand8(cw[t][0][j >> 1], j, q, cs[t]);
            }
        };
        auto mfma = [&](int buf) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    acc[mb][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[buf][mb], bf[buf][t], acc[mb][t], 0, 0, 0);
        };

        // Every group issues the same copies in the same order (past the wave's range they are
        // clamped repeats): after stage s's copies come those of the later stages, and a group's
        // copies after each odd stage (a group's second).  Stage 0 has landed once at most the
        // copies issued after it in the prologue are outstanding.
        vm_wait<(NB - 1) * 4 * MB + (NB / 2) * GC>();
        read_codes(0);
        read_a(0, 0, 0);
        make_b(0, 0);

        // Group g of the wave in group slot r.  The last slice of stage st fetches the first
        // operands of stage st + 1 (and, at the group's end, the next group's codes, which were
        // copied before that stage): it waits until at most the copies issued after stage st + 1
        // are outstanding -- the stages up to st + NB - 1 and a group's copies after each odd one
        // of them -- then issues the copies of stage st + NB into the slot stage st used.
        auto do_group = [&](auto rc, int g) {
            constexpr int r = decltype(rc)::value;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int st = 2 * (g - g0) + h;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int cur = jj & 1, nxt = cur ^ 1;
                    if (jj < 3) {
                        read_a(nxt, st, jj + 1);
                        make_b(nxt, 4 * h + jj + 1);
                    } else {
                        // st has the parity of h: NB / 2 - h odd stages among st + 1 .. st + NB - 1
                        if (h == 0) vm_wait<(NB - 2) * 4 * MB + (NB / 2) * GC>();
                        else vm_wait<(NB - 2) * 4 * MB + (NB / 2 - 1) * GC>();
                        read_a(nxt, st + 1, 0);
                        if (h == 0) {
                            make_b(nxt, 4);
                        } else {
                            read_codes((r + 1) % 3);
                            make_b(nxt, 0);
                        }
                    }
                    mfma(cur);
#pragma unroll
                    for (int i = 0; i < 2 * MB; ++i) {
                        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                        if (i < MB) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(SG_VALU, 24 / (2 * MB), 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                copy_stage(st + NB);
            }
            copy_group(g + 3, r);
        };
        // whole triples of groups with no branch inside, then the one or two left
        int gb = g0;
        for (; gb + 3 <= g1; gb += 3) {
            do_group(IC<0>{}, gb);
            do_group(IC<1>{}, gb + 1);
            do_group(IC<2>{}, gb + 2);
        }
        if (gb < g1) do_group(IC<0>{}, gb);
        if (gb + 1 < g1) do_group(IC<1>{}, gb + 1);
    }
    vm_wait<0>();                               // no copy into LDS outlives its reads
    __syncthreads();                            // the rings become the reduction's space

    // the four waves' partials: wave w writes its accumulators at red[w][mb][t][i][lane], then
    // every thread adds the four waves' values of its outputs in wave order and stores them.
    // D layout (32 x 32): lane holds column lane % 32, rows 8 (i / 4) + 4 (lane / 32) + i % 4.
    constexpr int PER_WAVE = MB * 2 * 16 * 64;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) red[wave * PER_WAVE + ((mb * 2 + t) * 16 + i) * 64 + lane] = acc[mb][t][i];
    __syncthreads();
    for (int e = threadIdx.x; e < PER_WAVE; e += kSkWaves * 64) {
        float v = red[e];
#pragma unroll
        for (int w = 1; w < kSkWaves; ++w) v += red[w * PER_WAVE + e];
        const int ln = e & 63, i = (e >> 6) & 15, t = (e >> 10) & 1, mb = e >> 11;
        const int m = 32 * mb + 8 * (i >> 2) + 4 * (ln >> 5) + (i & 3);
        const int n = n0 + 32 * t + (ln & 31);
        if (m < M && n < N) y[(size_t)m * N + n] = TERN ? 0.5f * v : v;
    }
}

template <bool TERN, int MB, int NB>
hipError_t launch_skinny_t(const uint32_t *codes, const uint16_t *scales, const uint16_t *x, float *y, int M, int N,
                           int K, hipStream_t stream)
{
    const void *fn = reinterpret_cast<const void *>(&skinny_gemm_kernel<TERN, MB, NB>);
    // the x rings, reused by the reduction (4 waves x MB x 8 KB of partial sums)
    constexpr size_t gslot = 64 * 4 * (TERN ? 8 : 4) + 256;   // a group's codes and scales
    const size_t lds = std::max<size_t>((size_t)kSkWaves * (NB * MB * 4096 + 3 * gslot),
                                        sizeof(float) * kSkWaves * MB * 2 * 16 * 64);
    if (!set_lds_limit(fn, (int)lds)) return hipErrorInvalidValue;
    void *args[] = {&codes, &scales, &x, &y, &M, &N, &K};
    return launch_kernel(fn, __PRETTY_FUNCTION__, dim3((unsigned)((N + kSkRows - 1) / kSkRows)), dim3(kSkWaves * 64),
                         args, lds, stream);
}

}  // namespace

int skinny_max_m() { return 128; }

hipError_t launch_skinny(bool tern, const uint32_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                         int M, int N, int K, hipStream_t stream)
{
    if (M < 1 || M > skinny_max_m() || N < 1 || K < 128) return hipErrorInvalidValue;
    if (M <= 32)
        return tern ? launch_skinny_t<true, 1, 4>(codes, scales, x, y, M, N, K, stream)
                    : launch_skinny_t<false, 1, 4>(codes, scales, x, y, M, N, K, stream);
    if (M <= 64)
        return tern ? launch_skinny_t<true, 2, 4>(codes, scales, x, y, M, N, K, stream)
                    : launch_skinny_t<false, 2, 4>(codes, scales, x, y, M, N, K, stream);
    return tern ? launch_skinny_t<true, 4, 2>(codes, scales, x, y, M, N, K, stream)
                : launch_skinny_t<false, 4, 2>(codes, scales, x, y, M, N, K, stream);
}

}  // namespace bonsai
