// q1_gemm.hip -- binary g128 prefill GEMM on gfx950 MFMA:  y[M][N] = x[M][K] W^T.
//
// Prefill is the compute-bound phase ("1-bit Bonsai 27B" model card, cross-platform
// throughput: pp512), so the contraction runs on the matrix cores (v_mfma_f32_32x32x16_f16,
// fp16 in, fp32 accumulate).  The weights reach the MFMA B operand straight from the packed
// sign words: each lane expands its bits to binary16 +-s in registers (exact: -s is s with the
// sign bit flipped), so the group scale is folded into the operand and one accumulator set
// runs across all groups.  No FP16 copy of W is written anywhere.
//
// Tiling.  A workgroup of 4 waves (one per SIMD) computes a 128 (M) x 256 (N) tile; wave w
// owns columns 64w .. 64w+63 of it, all 128 rows, as 4 x 2 MFMA tiles of 32 x 32.  K advances
// 64 per step.
//
// Operand staging.
//  * X: 128 rows x 128 B per step, copied into a 4-deep LDS ring by direct global->LDS loads
//    (8 rows x 128 B per instruction), the 16-byte chunk c of row r stored at
//    128 r + 16 (c ^ ((r >> 1) & 7)) so the A-operand reads are free of bank conflicts.
//  * W: sign words and scales travel in 1024-k chunks (128 B of words and 8 scales per
//    column), double buffered in LDS and copied one chunk ahead by direct global->LDS loads:
//    8 columns x 128 B per instruction (whole lines), and the scales either as one 16-byte copy
//    per column (K a multiple of 1024) or one 2-byte copy per column and group.  Cell u (steps
//    2u, 2u+1) of column c sits at 128 c + 16 (u ^ ((c >> 1) & 7)).  A lane reads its two
//    columns' cell every other step in a small asm block that also waits for it: these reads
//    are ordered against the copies by the barriers, and keeping them out of the compiler's
//    view keeps its conservative copy-versus-read waits off the A-operand reads.
//
// Pipeline.  Within a step, the A fragments and the expanded B fragments of the next k16
// slice are produced while the 8 MFMAs of the current one run; sched_group_barrier interleaves
// them (MFMA, LDS read, VALU, ...) so the matrix core stays busy.  Once per step, between the
// third and fourth k16 slice, each wave waits for its own copies of the next X stage
// (s_waitcnt with an exact count of the loads issued after them), a bare s_barrier makes all
// waves' copies visible (__syncthreads would also drain every later stage), the stage three
// steps ahead is issued into the slot just freed, and the last slice runs while the first
// operands of the next step are fetched.  Every step issues the same loads (clamped to the
// last chunk and stage near the end, into buffers no longer read), so the counts hold on every
// path; steps past K in the last chunk skip only their arithmetic.
//
// Sign expansion in natural k order.  An MFMA lane holds 8 consecutive k of its operand as 4
// half pairs (k, k+1).  Merging a word with itself shifted (u = bits 0..15 | bits 1..16 in the
// high half, u2 likewise for bits 16..31) places bits k and k+1 at positions q and 16+q, so
// one shift puts both on the binary16 sign bits and an and-xor with (-s, -s) yields (+-s, +-s).
#include <limits.h>

#include <type_traits>
#include <utility>

#include "device.h"
#include "expand.h"
#include "launch.h"

namespace bonsai {
namespace {

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int NS = 4;                           // X stages in the LDS ring
constexpr int XTILE = BM * BK * 2;              // 16 KB per stage
// K-steps per LDS chunk of codes: 1024 k of sign words or 512 k of ternary codes, 128 B per
// column either way (8 cells of 16 bytes)
template <bool TERN> constexpr int chunk_steps() { return TERN ? 8 : 16; }
constexpr int WCH = BN * 128;                   // 32 KB of codes per chunk
constexpr int SCH = BN * 32;                    // 8 KB of scales per chunk (room for one dword per scale)
constexpr int LDS_BYTES = NS * XTILE + 2 * WCH + 2 * SCH;   // 144 KB

typedef float float16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glb_void_t;

// s_waitcnt vmcnt(n), as an asm statement no memory access moves across
template <int n>
__device__ __forceinline__ void wait_vmcnt()
{
    vm_wait<n>();
}

// sched_group_barrier masks
constexpr int SG_MFMA = 0x008, SG_VALU = 0x002, SG_DS_READ = 0x100;

// Scale copies of one chunk per column: binary SMODE 16, one 16-byte copy of the chunk's 8
// scales (K % 1024 == 0), or SMODE 2, one 2-byte copy per group (low half of a dword); ternary
// SMODE 4, one 4-byte copy per pair of the chunk's 4 groups (G even), or SMODE 2 per group.
template <bool TERN, int SMODE> constexpr int scale_copies() { return TERN ? (SMODE == 4 ? 2 : 4) : (SMODE == 16 ? 1 : 8); }

// Copies of the next chunk issued at mid-step j: binary, sign-word copy j (j < 8) and then the
// scales at position 8 (SMODE 16) or 8 .. 15; ternary (8 steps per chunk), code copies 2j and
// 2j + 1 (j < 4) and then scale copy j - 4.  A copy issued at mid-step j has landed by the wait
// of mid-step j + 3, so every copy lands before the first read of what it brings: the next
// chunk's cell 0 and first scales are read at the end of the chunk's last step.
template <bool TERN, int SMODE> constexpr int copies_at(int j)
{
    return TERN ? (j < 4 ? 2 : (j - 4 < scale_copies<TERN, SMODE>() ? 1 : 0))
                : (j < 8 ? 1 : 0) + (SMODE == 16 ? (j == 8 ? 1 : 0) : (j >= 8 ? 1 : 0));
}

template <int... J, class F>
__device__ __forceinline__ void for_each_step(std::integer_sequence<int, J...>, F &&f)
{
    (f(std::integral_constant<int, J>{}), ...);
}

template <bool TERN, int SMODE>
__global__ __launch_bounds__(256) void q1_gemm_kernel(const uint32_t *__restrict__ wbits,
                                                      const uint16_t *__restrict__ scales,
                                                      const uint16_t *__restrict__ x,
                                                      float *__restrict__ y, int M, int N, int K)
{
    // One LDS object (X ring, sign-word chunks, scale chunks): with a single object the
    // compiler's copy-versus-read waits stay off the A-operand reads of the ring.
    __shared__ __attribute__((aligned(16))) char xs[LDS_BYTES];
    char *const wls = xs + NS * XTILE;
    char *const sls = wls + 2 * WCH;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = lane >> 5, l32 = lane & 31;
    const int tiles_n = (N + BN - 1) / BN;
    const int m0 = (blockIdx.x / tiles_n) * BM, n0 = (blockIdx.x % tiles_n) * BN;
    constexpr int CH = chunk_steps<TERN>();
    const int G = K >> 7;                       // groups per row
    const int U = TERN ? 2 * G : G;             // 16-byte units of codes per row
    const int KT = K / BK;
    const int nchunks = (KT + CH - 1) / CH;

    // X staging: this wave issues instructions 4 wave .. 4 wave + 3 of a stage's 16
    // (8 rows x 128 B each): lane -> row 8i + lane/8, chunk (lane%8) ^ ((row >> 1) & 7)
    const u32x4 *xg = reinterpret_cast<const u32x4 *>(x);           // row m, chunk c at m * (K/8) + c
    size_t xsrc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 8 * (4 * wave + j) + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        xsrc[j] = (size_t)min(m0 + r, M - 1) * (K >> 3) + c;
    }

    // W chunk copies: instruction i of this wave covers columns 64 wave + 8 i .. +7, 128 B each;
    // lane -> column 64 wave + 8 i + lane / 8, 16-byte piece (lane % 8) ^ ((column >> 1) & 7)
    const u32x4 *wsrc[8];
    int wu[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = 64 * wave + 8 * i + (lane >> 3);
        wu[i] = (lane & 7) ^ ((c >> 1) & 7);
        wsrc[i] = reinterpret_cast<const u32x4 *>(wbits) + (size_t)min(n0 + c, N - 1) * U;
    }
    const uint16_t *ssrc = scales + (size_t)min(n0 + 64 * wave + lane, N - 1) * G;

    auto issue_x = [&](int kt, int slot) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_global_load_lds((glb_void_t *)(xg + xsrc[j] + kt * (BK / 8)),
                                             (lds_void_t *)(xs + slot * XTILE + (4 * wave + j) * 1024), 16, 0, 0);
    };
    auto issue_w = [&](int cc, int par, int i) {
        __builtin_amdgcn_global_load_lds((glb_void_t *)(wsrc[i] + min(cc * 8 + wu[i], U - 1)),
                                         (lds_void_t *)(wls + par * WCH + (64 * wave + 8 * i) * 128), 16, 0, 0);
    };
    constexpr int GPC = TERN ? 4 : 8;           // groups per chunk
    auto issue_s = [&](int cc, int par, int g) {
        if constexpr (!TERN && SMODE == 16)      // the chunk's 8 scales of column 64 wave + lane
            __builtin_amdgcn_global_load_lds((glb_void_t *)(ssrc + min(cc * 8, G - 8)),
                                             (lds_void_t *)(sls + par * SCH + (64 * wave) * 16), 16, 0, 0);
        else if constexpr (TERN && SMODE == 4)   // groups 2g, 2g + 1 of the chunk, one dword per column
            __builtin_amdgcn_global_load_lds((glb_void_t *)(ssrc + min(cc * GPC + 2 * g, G - 2)),
                                             (lds_void_t *)(sls + par * SCH + (g * 256 + 64 * wave) * 4), 4, 0, 0);
        else                                      // group g of the chunk, low half of a dword per column
            __builtin_amdgcn_global_load_lds((glb_void_t *)(ssrc + min(cc * GPC + g, G - 1)),
                                             (lds_void_t *)(sls + par * SCH + (g * 256 + 64 * wave) * 4), 2, 0, 0);
    };

    float16_t acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

    half8_t af[2][4], bf[2][2];                  // operands of the current / next k16 slice
    // code words of the step being expanded (binary: 2 words, the cell's other 2 saved for the
    // next step; ternary: the cell's 4 words) and the scale pair, (-s, -s) binary or (s, s) ternary
    uint32_t wcur[2][4], cs[2];
    uint32_t wnxt[2][2];
    const uint32_t wls_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char *)wls);
    const uint32_t sls_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char *)sls);

    auto read_a = [&](int slot, int s, int buf) {
        const char *xb = xs + slot * XTILE;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int r = 32 * mt + l32;
            const int c = 2 * s + q;
            af[buf][mt] = *reinterpret_cast<const half8_t *>(xb + 128 * r + 16 * (c ^ ((r >> 1) & 7)));
        }
    };
    // cell u of the chunk in buffer par: both columns' words (binary: steps 2u, 2u + 1, group
    // u; ternary: step u, group u / 2) and the group's scales, waited for inside the block; the
    // outputs are early-clobber so that no output register doubles as an address the block has
    // yet to use
    auto read_cell = [&](int par, int u) {
        uint32_t aw[2], as[2];
        const int g = TERN ? u >> 1 : u;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int c = 64 * wave + 32 * t + l32;
            aw[t] = wls_base + par * WCH + c * 128 + 16 * (u ^ ((c >> 1) & 7));
            if constexpr (!TERN && SMODE == 16) as[t] = sls_base + par * SCH + c * 16 + 2 * g;
            else if constexpr (TERN && SMODE == 4) as[t] = sls_base + par * SCH + ((g >> 1) * 256 + c) * 4 + 2 * (g & 1);
            else as[t] = sls_base + par * SCH + (g * 256 + c) * 4;
        }
        u32x4 w0, w1;
        uint32_t s0, s1;
        asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_u16 %2, %6\n\t"
                     "ds_read_u16 %3, %7\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(w0), "=&v"(w1), "=&v"(s0), "=&v"(s1)   // early clobber: a load landing
                     : "v"(aw[0]), "v"(aw[1]), "v"(as[0]), "v"(as[1])  // must not overwrite a later
                     : "memory");                                      // load's address
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wcur[0][e] = w0[e];
            wcur[1][e] = w1[e];
        }
        if constexpr (!TERN) {
            wnxt[0][0] = w0[2]; wnxt[0][1] = w0[3];
            wnxt[1][0] = w1[2]; wnxt[1][1] = w1[3];
        }
        const uint32_t flip = TERN ? 0u : 0x80008000u;     // binary (-s, -s), ternary (s, s)
        cs[0] = (s0 | (s0 << 16)) ^ flip;
        cs[1] = (s1 | (s1 << 16)) ^ flip;
    };
    // words of step j of the chunk in buffer par: ternary, cell j; binary, a cell read at even
    // j, else its saved half
    auto read_w = [&](int par, int j) {
        if (TERN) read_cell(par, j);
        else if ((j & 1) == 0) read_cell(par, j >> 1);
        else {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                wcur[t][0] = wnxt[t][0];
                wcur[t][1] = wnxt[t][1];
            }
        }
    };
    auto make_b = [&](int s, int buf) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
            bf[buf][t] = TERN ? expand8_tern(wcur[t][s], q, cs[t]) : expand8(wcur[t][s >> 1], s, q, cs[t]);
    };
    auto mfma8 = [&](int buf) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                acc[mt][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[buf][mt], bf[buf][t], acc[mt][t], 0, 0, 0);
    };

    // prologue: chunk 0 and X stages 0 .. NS - 2
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_w(0, 0, i);
#pragma unroll
    for (int g = 0; g < scale_copies<TERN, SMODE>(); ++g) issue_s(0, 0, g);
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue_x(min(st, KT - 1), st);
    wait_vmcnt<4 * (NS - 2)>();                 // chunk 0 and stage 0 landed
    asm volatile("s_barrier" ::: "memory");
    read_w(0, 0);
    read_a(0, 0, 0);
    make_b(0, 0);

    // Mid-step m issues stage m + 3 and then that position's chunk copies for the next chunk
    // (copies_at).
    // Every chunk does so (the last one re-copies itself into the idle buffer), so the number
    // of copies issued after any stage is known at compile time.
    for (int cc = 0; cc < nchunks; ++cc) {
        const int cn = min(cc + 1, nchunks - 1);
        const int par = cc & 1;
        auto step = [&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr int slot = j % NS;
            const int kt = cc * CH + j;
            const bool live = kt < KT;
            // k16 slices 0..2: operands of slice s + 1 are fetched / expanded under the MFMAs of s
            if (live) {
#pragma unroll
                for (int s = 0; s < 3; ++s) {
                    read_a(slot, s + 1, (s + 1) & 1);
                    make_b(s + 1, (s + 1) & 1);
                    mfma8(s & 1);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                        if (i < 4) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(SG_VALU, 3, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // Stage kt + 1 has landed once only the copies issued after it are outstanding:
            // mid-step kt - 2's chunk copies, then stage kt + 2 and mid-step kt - 1's.
            constexpr int jm2 = (j + CH - 2) % CH, jm1 = (j + CH - 1) % CH;
            constexpr int pm2 = copies_at<TERN, SMODE>(jm2);
            constexpr int pm1 = copies_at<TERN, SMODE>(jm1);
            if (j < 2 && cc == 0) {
                if (j == 0) wait_vmcnt<4>();
                else wait_vmcnt<4 + copies_at<TERN, SMODE>(0)>();   // mid-step 0: stage 3, then its copies
            } else {
                wait_vmcnt<pm2 + 4 + pm1>();
            }
            asm volatile("s_barrier" ::: "memory");
            issue_x(min(kt + NS - 1, KT - 1), (slot + NS - 1) % NS);
            if constexpr (TERN) {
                if constexpr (j < 4) {
                    issue_w(cn, par ^ 1, 2 * j);
                    issue_w(cn, par ^ 1, 2 * j + 1);
                } else if constexpr (j - 4 < scale_copies<TERN, SMODE>()) {
                    issue_s(cn, par ^ 1, j - 4);
                }
            } else {
                if constexpr (j < 8) issue_w(cn, par ^ 1, j);
                else if constexpr (SMODE == 16) { if constexpr (j == 8) issue_s(cn, par ^ 1, 0); }
                else issue_s(cn, par ^ 1, j - 8);
            }
            // slice 3, with the first operands of step kt + 1 fetched under it
            if (live) {
                read_w(j == CH - 1 ? par ^ 1 : par, (j + 1) % CH);
                read_a((slot + 1) % NS, 0, 0);
                mfma8(1);
                make_b(0, 0);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                    if (i < 4) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
                    if (i >= 1) __builtin_amdgcn_sched_group_barrier(SG_VALU, 4, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        for_each_step(std::make_integer_sequence<int, CH>{}, step);
    }
    wait_vmcnt<0>();                            // no copy into LDS outlives the workgroup

    // D layout (32 x 32): lane holds column lane % 32, rows 8 (i / 4) + 4 (lane / 32) + i % 4
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int col = n0 + 64 * wave + 32 * t + l32;
            if (col >= N) continue;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int rowm = m0 + 32 * mt + 8 * (i >> 2) + 4 * q + (i & 3);
                if (rowm < M) y[(size_t)rowm * N + col] = TERN ? 0.5f * acc[mt][t][i] : acc[mt][t][i];
            }
        }
}

}  // namespace

// Up to 16 rows of x the small-M kernel (one pass of 16 rows of x over the weights) is the
// fastest; from 17 to 128 rows the skinny GEMM (every weight expanded once for all rows of x,
// gemm_skinny.hip), then the 128 x 256 tiles.  Measured at N = 13824, K = 5120 (binary;
// ternary alike): M = 16: 10.6 us small-M, 11.9 skinny; M = 32: 18.6 / 12.2; M = 64: 33.9 /
// 17.2; M = 128: 51.3 on the tiles (54 of them, most CUs idle), 28.0 skinny.
constexpr int kSmallM = 16;

hipError_t launch_q1_gemm(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x, float *y,
                          int M, int N, int K, hipStream_t stream)
{
    if (M == 1) return launch_q1_gemv(wbits, scales, x, y, M, N, K, stream);
    if (M <= kSmallM) return launch_gemv_mfma(false, wbits, scales, x, y, M, N, K, stream);
    if (M <= skinny_max_m()) return launch_skinny(false, wbits, scales, x, y, M, N, K, stream);
    const int64_t tiles = (int64_t)((N + BN - 1) / BN) * ((M + BM - 1) / BM);
    if (tiles > INT_MAX || K % 128 != 0 || K <= 0) return hipErrorInvalidValue;
    void *args[] = {&wbits, &scales, &x, &y, &M, &N, &K};
    const bool s16 = K % 1024 == 0;
    const void *fn = s16 ? reinterpret_cast<const void *>(&q1_gemm_kernel<false, 16>)
                         : reinterpret_cast<const void *>(&q1_gemm_kernel<false, 2>);
    return launch_kernel(fn, s16 ? "q1_gemm_kernel<false, 16>" : "q1_gemm_kernel<false, 2>", dim3((unsigned)tiles),
                         dim3(256), args, 0, stream);
}

// Ternary prefill ("Ternary Bonsai 27B" article, cross-platform throughput: pp512) on the
// same tiles, 2-bit codes expanded to 0 / +-2s operands.
hipError_t launch_q2t_gemm(const uint32_t *wcodes, const uint16_t *scales, const uint16_t *x, float *y,
                           int M, int N, int K, hipStream_t stream)
{
    if (M <= kSmallM) return launch_gemv_mfma(true, wcodes, scales, x, y, M, N, K, stream);
    if (M <= skinny_max_m()) return launch_skinny(true, wcodes, scales, x, y, M, N, K, stream);
    const int64_t tiles = (int64_t)((N + BN - 1) / BN) * ((M + BM - 1) / BM);
    if (tiles > INT_MAX || K % 128 != 0 || K <= 0) return hipErrorInvalidValue;
    void *args[] = {&wcodes, &scales, &x, &y, &M, &N, &K};
    const bool s4 = (K / 128) % 2 == 0;
    const void *fn = s4 ? reinterpret_cast<const void *>(&q1_gemm_kernel<true, 4>)
                        : reinterpret_cast<const void *>(&q1_gemm_kernel<true, 2>);
    return launch_kernel(fn, s4 ? "q1_gemm_kernel<true, 4>" : "q1_gemm_kernel<true, 2>", dim3((unsigned)tiles),
                         dim3(256), args, 0, stream);
}

}  // namespace bonsai
