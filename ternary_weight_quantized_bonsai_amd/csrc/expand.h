// expand.h -- packed weight codes to MFMA operands (binary16 pairs), shared by the prefill GEMM
// and the skinny GEMM.  An MFMA lane holds 8 consecutive k of its operand as 4 half pairs
// (k, k+1); the group scale is folded into the operand, exactly ("1-bit Bonsai 27B" model card,
// "Weight representation: Binary g128": bit 1 -> +s, bit 0 -> -s; ternary {-1, 0, +1} s).
#pragma once

#include "device.h"

namespace bonsai {

// 8 halves (+-s) of the k16 slice s of one 64-k step: w is the word holding it, q selects
// k 0..7 or 8..15 of the slice, cs = (-s, -s)
__device__ __forceinline__ half8_t expand8(uint32_t w, int s, int q, uint32_t cs)
{
    const uint32_t hi = 0xFFFF0000u;
    const uint32_t v = (s & 1) ? (((w >> 1) & hi) | (((w >> 16) | (w << 16)) & ~hi))
                               : (((w << 15) & hi) | (w & ~hi));
    const int p = 8 * q;
    u32x4 e;
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = ((v << (15 - (p + 2 * i))) & 0x80008000u) ^ cs;
    return __builtin_bit_cast(half8_t, e);
}

// Ternary: 8 halves of the k16 slice held by word w (16 codes, code j of k = j), k 8q .. 8q + 7,
// times the scale.  Merging the word's half q with the same half shifted by one code puts codes
// k and k + 1 16 bits apart, so one shift and one mask read a pair as binary16 (0 or +-2: code
// 01 sets the top exponent bit, 11 also the sign); cs2 = (s, s) scales the pair exactly (2s is
// finite for |s| < 32752), and the factor 2 comes off the fp32 sums.
__device__ __forceinline__ half8_t expand8_tern(uint32_t w, int q, uint32_t cs2)
{
    const uint32_t lo = w >> (16 * q), hi = w >> (16 * q + 2);
    const uint32_t v = (lo & 0xFFFFu) | (hi << 16);
    u32x4 e;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2_t t = as_half2((v << (14 - 4 * i)) & 0xC000C000u);
        e[i] = __builtin_bit_cast(uint32_t, t * as_half2(cs2));
    }
    return __builtin_bit_cast(half8_t, e);
}

}  // namespace bonsai
