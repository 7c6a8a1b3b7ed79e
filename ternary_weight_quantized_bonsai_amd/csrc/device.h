// device.h -- small device-side helpers shared by the gfx950 kernels of libbonsai.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bonsai {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // register-friendly 16-byte vector

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

// fp32 += a.lo*b.lo + a.hi*b.hi, both halves exact products (v_dot2_f32_f16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(as_half2(a), as_half2(b), c, false);
}

// Sum over each row of 16 lanes, left in every lane of the row (DPP row rotations, no LDS).
__device__ __forceinline__ float row16_sum(float t)
{
    // dpp_ctrl 0x121 + (r - 1) = row_ror:r
    t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, t), 0x128, 0xF, 0xF, false));
    t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, t), 0x124, 0xF, 0xF, false));
    t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, t), 0x122, 0xF, 0xF, false));
    t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, t), 0x121, 0xF, 0xF, false));
    return t;
}

// Two binary16 halves picked from two dwords: (lo(a), lo(b)) or (hi(a), hi(b)).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

}  // namespace bonsai
