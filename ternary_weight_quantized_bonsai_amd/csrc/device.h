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

// s_waitcnt as asm statements with a memory clobber.  The builtin is modelled as touching no
// memory, so the compiler may move a load above it; no memory access moves across these.  Any
// LDS read of data that a direct global->LDS copy brings in is ordered after one of them.
template <int N>
__device__ __forceinline__ void vm_wait()
{
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void lgkm_wait0() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

// Two binary16 halves picked from two dwords: (lo(a), lo(b)) or (hi(a), hi(b)).
// One v_perm_b32 each: selector bytes 0..3 pick bytes of the second source (a), 4..7 of the first (b).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

}  // namespace bonsai
