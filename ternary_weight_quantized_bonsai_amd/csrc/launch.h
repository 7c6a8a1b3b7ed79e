// launch.h -- host-side launchers of the gfx950 kernels (arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bonsai {

hipError_t launch_q1_gemv(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x, float *y,
                          int M, int N, int K, hipStream_t stream);
hipError_t launch_q2t_gemv(const uint32_t *wcodes, const uint16_t *scales, const uint16_t *x, float *y,
                           int M, int N, int K, hipStream_t stream);
hipError_t launch_q1_gemm(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x, float *y,
                          int M, int N, int K, hipStream_t stream);
hipError_t launch_q2t_gemm(const uint32_t *wcodes, const uint16_t *scales, const uint16_t *x, float *y,
                           int M, int N, int K, hipStream_t stream);
// Small-M products on the matrix cores: 16 rows of x per column block, any M >= 1 (the GEMV
// entry points use it for ternary M = 1..8 and binary M = 2..8, the GEMMs for small M).
hipError_t launch_gemv_mfma(bool ternary, const uint32_t *codes, const uint16_t *scales, const uint16_t *x,
                            float *y, int M, int N, int K, hipStream_t stream);
// Binary weights, one row of x, many rows: byte lookup tables, a slice of K at a time (q1_lut8.hip);
// it takes N >= 8 and K up to what its LDS holds beside the tables (lut8_fits).
bool lut8_fits(int N, int K);
hipError_t launch_lut8(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x, float *y, int N, int K,
                       hipStream_t stream);
// The same for affine 1-bit weights (scale and bias per group), K up to lut8a_fits.
bool lut8a_fits(int N, int K);
hipError_t launch_lut8a(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases, const uint16_t *x,
                        float *y, int N, int K, hipStream_t stream);
// Affine 1-bit weights at M = 1 on the table kernels, where their tables fit (q1a_lut_fits).
bool q1a_lut_fits(int N, int K);
hipError_t launch_q1a_lut(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases, const uint16_t *x,
                          float *y, int N, int K, hipStream_t stream);
// Affine 1-bit weights (binary words with a binary16 scale and bias per group), any M >= 1.
hipError_t launch_q1a_matmul(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases,
                             const uint16_t *x, float *y, int M, int N, int K, hipStream_t stream);
// Binary (tern = false) or 2-bit ternary weights, 1 <= M <= skinny_max_m() rows of x: each weight
// expanded once for all rows of x (gemm_skinny.hip).
int skinny_max_m();
hipError_t launch_skinny(bool tern, const uint32_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                         int M, int N, int K, hipStream_t stream);
// Base-3 ternary weights (five trits per byte, 32-byte superblocks of 160 k), any M >= 1.
hipError_t launch_t5_matmul(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                            int M, int N, int K, hipStream_t stream);
hipError_t launch_fill_zero(float *y, int64_t count, hipStream_t stream);
hipError_t launch_q1_embed(const uint32_t *wbits, const uint16_t *scales, const int64_t *ids, uint16_t *out,
                           int64_t n_ids, int64_t V, int K, hipStream_t stream);
// Measurement probes (probe.hip): a stream over device memory, and a clock stamp.
hipError_t launch_probe_stream(void *buf, int64_t bytes, int mode, uint32_t *sink, hipStream_t stream);
hipError_t launch_probe_clock(uint64_t *stamps, int64_t spin_ns, hipStream_t stream);

// LDS bytes of one CU on gfx950.
constexpr int kLdsPerCu = 160 * 1024;

// Facts of the device the calling thread has current, looked up once per device (the routing
// reads them on every call).  During a launch plan (bonsai_plan) the compute-unit count is the
// planned one and no HIP call is made.
int device_cus();
// hipFuncSetAttribute(fn, MaxDynamicSharedMemorySize, bytes), once per (device, fn).
bool set_lds_limit(const void *fn, int bytes);
// VGPRs per lane of a kernel (hipFuncGetAttributes, once per (device, fn)); 0 if unknown.
int func_vgprs(const void *fn);
// Waves of a kernel that one CU holds by its registers: 512 VGPRs per SIMD lane, in granules of
// 8, at most 8 waves per SIMD, 4 SIMDs (8 per SIMD when the register count is unknown).
inline int reg_waves_per_cu(int vgprs)
{
    if (vgprs <= 0) return 32;
    const int per_simd = 512 / ((vgprs + 7) / 8 * 8);
    return 4 * (per_simd < 8 ? per_simd : 8);
}

// Every kernel launch of the library goes through here: a plain hipLaunchKernel, or, when the
// caller armed the timing hook for this call, hipExtLaunchKernel with the caller's events.
// During a launch plan nothing is launched: the launch is recorded instead.  `name` is a
// static description of the kernel (the launcher's signature with its template arguments).
hipError_t launch_kernel(const void *fn, const char *name, dim3 grid, dim3 block, void **args, size_t lds,
                         hipStream_t stream);

}  // namespace bonsai
