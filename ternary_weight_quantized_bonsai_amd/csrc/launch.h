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
// Affine 1-bit weights at M = 1 on the table kernels, where their tables fit (q1a_lut_fits).
bool q1a_lut_fits(int N, int K);
hipError_t launch_q1a_lut(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases, const uint16_t *x,
                          float *y, int N, int K, hipStream_t stream);
// Affine 1-bit weights (binary words with a binary16 scale and bias per group), any M >= 1.
hipError_t launch_q1a_matmul(const uint32_t *wbits, const uint16_t *scales, const uint16_t *biases,
                             const uint16_t *x, float *y, int M, int N, int K, hipStream_t stream);
// Base-3 ternary weights (five trits per byte, 32-byte superblocks of 160 k), any M >= 1.
hipError_t launch_t5_matmul(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                            int M, int N, int K, hipStream_t stream);
hipError_t launch_fill_zero(float *y, int64_t count, hipStream_t stream);
hipError_t launch_q1_embed(const uint32_t *wbits, const uint16_t *scales, const int64_t *ids, uint16_t *out,
                           int64_t n_ids, int64_t V, int K, hipStream_t stream);

// Every kernel launch of the library goes through here: a plain hipLaunchKernel, or, when the
// caller armed the timing hook on this thread, hipExtLaunchKernel with the caller's events.
hipError_t launch_kernel(const void *fn, dim3 grid, dim3 block, void **args, size_t lds, hipStream_t stream);

}  // namespace bonsai
