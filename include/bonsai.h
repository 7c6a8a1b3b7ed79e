/*
 * bonsai.h -- C ABI of the binary / ternary g128 weight-only matmul library (libbonsai.so).
 *
 * The method ("1-bit Bonsai 27B" model card, section "Weight representation: Binary g128"):
 * every weight is a single sign bit, 0 standing for -scale and 1 for +scale, and each run of
 * 128 consecutive weights along K shares one FP16 scale.  The model card's CUDA quick-start
 * and its highlights describe the matmul running straight on the packed signs, unpacking them
 * inside the kernel and applying the group scales there, with no dense FP16 weight copy.  The
 * ternary companion ("Ternary Bonsai 27B" article, ternary-format and limitations sections)
 * uses {-1, 0, +1} x the same FP16 group scale, stored today in 2 bits per weight.
 *
 * LAYOUT (normative; the pages fix no bit order, this is the library's reading)
 *   Binary  wbits  : uint32 [N][K/32], row-major.  The sign of W[n][k] is bit (k % 32) of
 *                    wbits[n][k / 32]; bit = 1 -> +s, bit = 0 -> -s.  In little-endian memory
 *                    byte b of a row holds k = 8b .. 8b+7, least significant bit first.
 *   Ternary wcodes : uint32 [N][K/16], row-major.  W[n][k] is the 2-bit field of
 *                    wcodes[n][k / 16] whose low bit is bit 2*(k % 16); field value
 *                    0 -> 0, 1 -> +1, 3 -> -1; the value 2 is reserved (never produced by the
 *                    packer, rejected by the unpacker; GPU results on it are unspecified).
 *   Scales         : IEEE binary16 bit patterns, uint16 [N][K/128], row-major;
 *                    W[n][k] uses scales[n][k / 128].  Any value is taken literally.
 *   x              : IEEE binary16, [M][K] row-major.      y : float32, [M][N] row-major.
 *   Every entry point computes  y[m][n] = sum_k W[n][k] * x[m][k]  (y = x W^T),
 *   accumulating in float32.  K must be a multiple of 128.
 *
 * CONVENTIONS
 *   Ownership : the caller allocates and owns every buffer; for the GPU entry points they are
 *               device memory.  The library allocates nothing, frees nothing and never
 *               synchronises in these calls; apart from the per-thread measurement hook
 *               and last-error name below, it keeps no state between calls.
 *   Streams   : GPU work is enqueued on `hip_stream` (a hipStream_t; NULL = default stream).
 *               BONSAI_OK means "validated and enqueued"; faults during execution surface at
 *               the caller's next synchronisation.
 *   Errors    : arguments are checked on the host before anything is enqueued; on any error
 *               nothing is enqueued and the status says why.  No C++ exception crosses the ABI.
 *   Aliasing  : y must not overlap the inputs.  Device pointers must be 16-byte aligned.
 *   Empty     : M == 0 or N == 0 is a no-op (BONSAI_OK).  K == 0 writes y = 0.
 *   Threads   : every entry point is reentrant and thread-safe.
 *   Results   : float32 sums in a kernel-defined order; they match the exact product within
 *               1e-3 * sum_k |W[n][k] x[m][k]| + 1e-6, are bitwise reproducible run to run for
 *               a given shape, and are exact whenever every partial sum is exactly
 *               representable in float32 (e.g. small integer x and power-of-two scales).
 */
#ifndef BONSAI_H
#define BONSAI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BONSAI_OK = 0,
    BONSAI_ERR_NULL = 1,    /* a required pointer is NULL                                   */
    BONSAI_ERR_SHAPE = 2,   /* M, N or K negative or out of range, or K % 128 != 0           */
    BONSAI_ERR_ALIGN = 3,   /* a device pointer is not 16-byte aligned                       */
    BONSAI_ERR_VALUE = 4,   /* pack input outside {-1,+1} (binary) or {-1,0,+1} (ternary);
                               an affine conversion whose result is not exact (see below)    */
    BONSAI_ERR_CODE = 5,    /* unpack met a reserved ternary code (2-bit field value 2; base-3
                               byte 243..255, or a nonzero weight in a base-3 row's padding)  */
    BONSAI_ERR_DEVICE = 6   /* the HIP runtime refused the launch                            */
} bonsai_status;

/* Largest K the GPU entry points accept (a multiple of 128). */
#define BONSAI_MAX_K 131072
/* Largest M of the GEMV entry points (M and N of every GPU entry point are at most 2^30). */
#define BONSAI_GEMV_MAX_M 8

/* Binary decode GEMV: y[M][N] = x[M][K] * W^T for 1 <= M <= 8 (M == 0: no-op).
 * The bandwidth-bound decode step (model card, cross-platform throughput: tg128 is the
 * memory-bound phase).  wbits, scales, x, y: device pointers laid out as above. */
bonsai_status bonsai_q1_gemv(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x,
                             float *y, int64_t M, int64_t N, int64_t K, void *hip_stream);

/* Binary prefill GEMM: y[M][N] = x[M][K] * W^T for any M >= 0 (tuned for M = 512, the pp512
 * prompt length of the model card's throughput table, its compute-bound phase). */
bonsai_status bonsai_q1_gemm(const uint32_t *wbits, const uint16_t *scales, const uint16_t *x,
                             float *y, int64_t M, int64_t N, int64_t K, void *hip_stream);

/* Ternary decode GEMV on 2-bit codes: y[M][N] = x[M][K] * W^T for 1 <= M <= 8 (M == 0: no-op).
 * The weights are {-1, 0, +1} times the FP16 group scale, stored in 2 bits each in the current
 * release ("Ternary Bonsai 27B" article, ternary format and limitations sections); decode
 * streams them once, as for the binary weights.  Otherwise as bonsai_q1_gemv. */
bonsai_status bonsai_q2t_gemv(const uint32_t *wcodes, const uint16_t *scales, const uint16_t *x,
                              float *y, int64_t M, int64_t N, int64_t K, void *hip_stream);

/* Ternary prefill GEMM on 2-bit codes: y[M][N] = x[M][K] * W^T for any M >= 0, tuned for M = 512
 * (the ternary article's cross-platform throughput table reports pp512 for this format).  The
 * codes are expanded to binary16 operands 0 and +-2s, so the scales must satisfy |s| < 32752
 * (2s finite in binary16); larger scales give non-finite results.  Otherwise as the other
 * entry points. */
bonsai_status bonsai_q2t_gemm(const uint32_t *wcodes, const uint16_t *scales, const uint16_t *x,
                              float *y, int64_t M, int64_t N, int64_t K, void *hip_stream);

/* Binary embedding gather: out[i][k] = W[ids[i]][k] (+-s, exact in binary16) for i < n_ids,
 * from a binary g128 table wbits [V][K/32], scales [V][K/128].  The model card's highlights
 * count the embeddings among the binary weights.  ids: int64 device array; out: binary16
 * [n_ids][K] device array.  An id outside [0, V) gives a row of zeros (nothing outside the
 * table is read).  n_ids == 0 or K == 0 is a no-op; otherwise as the other GPU entry points. */
bonsai_status bonsai_q1_embed(const uint32_t *wbits, const uint16_t *scales, const int64_t *ids,
                              uint16_t *out, int64_t n_ids, int64_t V, int64_t K, void *hip_stream);

/* Base-3 ternary weights ("t5"): the ternary weights at near their native density.  The ternary
 * article's limitations section puts the information content at log2(3) ~ 1.585 bits per weight
 * (about 1.71 with the scales) against the 2.125 of today's 2-bit storage, and gives no layout;
 * this one is the library's own.
 *   codes : uint8 [N][32 * ceil(K/160)], row-major: each row is a run of 32-byte superblocks of
 *           160 weights.  Byte c (0..31) of superblock b holds W[n][k] for k = 160 b + c + 32 i,
 *           i = 0..4, as the base-3 number sum_i d_i 3^i with d = W mod 3 (0 -> 0, 1 -> +1,
 *           2 -> -1).  Positions k >= K hold zero weights.  Bytes 243..255 are reserved: never
 *           produced by the packer, rejected by the unpacker, unspecified on the GPU.
 *   scales, x, y : as for the other layouts.  1.6 bits per weight (1.725 with the scales).
 * bonsai_t5_matmul: y[M][N] = x[M][K] * W^T for any M >= 0 (16 rows of x per pass of a small-M
 * matrix-core kernel; built for decode).  Otherwise as the other GPU entry points.
 * bonsai_t5_pack / bonsai_t5_unpack: host functions as the other packers, for any K >= 0;
 * trits are int8 [N][K] in {-1, 0, +1}.  unpack also rejects (BONSAI_ERR_CODE) a nonzero
 * weight in a row's padding past K. */
bonsai_status bonsai_t5_matmul(const uint8_t *codes, const uint16_t *scales, const uint16_t *x,
                               float *y, int64_t M, int64_t N, int64_t K, void *hip_stream);
bonsai_status bonsai_t5_pack(const int8_t *trits, int64_t N, int64_t K, uint8_t *codes);
bonsai_status bonsai_t5_unpack(const uint8_t *codes, int64_t N, int64_t K, int8_t *trits);
/* Direct host conversions between the 2-bit codes and the base-3 layout, a row at a time with no
 * int8 intermediate (the 2-bit storage of today's release to native density, and back).  K must
 * be a multiple of 16.  q2t_to_t5 rejects field value 2, t5_to_q2t reserved bytes and nonzero
 * padding (BONSAI_ERR_CODE); on an error the output is unspecified. */
bonsai_status bonsai_q2t_to_t5(const uint32_t *wcodes, int64_t N, int64_t K, uint8_t *codes);
bonsai_status bonsai_t5_to_q2t(const uint8_t *codes, int64_t N, int64_t K, uint32_t *wcodes);

/* Affine 1-bit matmul: y[M][N] = x[M][K] * W^T with W[n][k] = a * q + b, q the bit of W[n][k] in
 * the binary layout above and (a, b) = (mlx_scales, biases)[n][k / 128], binary16 [N][K/128]
 * each.  This is MLX's grouped low-bit format at one bit (model card, "MLX packaging": one
 * scale and one bias per group of 128; the binary weights travel in it as a = 2s, b = -s).
 * Any M >= 0 (16 rows of x per pass of the small-M matrix-core kernel; built for decode and
 * short M).  The sum is taken as a * sum(q x) + b * sum(x) per group in float32, so the
 * accuracy bound is 1e-3 * sum_k (|a q x| + |b x|) + 1e-6, which for a = 2s, b = -s is at most
 * three times the binary entry points' bound.  Otherwise as the other GPU entry points;
 * biases is a device pointer like mlx_scales. */
bonsai_status bonsai_q1a_matmul(const uint32_t *wbits, const uint16_t *mlx_scales, const uint16_t *biases,
                                const uint16_t *x, float *y, int64_t M, int64_t N, int64_t K, void *hip_stream);

/* Host conversions between the binary scales and MLX's (scale, bias) pairs for the same sign
 * words (model card, "MLX packaging"), bit-exact, on host arrays of n_groups binary16 values:
 * to_affine writes a = 2s and b = -s (BONSAI_ERR_VALUE if 2s is not finite: |s| > 32752,
 * inf or NaN); from_affine writes s = -b and returns BONSAI_ERR_VALUE unless a == 2s exactly
 * for every group (i.e. unless the affine weights are exactly +-s).  On an error the outputs
 * are unspecified.  n_groups == 0 is a no-op. */
bonsai_status bonsai_q1_to_affine(const uint16_t *scales, int64_t n_groups, uint16_t *mlx_scales,
                                  uint16_t *mlx_biases);
bonsai_status bonsai_q1_from_affine(const uint16_t *mlx_scales, const uint16_t *mlx_biases, int64_t n_groups,
                                    uint16_t *scales);

/* Host-side executable layout spec: pure functions on host memory, no device, no allocation.
 * They fix the bit order and code values given above: one sign bit per weight, bit 1 -> +s
 * (model card, "Weight representation: Binary g128"), and the ternary weights in two bits
 * ("Ternary Bonsai 27B" article, ternary format).
 * signs/trits are int8 [N][K] row-major; K must be a multiple of 32 (binary) or 16 (ternary).
 * pack rejects values outside the alphabet with BONSAI_ERR_VALUE (output then unspecified);
 * unpack of ternary rejects field value 2 with BONSAI_ERR_CODE. */
bonsai_status bonsai_q1_pack(const int8_t *signs, int64_t N, int64_t K, uint32_t *wbits);
bonsai_status bonsai_q1_unpack(const uint32_t *wbits, int64_t N, int64_t K, int8_t *signs);
bonsai_status bonsai_q2t_pack(const int8_t *trits, int64_t N, int64_t K, uint32_t *wcodes);
bonsai_status bonsai_q2t_unpack(const uint32_t *wcodes, int64_t N, int64_t K, int8_t *trits);

/* Name of the HIP runtime error behind the most recent BONSAI_ERR_DEVICE returned on the
 * calling thread ("none" if there was none).  Static string; never NULL.  A call that returns
 * BONSAI_ERR_DEVICE also clears the HIP runtime's last-error state (hipGetLastError), so the
 * caller's next HIP call does not report the refused launch again. */
const char *bonsai_last_device_error(void);

/* Measurement hook.  The next GPU entry point called on this thread launches its kernel with
 * hipExtLaunchKernel, recording start_event when the kernel starts executing and stop_event
 * when it completes, so hipEventElapsedTime(start, stop) is that kernel's device duration.
 * The events are hipEvent_t handles created and owned by the caller (either may be NULL);
 * the hook is consumed by that one call, whatever it returns: a call that fails its argument
 * checks or enqueues nothing disarms it too.  Do not arm it around stream capture. */
bonsai_status bonsai_time_next_launch(void *start_event, void *stop_event);

/* Launch plan (diagnostic).  Describes the kernel launch that a GPU entry point would enqueue
 * for these sizes, without reading or writing device memory and without launching anything:
 * "<kernel> grid=<x>,<y> block=<threads> lds=<bytes>" (NUL-terminated, truncated to len bytes),
 * followed by " timed" when the measurement hook below was armed and would time that launch (the
 * plan consumes the hook like a launch would); "none" when the call would enqueue nothing
 * (M == 0 or N == 0).  <kernel> is the launcher's name and template arguments.  op selects the entry point:
 * 0 bonsai_q1_gemv, 1 bonsai_q1_gemm, 2 bonsai_q2t_gemv, 3 bonsai_q2t_gemm, 4 bonsai_t5_matmul,
 * 5 bonsai_q1a_matmul, 6 bonsai_q1_embed (M = n_ids, N = V).  cus > 0 plans for a device with
 * that many compute units and makes no HIP call at all (so it runs on a host without a GPU; the
 * kernels' register counts are then taken as unknown, i.e. 8 waves per SIMD); cus <= 0 plans
 * for the calling thread's current device.  Returns what the entry point would return (its
 * argument checks run), or BONSAI_ERR_VALUE for an unknown op.  buf may be NULL. */
bonsai_status bonsai_plan(int op, int64_t M, int64_t N, int64_t K, int cus, char *buf, int64_t len);

/* Stream probe (diagnostic; the decode GEMVs are bound by memory bandwidth -- model card,
 * cross-platform throughput -- and this gives the rate a kernel that only moves bytes reaches
 * on the same device).  Streams `bytes` of device memory at buf once, one workgroup of eight
 * waves per compute unit:
 *   mode 0: reads by 16-byte vector loads (non-temporal);
 *   mode 1: reads by direct global->LDS copies of 16 bytes per lane, three 1 KB copies in
 *           flight per wave (the load path of the table GEMVs);
 *   mode 2: writes zeros over the buffer.
 * bytes: a positive multiple of 1024.  sink: device buffer of at least 64 KiB; modes 0 and 1
 * store one word per wave there (a digest of the bytes read, so that no load is dead); mode 2
 * leaves it alone.  buf and sink must be 16-byte aligned. */
bonsai_status bonsai_probe_stream(void *buf, int64_t bytes, int mode, uint32_t *sink, void *hip_stream);

/* Clock probe (diagnostic).  One wave stores the shader clock counter (s_memtime) and the
 * 100 MHz real-time counter (s_memrealtime), waits until spin_ns nanoseconds of real time have
 * passed (0 <= spin_ns <= 1e9), and stores both again: stamps = device uint64 [4] = {memtime0,
 * realtime0, memtime1, realtime1}.  The shader clock over that interval is
 * 100 MHz * (memtime1 - memtime0) / (realtime1 - realtime0).  Run beside a workload on another
 * stream, it reads the clock the workload runs at. */
bonsai_status bonsai_probe_clock(uint64_t *stamps, int64_t spin_ns, void *hip_stream);

/* Static, NUL-terminated description of a status value. */
const char *bonsai_status_str(bonsai_status s);

#ifdef __cplusplus
}
#endif

#endif /* BONSAI_H */
