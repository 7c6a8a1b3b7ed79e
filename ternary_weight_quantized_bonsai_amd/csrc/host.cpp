// host.cpp -- the host-only part of the C ABI of libbonsai: pack / unpack of the three weight
// layouts, the direct conversions between them and the affine scale pairs, and the status
// strings.  Plain C++ with no device code, so that it also builds with a host compiler alone
// (the sanitizer tests compile it with g++ -fsanitize=address,undefined).  Declarations and the
// normative layout are in include/bonsai.h.
#include <stdint.h>

#include "../../include/bonsai.h"

namespace {

// 2 s in binary16, exactly (an exponent step, or a shift of a subnormal's fraction, which
// carries into the exponent by itself); false when 2 s is not finite or s is inf / NaN
bool f16_twice(uint16_t s, uint16_t *out)
{
    const uint16_t sign = s & 0x8000u, mag = s & 0x7FFFu;
    const unsigned e = mag >> 10;
    if (e >= 30) return false;
    *out = (uint16_t)(sign | (e == 0 ? mag << 1 : mag + 0x400u));
    return true;
}

}  // namespace

extern "C" {

bonsai_status bonsai_t5_pack(const int8_t *trits, int64_t N, int64_t K, uint8_t *codes)
{
    if (N < 0 || K < 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!trits || !codes) return BONSAI_ERR_NULL;
    const int64_t sb = (K + 159) / 160;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < sb; ++b)
            for (int c = 0; c < 32; ++c) {
                unsigned v = 0, place = 1;
                for (int i = 0; i < 5; ++i, place *= 3) {
                    const int64_t k = 160 * b + c + 32 * i;
                    if (k >= K) continue;
                    const int8_t t = trits[n * K + k];
                    if (t < -1 || t > 1) return BONSAI_ERR_VALUE;
                    v += (unsigned)(t < 0 ? 2 : t) * place;
                }
                codes[n * 32 * sb + 32 * b + c] = (uint8_t)v;
            }
    return BONSAI_OK;
}

bonsai_status bonsai_t5_unpack(const uint8_t *codes, int64_t N, int64_t K, int8_t *trits)
{
    if (N < 0 || K < 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!trits || !codes) return BONSAI_ERR_NULL;
    const int64_t sb = (K + 159) / 160;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < sb; ++b)
            for (int c = 0; c < 32; ++c) {
                unsigned v = codes[n * 32 * sb + 32 * b + c];
                if (v >= 243) return BONSAI_ERR_CODE;
                for (int i = 0; i < 5; ++i, v /= 3) {
                    const int64_t k = 160 * b + c + 32 * i;
                    const int d = (int)(v % 3);
                    if (k >= K) {
                        if (d != 0) return BONSAI_ERR_CODE;      // padding must hold zero weights
                        continue;
                    }
                    trits[n * K + k] = (int8_t)(d == 2 ? -1 : d);
                }
            }
    return BONSAI_OK;
}

bonsai_status bonsai_q2t_to_t5(const uint32_t *wcodes, int64_t N, int64_t K, uint8_t *codes)
{
    if (N < 0 || K < 0 || K % 16 != 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!wcodes || !codes) return BONSAI_ERR_NULL;
    const int64_t sb = (K + 159) / 160;
    for (int64_t n = 0; n < N; ++n) {
        const uint32_t *row = wcodes + n * (K / 16);
        for (int64_t b = 0; b < sb; ++b)
            for (int c = 0; c < 32; ++c) {
                unsigned v = 0, place = 1;
                for (int i = 0; i < 5; ++i, place *= 3) {
                    const int64_t k = 160 * b + c + 32 * i;
                    if (k >= K) continue;
                    const unsigned f = (row[k / 16] >> (2 * (k % 16))) & 3u;
                    if (f == 2) return BONSAI_ERR_CODE;
                    v += (f == 0 ? 0u : f == 1 ? 1u : 2u) * place;   // digit = w mod 3
                }
                codes[n * 32 * sb + 32 * b + c] = (uint8_t)v;
            }
    }
    return BONSAI_OK;
}

bonsai_status bonsai_t5_to_q2t(const uint8_t *codes, int64_t N, int64_t K, uint32_t *wcodes)
{
    if (N < 0 || K < 0 || K % 16 != 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!wcodes || !codes) return BONSAI_ERR_NULL;
    const int64_t sb = (K + 159) / 160;
    for (int64_t n = 0; n < N; ++n) {
        uint32_t *row = wcodes + n * (K / 16);
        for (int64_t w = 0; w < K / 16; ++w) row[w] = 0;
        for (int64_t b = 0; b < sb; ++b)
            for (int c = 0; c < 32; ++c) {
                unsigned v = codes[n * 32 * sb + 32 * b + c];
                if (v >= 243) return BONSAI_ERR_CODE;
                for (int i = 0; i < 5; ++i, v /= 3) {
                    const int64_t k = 160 * b + c + 32 * i;
                    const unsigned d = v % 3;
                    if (k >= K) {
                        if (d != 0) return BONSAI_ERR_CODE;      // padding must hold zero weights
                        continue;
                    }
                    row[k / 16] |= (d == 0 ? 0u : d == 1 ? 1u : 3u) << (2 * (k % 16));
                }
            }
    }
    return BONSAI_OK;
}

bonsai_status bonsai_q1_to_affine(const uint16_t *scales, int64_t n_groups, uint16_t *mlx_scales,
                                  uint16_t *mlx_biases)
{
    if (n_groups < 0) return BONSAI_ERR_SHAPE;
    if (n_groups == 0) return BONSAI_OK;
    if (!scales || !mlx_scales || !mlx_biases) return BONSAI_ERR_NULL;
    for (int64_t g = 0; g < n_groups; ++g) {
        if (!f16_twice(scales[g], &mlx_scales[g])) return BONSAI_ERR_VALUE;
        mlx_biases[g] = (uint16_t)(scales[g] ^ 0x8000u);
    }
    return BONSAI_OK;
}

bonsai_status bonsai_q1_from_affine(const uint16_t *mlx_scales, const uint16_t *mlx_biases, int64_t n_groups,
                                    uint16_t *scales)
{
    if (n_groups < 0) return BONSAI_ERR_SHAPE;
    if (n_groups == 0) return BONSAI_OK;
    if (!scales || !mlx_scales || !mlx_biases) return BONSAI_ERR_NULL;
    for (int64_t g = 0; g < n_groups; ++g) {
        const uint16_t s = (uint16_t)(mlx_biases[g] ^ 0x8000u);
        uint16_t twice;
        if (!f16_twice(s, &twice) || twice != mlx_scales[g]) return BONSAI_ERR_VALUE;
        scales[g] = s;
    }
    return BONSAI_OK;
}

bonsai_status bonsai_q1_pack(const int8_t *signs, int64_t N, int64_t K, uint32_t *wbits)
{
    if (N < 0 || K < 0 || K % 32 != 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!signs || !wbits) return BONSAI_ERR_NULL;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t w = 0; w < K / 32; ++w) {
            uint32_t word = 0;
            for (int j = 0; j < 32; ++j) {
                const int8_t v = signs[n * K + 32 * w + j];
                if (v != 1 && v != -1) return BONSAI_ERR_VALUE;
                word |= (uint32_t)(v > 0) << j;
            }
            wbits[n * (K / 32) + w] = word;
        }
    return BONSAI_OK;
}

bonsai_status bonsai_q1_unpack(const uint32_t *wbits, int64_t N, int64_t K, int8_t *signs)
{
    if (N < 0 || K < 0 || K % 32 != 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!signs || !wbits) return BONSAI_ERR_NULL;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            signs[n * K + k] = ((wbits[n * (K / 32) + k / 32] >> (k % 32)) & 1u) ? 1 : -1;
    return BONSAI_OK;
}

bonsai_status bonsai_q2t_pack(const int8_t *trits, int64_t N, int64_t K, uint32_t *wcodes)
{
    if (N < 0 || K < 0 || K % 16 != 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!trits || !wcodes) return BONSAI_ERR_NULL;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t w = 0; w < K / 16; ++w) {
            uint32_t word = 0;
            for (int j = 0; j < 16; ++j) {
                const int8_t v = trits[n * K + 16 * w + j];
                uint32_t code;
                if (v == 0) code = 0u;
                else if (v == 1) code = 1u;
                else if (v == -1) code = 3u;
                else return BONSAI_ERR_VALUE;
                word |= code << (2 * j);
            }
            wcodes[n * (K / 16) + w] = word;
        }
    return BONSAI_OK;
}

bonsai_status bonsai_q2t_unpack(const uint32_t *wcodes, int64_t N, int64_t K, int8_t *trits)
{
    if (N < 0 || K < 0 || K % 16 != 0) return BONSAI_ERR_SHAPE;
    if (N == 0 || K == 0) return BONSAI_OK;
    if (!trits || !wcodes) return BONSAI_ERR_NULL;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const uint32_t code = (wcodes[n * (K / 16) + k / 16] >> (2 * (k % 16))) & 3u;
            if (code == 2u) return BONSAI_ERR_CODE;
            trits[n * K + k] = code == 0u ? 0 : (code == 1u ? 1 : -1);
        }
    return BONSAI_OK;
}

const char *bonsai_status_str(bonsai_status s)
{
    switch (s) {
    case BONSAI_OK: return "ok";
    case BONSAI_ERR_NULL: return "a required pointer is NULL";
    case BONSAI_ERR_SHAPE: return "M, N or K out of range, or K not a multiple of 128";
    case BONSAI_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case BONSAI_ERR_VALUE: return "input outside the weight alphabet, or not an exact binary-weight scale/bias pair";
    case BONSAI_ERR_CODE: return "reserved ternary code (2-bit field 0b10, base-3 byte above 242 or nonzero padding)";
    case BONSAI_ERR_DEVICE: return "HIP launch failed";
    }
    return "unknown status";
}

}  // extern "C"
