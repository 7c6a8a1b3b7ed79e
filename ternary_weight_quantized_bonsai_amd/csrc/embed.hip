// embed.hip -- gather of binary g128 embedding rows, dequantized to binary16.
//
// The embeddings are binary weights too ("1-bit Bonsai 27B" model card, highlights: the
// binary language weights cover the embeddings as well as the projections and the LM head),
// stored like any other binary g128 matrix: sign words [V][K/32] and scales [V][K/128].  A
// lookup of token ids turns rows of it into activations: out[i][k] = +-s of row ids[i], which
// is exactly representable in binary16 (s with its sign bit set for a 0 bit).
//
// One thread per sign word: it reads the word and its group's scale and writes the 32 halves
// as four 16-byte stores; consecutive threads take consecutive words of a row, so loads and
// stores are both contiguous.  Ids outside [0, V) give rows of zeros (no read outside the table).
#include "device.h"
#include "launch.h"

namespace bonsai {
namespace {

__global__ __launch_bounds__(256) void q1_embed_kernel(const uint32_t *__restrict__ wbits,
                                                       const uint16_t *__restrict__ scales,
                                                       const int64_t *__restrict__ ids,
                                                       uint16_t *__restrict__ out, int64_t n_ids, int64_t V, int K)
{
    const int W = K >> 5;                           // sign words per row
    const int G = K >> 7;
    const int64_t total = n_ids * W;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
        const int64_t i = t / W;
        const int c = (int)(t - i * W);
        const int64_t id = ids[i];
        u32x4 *dst = reinterpret_cast<u32x4 *>(out + i * K + 32 * c);
        if (id < 0 || id >= V) {
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[q] = u32x4{0u, 0u, 0u, 0u};
            continue;
        }
        const uint32_t w = wbits[id * W + c];
        const uint32_t s = scales[id * G + (c >> 2)];
        const uint32_t s2 = s | (s << 16);
        // halves (k, k + 1) of pair p: bits 2p and 2p + 1; a 0 bit sets the half's sign
        const uint32_t nw = ~w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            u32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int p = 4 * q + e;
                const uint32_t neg = (((nw >> (2 * p)) & 1u) << 15) | (((nw >> (2 * p + 1)) & 1u) << 31);
                v[e] = s2 ^ neg;
            }
            dst[q] = v;
        }
    }
}

}  // namespace

hipError_t launch_q1_embed(const uint32_t *wbits, const uint16_t *scales, const int64_t *ids, uint16_t *out,
                           int64_t n_ids, int64_t V, int K, hipStream_t stream)
{
    const int64_t total = n_ids * (K / 32);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    void *args[] = {&wbits, &scales, &ids, &out, &n_ids, &V, &K};
    return launch_kernel(reinterpret_cast<const void *>(&q1_embed_kernel), "q1_embed_kernel", dim3((unsigned)blocks),
                         dim3(256), args, 0, stream);
}

}  // namespace bonsai
