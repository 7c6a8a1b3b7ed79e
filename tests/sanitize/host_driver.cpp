// host_driver.cpp -- drives every host-only entry point of libbonsai (pack / unpack of the three
// weight layouts, the conversions between them and the affine scale pairs, the status strings)
// through round trips, cross-layout consistency and every documented error status.  Built with
// -fsanitize=address,undefined against host.cpp alone by tests/test_sanitizers.py; every buffer
// is a std::vector of exactly the documented size, so an access past it is reported.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "bonsai.h"

static int failures = 0;

#define CHECK(cond)                                                                  \
    do {                                                                             \
        if (!(cond)) {                                                               \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                              \
        }                                                                            \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32()
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 16);
}

static std::vector<int8_t> random_signs(int64_t n)
{
    std::vector<int8_t> v((size_t)n);
    for (auto &e : v) e = (next_u32() & 1) ? 1 : -1;
    return v;
}

static std::vector<int8_t> random_trits(int64_t n)
{
    std::vector<int8_t> v((size_t)n);
    for (auto &e : v) e = (int8_t)((int)(next_u32() % 3) - 1);
    return v;
}

static int64_t t5_row_bytes(int64_t K) { return 32 * ((K + 159) / 160); }

static void binary_layout()
{
    const int64_t shapes[][2] = {{1, 32}, {3, 96}, {2, 5120}, {7, 160}};
    for (const auto &sh : shapes) {
        const int64_t N = sh[0], K = sh[1];
        const std::vector<int8_t> signs = random_signs(N * K);
        std::vector<uint32_t> words((size_t)(N * K / 32));
        std::vector<int8_t> back((size_t)(N * K));
        CHECK(bonsai_q1_pack(signs.data(), N, K, words.data()) == BONSAI_OK);
        CHECK(bonsai_q1_unpack(words.data(), N, K, back.data()) == BONSAI_OK);
        CHECK(back == signs);
    }
    std::vector<int8_t> bad = random_signs(64);
    std::vector<uint32_t> w2(2);
    bad[37] = 0;
    CHECK(bonsai_q1_pack(bad.data(), 1, 64, w2.data()) == BONSAI_ERR_VALUE);
    CHECK(bonsai_q1_pack(bad.data(), 1, 48, w2.data()) == BONSAI_ERR_SHAPE);
    CHECK(bonsai_q1_pack(bad.data(), -1, 64, w2.data()) == BONSAI_ERR_SHAPE);
    CHECK(bonsai_q1_pack(nullptr, 1, 64, w2.data()) == BONSAI_ERR_NULL);
    CHECK(bonsai_q1_unpack(w2.data(), 1, 64, nullptr) == BONSAI_ERR_NULL);
    CHECK(bonsai_q1_pack(nullptr, 0, 64, nullptr) == BONSAI_OK);   // empty: nothing is read
}

static void ternary_layout()
{
    const int64_t shapes[][2] = {{1, 16}, {3, 48}, {2, 5120}, {5, 640}};
    for (const auto &sh : shapes) {
        const int64_t N = sh[0], K = sh[1];
        const std::vector<int8_t> trits = random_trits(N * K);
        std::vector<uint32_t> words((size_t)(N * K / 16));
        std::vector<int8_t> back((size_t)(N * K));
        CHECK(bonsai_q2t_pack(trits.data(), N, K, words.data()) == BONSAI_OK);
        CHECK(bonsai_q2t_unpack(words.data(), N, K, back.data()) == BONSAI_OK);
        CHECK(back == trits);
    }
    std::vector<int8_t> bad = random_trits(32);
    std::vector<uint32_t> w2(2);
    bad[5] = 2;
    CHECK(bonsai_q2t_pack(bad.data(), 1, 32, w2.data()) == BONSAI_ERR_VALUE);
    CHECK(bonsai_q2t_pack(bad.data(), 1, 24, w2.data()) == BONSAI_ERR_SHAPE);
    std::vector<uint32_t> reserved = {0x00000008u, 0u};   // field 1 holds 0b10
    std::vector<int8_t> out(32);
    CHECK(bonsai_q2t_unpack(reserved.data(), 1, 32, out.data()) == BONSAI_ERR_CODE);
}

static void base3_layout()
{
    // K not a multiple of 160 leaves padding in the last superblock
    const int64_t shapes[][2] = {{1, 160}, {2, 100}, {3, 170}, {2, 1152}, {1, 5120}, {4, 16}};
    for (const auto &sh : shapes) {
        const int64_t N = sh[0], K = sh[1];
        const std::vector<int8_t> trits = random_trits(N * K);
        std::vector<uint8_t> codes((size_t)(N * t5_row_bytes(K)));
        std::vector<int8_t> back((size_t)(N * K));
        CHECK(bonsai_t5_pack(trits.data(), N, K, codes.data()) == BONSAI_OK);
        for (uint8_t c : codes) CHECK(c < 243);
        CHECK(bonsai_t5_unpack(codes.data(), N, K, back.data()) == BONSAI_OK);
        CHECK(back == trits);
        if (K % 16 == 0) {
            // the direct conversions agree with going through the trits
            std::vector<uint32_t> words((size_t)(N * K / 16)), words2((size_t)(N * K / 16));
            std::vector<uint8_t> codes2((size_t)(N * t5_row_bytes(K)));
            CHECK(bonsai_q2t_pack(trits.data(), N, K, words.data()) == BONSAI_OK);
            CHECK(bonsai_q2t_to_t5(words.data(), N, K, codes2.data()) == BONSAI_OK);
            CHECK(codes2 == codes);
            CHECK(bonsai_t5_to_q2t(codes.data(), N, K, words2.data()) == BONSAI_OK);
            CHECK(words2 == words);
        }
    }
    std::vector<uint8_t> codes((size_t)t5_row_bytes(100));
    std::vector<int8_t> trits(100);
    codes[3] = 243;
    CHECK(bonsai_t5_unpack(codes.data(), 1, 100, trits.data()) == BONSAI_ERR_CODE);
    codes[3] = 0;
    codes[10] = 81;          // digit 4 of byte 10 is weight 138, past K = 100: padding must be zero
    CHECK(bonsai_t5_unpack(codes.data(), 1, 100, trits.data()) == BONSAI_ERR_CODE);
    std::vector<uint32_t> words(7);
    CHECK(bonsai_t5_to_q2t(codes.data(), 1, 112, words.data()) == BONSAI_ERR_CODE);
    CHECK(bonsai_q2t_to_t5(words.data(), 1, 100, codes.data()) == BONSAI_ERR_SHAPE);
    std::vector<int8_t> bad = random_trits(160);
    std::vector<uint8_t> c32(32);
    bad[159] = -2;
    CHECK(bonsai_t5_pack(bad.data(), 1, 160, c32.data()) == BONSAI_ERR_VALUE);
}

static void affine_pairs()
{
    // every finite binary16 scale whose double is finite round-trips; inf, NaN and the largest
    // exponent (2 s overflows) are rejected
    std::vector<uint16_t> s(65536), a(65536), b(65536);
    for (int i = 0; i < 65536; ++i) s[(size_t)i] = (uint16_t)i;
    int finite_twice = 0;
    for (int i = 0; i < 65536; ++i) {
        const uint16_t one = s[(size_t)i];
        uint16_t aa, bb, ss;
        const bonsai_status st = bonsai_q1_to_affine(&one, 1, &aa, &bb);
        const unsigned e = (one >> 10) & 0x1F;
        CHECK((st == BONSAI_OK) == (e < 30));
        if (st != BONSAI_OK) continue;
        ++finite_twice;
        CHECK(bb == (uint16_t)(one ^ 0x8000u));
        CHECK(bonsai_q1_from_affine(&aa, &bb, 1, &ss) == BONSAI_OK);
        CHECK(ss == one);
    }
    CHECK(finite_twice == 2 * 30 * 1024);
    // a pair that is not (2 s, -s) is refused
    const uint16_t a1 = 0x4000u, b1 = 0xBC00u;      // (2, -1): fine
    const uint16_t a2 = 0x4200u;                    // (3, -1): not a binary-weight pair
    uint16_t out;
    CHECK(bonsai_q1_from_affine(&a1, &b1, 1, &out) == BONSAI_OK && out == 0x3C00u);
    CHECK(bonsai_q1_from_affine(&a2, &b1, 1, &out) == BONSAI_ERR_VALUE);
    CHECK(bonsai_q1_to_affine(nullptr, 1, a.data(), b.data()) == BONSAI_ERR_NULL);
    CHECK(bonsai_q1_to_affine(s.data(), -1, a.data(), b.data()) == BONSAI_ERR_SHAPE);
    CHECK(bonsai_q1_from_affine(a.data(), b.data(), 0, nullptr) == BONSAI_OK);
}

static void status_strings()
{
    const bonsai_status all[] = {BONSAI_OK, BONSAI_ERR_NULL, BONSAI_ERR_SHAPE, BONSAI_ERR_ALIGN,
                                 BONSAI_ERR_VALUE, BONSAI_ERR_CODE, BONSAI_ERR_DEVICE};
    for (bonsai_status st : all) {
        const char *msg = bonsai_status_str(st);
        CHECK(msg != nullptr && msg[0] != '\0');
    }
    CHECK(bonsai_status_str((bonsai_status)7) != nullptr);   // in the enum's range, not a status
}

int main()
{
    binary_layout();
    ternary_layout();
    base3_layout();
    affine_pairs();
    status_strings();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("host driver: all checks passed\n");
    return 0;
}
