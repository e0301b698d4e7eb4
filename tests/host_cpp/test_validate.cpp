// Host-only unit test of the argument validation layer (no HIP, no GPU).
// Built with g++ under AddressSanitizer and UBSan by tests/test_host_validate.py.
#include <cstdio>
#include <cstring>

#include <cmath>

#include "fastdiv.hpp"
#include "validate.hpp"

using namespace attnblk;

static int failures = 0;
#define EXPECT(cond)                                                  \
    do {                                                              \
        if (!(cond)) {                                                \
            std::printf("FAIL line %d: %s\n", __LINE__, #cond);       \
            ++failures;                                               \
        }                                                             \
    } while (0)

// n / d through make_fast_div's multiplier and shift, as the layout kernel computes it.
static uint32_t fdiv(uint32_t n, const FastDiv &f) { return (uint32_t)(((uint64_t)n * f.m) >> (32 + f.s)); }

int main() {
    // fast division: exact for every numerator below 2^31 the layout kernel can produce
    {
        const uint32_t ds[] = {1u, 2u, 3u, 5u, 7u, 64u, 512u, 1000u, 4096u, 65535u, 65537u, (1u << 20) + 3u,
                               (1u << 30) + 1u, 0x7fffffffu};
        uint64_t x = 88172645463325252ull;  // xorshift64 numerators
        for (uint32_t d : ds) {
            const FastDiv f = make_fast_div(d);
            EXPECT(f.m < (1ull << 33));
            const uint32_t edge[] = {0u, 1u, d - 1u, d, d + 1u, 2u * d - 1u, 0x7fffffffu};
            for (uint32_t n : edge)
                if (n < 0x80000000u) EXPECT(fdiv(n, f) == n / d);
            for (int i = 0; i < 20000; ++i) {
                x ^= x << 13;
                x ^= x >> 7;
                x ^= x << 17;
                const uint32_t n = (uint32_t)(x & 0x7fffffffu);
                EXPECT(fdiv(n, f) == n / d);
            }
        }
    }
    const void *P = reinterpret_cast<const void *>(0x1000);
    const float *F = reinterpret_cast<const float *>(0x1000);
    // create
    EXPECT(validate_create(false, 4096, 32, kF16, P, P, P, P, 65536).status == kOk);
    EXPECT(validate_create(false, 256, 4, kF32, P, P, P, P, 256).status == kOk);
    EXPECT(validate_create(true, 4096, 32, kF16, P, P, P, P, 16).status == kInvalid);
    EXPECT(validate_create(false, 4096, 0, kF16, P, P, P, P, 16).status == kInvalid);
    EXPECT(validate_create(false, 4096, 64, kF16, P, P, P, P, 16).status == kUnsupported);
    EXPECT(validate_create(false, 256, 8, kF32, P, P, P, P, 16).status == kUnsupported);
    EXPECT(validate_create(false, 4096, 32, 5, P, P, P, P, 16).status == kInvalid);
    EXPECT(validate_create(false, 4096, 32, kF16, P, P, P, P, kMaxTokens + 1).status == kUnsupported);
    Check c = validate_create(false, 4096, 32, kF16, nullptr, P, P, P, 16);
    EXPECT(c.status == kInvalid && std::strstr(c.msg, "NULL"));
    // forward
    EXPECT(validate_forward(false, kF16, 4096, 1024, P, reinterpret_cast<const char *>(P) + (1 << 24), 1024, 1,
                            nullptr).status == kOk);
    EXPECT(validate_forward(false, kF16, 4096, 1024, P, P, 1024, 1, nullptr).status == kInvalid);  // overlap
    EXPECT(validate_forward(false, kF16, 4096, 1024, P, nullptr, 1025, 1, nullptr).status == kInvalid);
    EXPECT(validate_forward(false, kF16, 4096, 1024, P, nullptr, 16, 2, nullptr).status == kUnsupported);
    EXPECT(validate_forward(false, kF16, 4096, 1024, P, nullptr, 16, 0, nullptr).status == kInvalid);
    EXPECT(validate_forward(false, kF16, 4096, 1024, nullptr, nullptr, 0, 1, nullptr).status == kOk);
    TapsView t{};
    t.qkv_only = 1;
    EXPECT(validate_forward(false, kF16, 4096, 1024, P, nullptr, 16, 1, &t).status == kOk);
    t.k = reinterpret_cast<const char *>(P) + 2;
    EXPECT(validate_forward(false, kF16, 4096, 1024, P, nullptr, 16, 1, &t).status == kInvalid);
    // partial
    EXPECT(validate_partial(32, 128, kF16, P, 4096, 4096 * 128, P, 4096, 32768 * 128, P, 128 * 32768, 32768, F,
                            F).status == kOk);
    EXPECT(validate_partial(32, 128, kF16, P, 4096, 4096 * 128, P, 4096, 32768 * 128, P, 128 * 32768, 4000, F,
                            F).status == kInvalid);
    EXPECT(validate_partial(32, 128, kF16, P, 1, 128, P, 0, 0, nullptr, 0, 0, F, F).status == kOk);
    EXPECT(validate_partial(4, 64, kF32, P, 256, 256 * 64, P, 64, 256 * 64, P, 64 * 256, 256, F, F).status == kOk);
    EXPECT(validate_partial(4, 64, kF16, P, 256, 256 * 64, P, 64, 256 * 64, P, 64 * 256, 256, F, F).status ==
           kUnsupported);
    // partial with row-major V
    EXPECT(validate_partial_rows("p", 32, 128, kF16, P, 4096, 4096 * 128, P, P, 4096, 32768 * 128, F, F).status ==
           kOk);
    EXPECT(validate_partial_rows("p", 32, 128, kF16, P, 4096, 4096 * 128, P, P, 4096, 4000 * 128, F, F).status ==
           kInvalid);
    EXPECT(validate_partial_rows("p", 32, 128, kF16, P, 4096, 4096 * 128, P, P, 4096, 4096 * 128 + 4, F, F).status ==
           kInvalid);
    EXPECT(validate_partial_rows("p", 32, 128, kF16, P, 4096, 4096 * 128, P, nullptr, 4096, 4096 * 128, F, F)
               .status == kInvalid);
    EXPECT(validate_partial_rows("p", 32, 128, kF16, P, 1, 128, nullptr, nullptr, 0, 0, F, F).status == kOk);
    EXPECT(validate_partial_rows("p", 4, 64, kF32, P, 256, 256 * 64, P, P, 64, 64 * 64, F, F).status == kOk);
    EXPECT(validate_partial_rows("p", 4, 64, kF32, P, 256, 256 * 64, P, P, 64, 64 * 64 + 2, F, F).status ==
           kInvalid);
    EXPECT(validate_partial_rows("p", 4, 128, kF16, P, 256, 256 * 128, P, reinterpret_cast<const char *>(P) + 8, 64,
                                 64 * 128, F, F).status == kInvalid);
    EXPECT(validate_partial_rows("p", 4, 128, kF16, P, 256, 256 * 128, P, P, kMaxTokens + 1, 0, F, F).status ==
           kUnsupported);
    t.k = nullptr;
    t.v = reinterpret_cast<const char *>(P) + 4;
    EXPECT(validate_forward(false, kF16, 4096, 1024, P, nullptr, 16, 1, &t).status == kInvalid);
    // merge
    EXPECT(validate_shard(32, 8, 7).status == kOk);
    EXPECT(validate_shard(32, 1, 0).status == kOk);
    EXPECT(validate_shard(32, 3, 0).status == kInvalid);
    EXPECT(validate_shard(32, 8, -1).status == kInvalid);
    EXPECT(validate_shard(32, 0, 0).status == kInvalid);
    EXPECT(validate_heads_forward(4, 128, kF16, P, P, P, 32768, P, 512, F).status == kOk);
    EXPECT(validate_heads_forward(4, 128, kF16, P, P, P, 32768, P, 500, F).status == kInvalid);
    EXPECT(validate_heads_forward(4, 64, kF32, P, P, P, 256, P, 256, nullptr).status == kOk);
    EXPECT(validate_heads_forward(4, 128, kF16, P, P, P, kMaxTokens + 1, P, 512, F).status == kUnsupported);
    EXPECT(validate_ulysses_gather(8, 4, 128, kF16, 32768, P, P, P, P, P, P).status == kOk);
    EXPECT(validate_ulysses_gather(8, 4, 128, kF16, 32768 + 8, P, P, P, P, P, P).status == kInvalid);
    EXPECT(validate_ulysses_gather(8, 4, 128, kF16, 8 * 12, P, P, P, P, P, P).status == kInvalid);
    EXPECT(validate_ulysses_gather(8, 4, 128, kF16, 32768, P, nullptr, P, P, P, P).status == kInvalid);
    EXPECT(validate_ulysses_unpack(8, 32, 128, kF16, 4096, P, P).status == kOk);
    EXPECT(validate_ulysses_unpack(8, 36, 128, kF16, 4096, P, P).status == kInvalid);
    EXPECT(validate_ring_create(false, 32, 128, kF16, 8, 4096, 4096).status == kOk);
    EXPECT(validate_ring_create(true, 32, 128, kF16, 8, 4096, 4096).status == kInvalid);
    EXPECT(validate_ring_create(false, 32, 128, kF16, kMaxParts + 1, 4096, 4096).status == kUnsupported);
    EXPECT(validate_ring_create(false, 32, 128, kF16, 8, 4096, kMaxTokens + 1).status == kUnsupported);
    {
        const void *kb[3] = {P, P, nullptr};
        const int64_t lens_ok[3] = {64, 100, 0}, lens_big[3] = {64, 5000, 0}, lens_null[3] = {64, 100, 8};
        EXPECT(validate_ring_forward(false, 3, 4096, 4096, P, 300, kb, kb, lens_ok, P, F).status == kOk);
        EXPECT(validate_ring_forward(false, 3, 4096, 4096, P, 300, kb, kb, lens_big, P, F).status == kInvalid);
        EXPECT(validate_ring_forward(false, 3, 4096, 4096, P, 300, kb, kb, lens_null, P, F).status == kInvalid);
        EXPECT(validate_ring_forward(false, 3, 4096, 4096, P, 5000, kb, kb, lens_ok, P, F).status == kInvalid);
        EXPECT(validate_ring_forward(true, 3, 4096, 4096, P, 300, kb, kb, lens_ok, P, F).status == kInvalid);
        EXPECT(validate_ring_forward(false, 3, 4096, 4096, P, 0, nullptr, nullptr, nullptr, nullptr, nullptr).status ==
               kOk);
    }
    EXPECT(validate_set_prenorm(false, 1e-6f, false).status == kOk);
    EXPECT(validate_set_prenorm(false, 0.0f, false).status == kOk);
    EXPECT(validate_set_prenorm(true, 1e-6f, false).status == kInvalid);
    EXPECT(validate_set_prenorm(false, -1e-6f, false).status == kInvalid);
    EXPECT(validate_set_prenorm(false, NAN, false).status == kInvalid);
    EXPECT(validate_set_prenorm(false, INFINITY, false).status == kInvalid);
    EXPECT(validate_set_prenorm(false, 1e-6f, true).status == kInvalid);
    EXPECT(validate_partial(32, 128, kF16, P, 4096, 4096 * 128, P, 4096, 32768 * 128, P, 128 * (kMaxTokens + 8),
                            kMaxTokens + 8, F, F).status == kUnsupported);
    EXPECT(validate_merge(8, 32, 128, 4096, F, F, P, kF16, nullptr).status == kOk);
    EXPECT(validate_merge(0, 32, 128, 4096, F, F, P, kF16, nullptr).status == kInvalid);
    EXPECT(validate_merge(8, 32, 128, 4096, F, F, reinterpret_cast<const char *>(P) + 4, kF16, nullptr).status ==
           kInvalid);
    EXPECT(validate_merge(kMaxParts + 1, 32, 128, 16, F, F, P, kF16, nullptr).status == kUnsupported);
    // long messages are truncated, not overflowed
    c = fail(kInvalid, "%s", std::string(1000, 'x').c_str());
    EXPECT(std::strlen(c.msg) == sizeof(c.msg) - 1);
    std::printf("%s (%d failures)\n", failures ? "FAILED" : "OK", failures);
    return failures ? 1 : 0;
}
