// Every C entry point on arguments its validation rejects (so no HIP call is
// made), plus the host-only helpers, for a host build of the library under
// AddressSanitizer and UndefinedBehaviorSanitizer (tests only).  Exit status 0
// when every call returned the expected status.
#include <cstdint>
#include <cstdio>

#include "fp4q.h"

static int fails = 0;
static void expect(int got, int want, const char *what) {
    if (got != want) {
        std::printf("FAIL %s: status %d, expected %d\n", what, got, want);
        ++fails;
    }
}

int main() {
    // fake, well-aligned device addresses far apart: never dereferenced
    auto A = [](uint64_t gib) { return reinterpret_cast<void *>((uint64_t{1} << 40) + (gib << 30)); };
    auto u8 = [&](uint64_t g) { return static_cast<uint8_t *>(A(g)); };
    auto f32 = [&](uint64_t g) { return static_cast<float *>(A(g)); };
    auto u16 = [&](uint64_t g) { return static_cast<uint16_t *>(A(g)); };
    size_t c, m, b;
    expect(fp4q_payload_bytes(32768, 4096, &c, &m, &b), FP4Q_OK, "payload_bytes");
    expect(c == 67108864 && m == 8388608 && b == 2097152 ? 0 : 1, 0, "payload sizes");
    expect(fp4q_payload_bytes(1, 300, &c, &m, &b), FP4Q_ERR_SHAPE, "payload_bytes shape");
    expect(fp4q_payload_bytes(INT64_MAX, 256, nullptr, nullptr, nullptr), FP4Q_ERR_SHAPE, "overflow");
    for (int s = -1; s < 9; ++s)
        if (!fp4q_status_str(s)) ++fails;

    expect(fp4q_compress(u16(0), 1, 100, u8(1), u8(2), f32(3), nullptr), FP4Q_ERR_SHAPE, "compress shape");
    expect(fp4q_compress(nullptr, 1, 256, u8(1), u8(2), f32(3), nullptr), FP4Q_ERR_NULL, "compress null");
    expect(fp4q_compress_ex(u16(0), 1, 256, u8(1), u8(2), f32(3), 8u, nullptr), FP4Q_ERR_ARG, "compress flags");
    expect(fp4q_compress(u16(0) + 1, 1, 256, u8(1), u8(2), f32(3), nullptr), FP4Q_ERR_ALIGN, "compress align");
    expect(fp4q_compress(u16(0), 4, 256, u8(0) + 64, u8(2), f32(3), nullptr), FP4Q_ERR_ARG, "compress overlap");
    expect(fp4q_compress(u16(0), 0, 256, nullptr, nullptr, nullptr, nullptr), FP4Q_OK, "compress empty");

    expect(fp4q_decompress(u8(0), u8(1), f32(2), -1, 256, f32(3), nullptr), FP4Q_ERR_SHAPE, "decompress shape");
    expect(fp4q_decompress_ex(u8(0), u8(1), f32(2), 1, 256, A(3), 5, 0u, nullptr), FP4Q_ERR_ARG, "out dtype");
    expect(fp4q_decompress(u8(0), u8(1) + 4, f32(2), 1, 256, f32(3), nullptr), FP4Q_ERR_ALIGN, "micro align");
    expect(fp4q_decompress(u8(0), u8(1), f32(2), 4, 256, f32(0) + 4, nullptr), FP4Q_ERR_ARG, "decompress overlap");

    const uint8_t *cs[17], *ms[17];
    const float *bs[17];
    for (int p = 0; p < 17; ++p) {
        cs[p] = u8(10 + 3 * p);
        ms[p] = u8(11 + 3 * p);
        bs[p] = f32(12 + 3 * p);
    }
    expect(fp4q_decompress_accumulate(0, cs, ms, bs, 1, 256, A(80), 0, nullptr), FP4Q_ERR_K, "acc k=0");
    expect(fp4q_decompress_accumulate(17, cs, ms, bs, 1, 256, A(80), 0, nullptr), FP4Q_ERR_K, "acc k=17");
    expect(fp4q_decompress_accumulate(2, cs, ms, bs, 1, 256, nullptr, 0, nullptr), FP4Q_ERR_NULL, "acc null");
    expect(fp4q_decompress_accumulate_ex(2, cs, ms, bs, 1, 256, A(80), 0, 2u, nullptr), FP4Q_ERR_ARG, "acc flags");
    expect(fp4q_decompress_accumulate(16, cs, ms, bs, 4, 256, (void *)(cs[15] + 16), 0, nullptr),
           FP4Q_ERR_ARG, "acc overlap with peer 15");

    expect(fp4q_reduce_requantize(0, cs, ms, bs, 1, 256, u8(80), u8(81), f32(82), nullptr), FP4Q_ERR_K, "req k=0");
    expect(fp4q_reduce_requantize_ex(0, nullptr, nullptr, nullptr, u16(90), 1, 256, u8(80), u8(81) + 4, f32(82),
                                     0u, nullptr), FP4Q_ERR_ALIGN, "req micro align");
    expect(fp4q_reduce_requantize_ex(16, cs, ms, bs, u16(90), 4, 256, u8(80), u8(81), (float *)(u8(90) + 64),
                                     0u, nullptr), FP4Q_ERR_ARG, "req local overlap");
    expect(fp4q_reduce_requantize_ex(16, cs, ms, bs, nullptr, 4, 256, u8(80), u8(81), f32(82), 4u, nullptr),
           FP4Q_ERR_ARG, "req flags");

    expect(fp4q_compress_mx(u16(0), 1, 256, u8(1), u8(2) + 4, 0u, nullptr), FP4Q_ERR_ALIGN, "mx align");
    expect(fp4q_decompress_mx(u8(0), u8(1), 1, 512 + 1, f32(2), 0, 0u, nullptr), FP4Q_ERR_SHAPE, "mx shape");
    if (fails == 0) std::printf("abi driver ok\n");
    return fails ? 1 : 0;
}
