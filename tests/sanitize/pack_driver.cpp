// Drives the host entry points of libbq's packer (bq_pack.cpp: bq_packed_bytes,
// bq_pack, bq_unpack, bq_last_error, bq_abi_version) under AddressSanitizer
// and UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py with g++,
// on the CPU, from bq_pack.cpp alone: no GPU code).  Exits 0 and prints "ok"
// when every check holds and the sanitizers report nothing.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../../include/bq.h"

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint8_t rnd8()
{
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    return (uint8_t)(st >> 56);
}

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            return 1;                                                     \
        }                                                                 \
    } while (0)

int main()
{
    CHECK(bq_abi_version() == BQ_ABI_VERSION);
    const int64_t shapes[6][2] = {{1, 1}, {63, 3}, {64, 8}, {65, 9}, {130, 17}, {200, 40}};
    for (int fmt = 1; fmt <= 2; ++fmt) {
        const int64_t qk = fmt == 1 ? 128 : 64;
        for (auto &s : shapes) {
            const int64_t rows = s[0], nb = s[1], cols = nb * qk;
            size_t bb = 0, sb = 0;
            CHECK(bq_packed_bytes(fmt, rows, cols, &bb, &sb) == BQ_OK);
            std::vector<uint8_t> canon((size_t)(rows * nb * 18)), back(canon.size());
            for (auto &c : canon)
                c = rnd8();
            std::vector<uint8_t> bits(bb);
            std::vector<uint16_t> scales(sb / 2);
            CHECK(bq_pack(fmt, canon.data(), rows, cols, bits.data(), scales.data()) == BQ_OK);
            CHECK(bq_unpack(fmt, bits.data(), scales.data(), rows, cols, back.data()) == BQ_OK);
            CHECK(canon == back);
        }
    }
    size_t bb = 0, sb = 0;
    CHECK(bq_packed_bytes(3, 4, 128, &bb, &sb) == BQ_EARG && strlen(bq_last_error()) > 0);
    CHECK(bq_packed_bytes(1, 4, 100, &bb, &sb) == BQ_EARG);
    CHECK(bq_packed_bytes(1, 4, 128, nullptr, &sb) == BQ_EARG);
    CHECK(bq_packed_bytes(1, int64_t(1) << 31, 128, &bb, &sb) == BQ_EARG);
    CHECK(bq_packed_bytes(1, 64, int64_t(2097152) * 128, &bb, &sb) == BQ_EARG);
    uint8_t one[18] = {0};
    uint16_t sc[8];
    uint8_t bits[1024];
    CHECK(bq_pack(1, nullptr, 1, 128, bits, sc) == BQ_EARG);
    CHECK(bq_pack(1, one, 1, 128, nullptr, sc) == BQ_EARG);
    CHECK(bq_unpack(2, bits, nullptr, 1, 64, one) == BQ_EARG);
    printf("ok\n");
    return 0;
}
