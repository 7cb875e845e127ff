// Drives the host-side planning of libqsgd (bucket counts, capacities, the
// ragged bucket table, the no-allocation capacity, argument checks that return
// before anything is enqueued) for a build under AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py). No kernel is launched.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "qsgd.h"

#define CHECK(c) do { if (!(c)) { std::printf("check failed line %d: %s\n", __LINE__, #c); return 1; } } while (0)

int main() {
    const uint32_t ss[] = {1, 3, 4, 16, 64, 1000, 1u << 24};
    const uint64_t ns[] = {0, 1, 15, 4096, 4097, 100000, 60192808ull, 1ull << 28};
    const uint32_t ds[] = {1, 7, 16, 512, 4081, 4082, 4096, 5000, 65536, 1u << 30};
    for (uint64_t n : ns)
        for (uint32_t s : ss)
            for (uint32_t d : ds) {
                const uint64_t nb = qsgd_num_buckets(n, d);
                CHECK(nb == (n + d - 1) / d);
                const uint64_t cap = qsgd_encode_capacity_words(n, s, d);
                CHECK(n == 0 ? cap == 1 : cap > nb / 2);
                const uint64_t na = qsgd_encode_noalloc_capacity_words(n, s, d);
                CHECK(na == 0 || na <= cap);
                CHECK(qsgd_encode_capacity_words_ex(n, nb, s, d, QSGD_CODE_GAMMA) >= (n ? 1u : 0u));
            }
    // ragged layouts
    std::vector<uint64_t> seg = {5, 0, 3, 8, 4081, 9000, 1};
    for (uint32_t d : {1u, 4u, 512u, 4081u}) {
        const uint64_t nb = qsgd_num_buckets_ragged(seg.data(), (uint32_t)seg.size(), d);
        std::vector<uint64_t> table(nb + 1);
        CHECK(qsgd_ragged_bucket_table(seg.data(), (uint32_t)seg.size(), d, table.data(), nb) == QSGD_OK);
        CHECK(qsgd_ragged_bucket_table(seg.data(), (uint32_t)seg.size(), d, table.data(), nb + 1) ==
              QSGD_ERR_INVALID_ARG);
        CHECK(table[nb] == 5 + 3 + 8 + 4081 + 9000 + 1);
        uint64_t n = table[nb];
        CHECK(qsgd_encode_capacity_words_ragged(n, nb, 8, d) > 0);
    }
    // argument checks that return before any launch
    std::vector<uint64_t> many(161, 100);
    CHECK(qsgd_encode_seglen(nullptr, many.data(), 161, 4, 64, 1, nullptr, nullptr, nullptr, nullptr) ==
          QSGD_ERR_UNSUPPORTED);
    CHECK(qsgd_encode(nullptr, 100, 0, 16, 1, nullptr, nullptr, nullptr, nullptr) == QSGD_ERR_INVALID_ARG);
    CHECK(qsgd_decode(nullptr, nullptr, 100, 4, 0, nullptr, nullptr) == QSGD_ERR_INVALID_ARG);
    CHECK(qsgd_quantize(nullptr, 100, (1u << 24) + 1, 16, 1, nullptr, nullptr, nullptr) == QSGD_ERR_INVALID_ARG);
    CHECK(qsgd_max_bucket() == 4081);
    for (int st = 0; st <= 5; ++st) CHECK(qsgd_status_string((qsgd_status)st) != nullptr);
    std::printf("host sanitizer driver ok\n");
    return 0;
}
