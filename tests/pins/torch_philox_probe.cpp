// Independent reference for the Philox4x32-10 stream: PyTorch's host engine
// (ATen/core/PhiloxRNGEngine.h), configured with key = seed and a counter whose
// words 0-1 hold the block offset. For each (seed, index) pair read from stdin it
// prints the 32-bit word that the engine produces at position (index & 3) of
// block (index >> 2).
#include <ATen/core/PhiloxRNGEngine.h>

#include <cinttypes>
#include <cstdio>

int main() {
    unsigned long long seed, index;
    while (std::scanf("%llu %llu", &seed, &index) == 2) {
        at::philox_engine engine(seed, /*subsequence=*/0, /*offset=*/index >> 2);
        uint32_t w = 0;
        for (unsigned t = 0; t <= (index & 3); ++t) w = engine();
        std::printf("%" PRIu32 "\n", w);
    }
    return 0;
}
