// Prints the persistent attention launch's XCD ranges and split plan, computed by
// the library's own host/device functions (dit_attn_common.hpp), so that a CPU
// test can compare them with the plan the GPU tests use to find split items.
// No GPU call is made.
#define DIT_ATTN_PERSISTENT
#include "dit_attn_common.hpp"

#include <cstdio>

int main() {
    using namespace dit::attn;
    for (int C = 1; C <= 40; ++C)
        for (int len = 0; len <= 400; ++len) {
            int T, s;
            split_plan(len, C, true, T, s);
            std::printf("P %d %d %d %d %d\n", C, len, T, s, xcd_units(len, T, s));
        }
    for (int total = 0; total <= 3000; total += 7)
        for (int x = 0; x < 8; ++x) {
            int start, len;
            xcd_slice(total, x, start, len);
            std::printf("X %d %d %d %d\n", total, x, start, len);
        }
    std::printf("K %d %d %d\n", kSplitC, kSplitMaxS, kSplitPieces);
    return 0;
}
