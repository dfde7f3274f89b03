// Prints, for a fixed set of per-head amax pairs, the score-scale exponent and
// q's float32 multiplier exactly as the FP8 kernels decide them (the library's
// own header, compiled for the host; no GPU call). Lines: "S aq_bits ak_bits n g_bits".
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "dit_fp8.hpp"

static uint32_t bits(float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    return u;
}

int main() {
    // a deterministic spread of magnitudes: 1e-30 .. 1e30, plus zeros and the
    // neighbours of powers of two
    uint64_t st = 0x9E3779B97F4A7C15ull;
    auto next = [&]() {
        st ^= st << 13; st ^= st >> 7; st ^= st << 17;
        return st;
    };
    float vals[400];
    int nv = 0;
    for (int i = 0; i < 300; ++i) {
        const uint64_t r = next();
        const int e = (int)(r % 200) - 100;                    // exponent spread
        const float m = 1.0f + (float)((r >> 20) & 0xffff) / 65536.0f;
        float v = m;
        for (int k = 0; k < (e < 0 ? -e : e); ++k) v = e < 0 ? v * 0.5f : v * 2.0f;
        vals[nv++] = v;
    }
    for (int e = -20; e <= 20; e += 4) {
        float p = 1.0f;
        for (int k = 0; k < (e < 0 ? -e : e); ++k) p = e < 0 ? p * 0.5f : p * 2.0f;
        uint32_t b = bits(p);
        float lo, hi;
        const uint32_t bl = b - 1, bh = b + 1;
        std::memcpy(&lo, &bl, 4);
        std::memcpy(&hi, &bh, 4);
        vals[nv++] = p; vals[nv++] = lo; vals[nv++] = hi;
    }
    vals[nv++] = 0.0f;
    for (int i = 0; i < nv; ++i)
        for (int j = 0; j < nv; j += 7) {
            const float aq = vals[i], ak = vals[(i + j) % nv];
            std::printf("S %u %u %d %u\n", bits(aq), bits(ak), dit::fp8::score_exponent(aq, ak),
                        bits(dit::fp8::q_multiplier(aq, ak)));
        }
    return 0;
}
