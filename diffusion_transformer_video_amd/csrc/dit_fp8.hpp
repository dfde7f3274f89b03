// Per-head FP8 (OCP E4M3) scales shared by the quantisation kernel and the FP8
// attention kernel, for head_dim 128 ("DiT, Flow Matching e 3D Attention",
// section "Engenharia de inferencia e paralelismo de contexto: Ulysses, Ring
// Attention e FP8", names 8-bit attention without a scaling rule).
//
// k and v: amax -> 448, dequantisation scale amax / 448.
// q: its scale is chosen together with k's so that the score scale -- q's and
// k's dequantisation scales times log2(e) / sqrt(128), the factor that turns a
// dot product of codes into the base-2 exponent of the softmax -- is exactly
// 2^n. n is the smallest integer with 2^n >= amax_q amax_k log2(e) /
// (448^2 sqrt(128)), decided in float64 (the product of two floats is exact
// there), and q is multiplied by g = amax_k log2(e) / (448 sqrt(128)) 2^-n
// (float64, rounded once to float32): the largest |q| then maps into
// (224, 448]. When amax_q or amax_k is 0 every score is 0 whatever q holds: q's
// codes are 0 and n = 0. So are they when n would lie below -127: every score
// is then below 2^-127 times the largest product of codes (< 1e-31), so the
// weights are uniform to float32 precision whatever q holds (and 2^-n would
// overflow q's float32 multiplier). Above 127, n is kept at 127 (one E8M0 block
// scale).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {
namespace fp8 {

constexpr double kScoreT = 0x1.5519f01ffd935p-21;   // log2(e) / (448 * 448 * sqrt(128))
constexpr double kQMul = 0x1.2a76b21bfde0fp-12;     // log2(e) / (448 * sqrt(128))

// (host and device: a host program checks both against the oracle)
// The unclamped exponent (0 when either amax is 0).
__host__ __device__ inline int score_exponent_raw(float amax_q, float amax_k) {
    if (!(amax_q > 0.f) || !(amax_k > 0.f)) return 0;
    const double t = ((double)amax_q * (double)amax_k) * kScoreT;   // a normal double
    const uint64_t b = __builtin_bit_cast(uint64_t, t);
    const int e = (int)((b >> 52) & 0x7ff) - 1023;                 // t = 1.f 2^e
    return (b & 0xfffffffffffffull) != 0 ? e + 1 : e;
}

// True when q's codes are all 0: a zero amax, or scores below 2^-127.
__host__ __device__ inline bool q_codes_zero(float amax_q, float amax_k) {
    return !(amax_q > 0.f) || !(amax_k > 0.f) || score_exponent_raw(amax_q, amax_k) < -127;
}

__host__ __device__ inline int score_exponent(float amax_q, float amax_k) {
    if (q_codes_zero(amax_q, amax_k)) return 0;
    const int n = score_exponent_raw(amax_q, amax_k);
    return n > 127 ? 127 : n;
}

// q's float32 multiplier (0: codes 0)
__host__ __device__ inline float q_multiplier(float amax_q, float amax_k) {
    if (q_codes_zero(amax_q, amax_k)) return 0.f;
    const int n = score_exponent(amax_q, amax_k);
    const double p2 = __builtin_bit_cast(double, (uint64_t)(1023 - n) << 52);   // 2^-n, exact
    return (float)(((double)amax_k * kQMul) * p2);
}

}  // namespace fp8
}  // namespace dit
