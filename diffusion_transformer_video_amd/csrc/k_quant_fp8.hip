// Quantisation of q, k, v to 8-bit floats (OCP E4M3) for the FP8 attention
// kernel, on gfx950.
//
// "DiT, Flow Matching e 3D Attention", section "Engenharia de inferencia e
// paralelismo de contexto: Ulysses, Ring Attention e FP8", pairs
// FlashAttention-3 with 8-bit floating point quantisation. One scale per
// (tensor, head). k and v: amax_h = max |x[:, h, :]| maps to 448, the largest
// finite E4M3 value; codes are x * (448 / amax_h) rounded to nearest even
// (v_cvt_pk_fp8_f32), clamped to +-448 first; the dequantisation scale is
// amax_h / 448. q: its scale makes the score scale a power of two 2^n
// (dit_fp8.hpp), so the attention kernel applies it as a matrix-core block
// scale; its largest magnitude maps into (224, 448]. An all-zero head gets
// codes 0.
//
// Layout written for the attention kernel:
//   q8, k8  [tokens][heads][128] bytes, row-major like q and k;
//   v8t     [heads][128][ldv] bytes: V transposed, each sequence's keys in
//           tiles of 64 (the sequence padded with zero codes to a multiple of
//           64, sequences placed one after another), and inside a tile key
//           32b + 8q + 4h + i stored at column 32h + 16b + 4q + i. In the
//           32x32 accumulator layout of the scores, lane half h holds exactly
//           the keys of columns 32h .. 32h+31, so each lane's probabilities
//           and its V^T operand pair up byte for byte with no exchange.
//
// Three launches: clear amax; per-head amax (blocks reduce in registers and
// LDS, one atomic max per block -- max is order independent, so the result is
// deterministic); quantise (one block per (64-key tile, head)).
#include "dit_device.hpp"
#include "dit_fp8.hpp"
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int HD = 128;
constexpr int kThreads = 256;
constexpr int kAmaxTokens = 256;   // tokens per block of the amax pass
constexpr float kE4M3Max = 448.0f;

__global__ void amax_clear_kernel(float* amax, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) amax[i] = 0.0f;
}

__device__ __forceinline__ float absmax8(const uint4& w) {
    const uint32_t m = 0x7fff7fffu;   // clear both bf16 sign bits; compare as floats
    const uint32_t a = w.x & m, b = w.y & m, c = w.z & m, d = w.w & m;
    float r = fmaxf(fmaxf(bf16lo(a), bf16hi(a)), fmaxf(bf16lo(b), bf16hi(b)));
    return fmaxf(r, fmaxf(fmaxf(bf16lo(c), bf16hi(c)), fmaxf(bf16lo(d), bf16hi(d))));
}

__global__ __launch_bounds__(kThreads) void amax_kernel(QuantFp8Args a) {
    __shared__ float red[3][kThreads / 64];
    const int head = blockIdx.y;
    const int64_t t0 = (int64_t)blockIdx.x * kAmaxTokens;
    float m[3] = {0.f, 0.f, 0.f};
    const void* src[3] = {a.q, a.k, a.v};
    for (int idx = threadIdx.x; idx < kAmaxTokens * (HD / 8); idx += kThreads) {
        const int64_t tok = t0 + idx / (HD / 8);
        if (tok >= a.tokens) break;
        const int64_t chunk = (tok * a.heads + head) * (HD / 8) + idx % (HD / 8);
#pragma unroll
        for (int t = 0; t < 3; ++t) m[t] = fmaxf(m[t], absmax8(reinterpret_cast<const uint4*>(src[t])[chunk]));
    }
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        float v = m[t];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
        if ((threadIdx.x & 63) == 0) red[t][threadIdx.x >> 6] = v;
    }
    __syncthreads();
    if (threadIdx.x < 3) {
        float v = 0.f;
        for (int w = 0; w < kThreads / 64; ++w) v = fmaxf(v, red[threadIdx.x][w]);
        // non-negative floats order like their bit patterns
        atomicMax(reinterpret_cast<unsigned int*>(a.amax) + threadIdx.x * a.heads + head, __float_as_uint(v));
    }
}

// A head's float32 multiplier, applied as (x * pre) * inv. k and v: 448 / amax,
// except below amax = 2^-100, where that quotient can overflow: there x is
// scaled by 2^64 first and the quotient taken of amax * 2^64 (both exact
// power-of-two scalings, so the product is the same float32 value wherever the
// plain form is finite). inv = 0: codes 0.
struct Mul {
    float pre, inv;
};
__device__ __forceinline__ Mul kv_multiplier(float amax) {
    if (!(amax > 0.f)) return {1.f, 0.f};
    if (amax < 0x1p-100f) return {0x1p64f, kE4M3Max / (amax * 0x1p64f)};
    return {1.f, kE4M3Max / amax};
}

// 8 bf16 values (one 16-byte chunk) -> 8 E4M3 codes (as two dwords)
__device__ __forceinline__ uint2 quant8(const uint4& w, Mul m) {
    if (m.inv == 0.f) return make_uint2(0, 0);   // all-zero head: codes 0
    float f[8];
    f[0] = bf16lo(w.x); f[1] = bf16hi(w.x); f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
    f[4] = bf16lo(w.z); f[5] = bf16hi(w.z); f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
    if (m.pre != 1.f) {   // block-uniform
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] *= m.pre;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = fminf(fmaxf(f[e] * m.inv, -kE4M3Max), kE4M3Max);
    int lo = 0, hi = 0;
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], lo, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], hi, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// column of key w (0..63) of a tile in v8t (see the header)
__device__ __forceinline__ int vt_col(int w) {
    const int b = w >> 5, q = (w >> 3) & 3, h = (w >> 2) & 1, i = w & 3;
    return 32 * h + 16 * b + 4 * q + i;
}

__global__ __launch_bounds__(kThreads) void quant_kernel(QuantFp8Args a) {
    __shared__ uint8_t vt[HD * 64];
    const int head = blockIdx.y;
    // tile -> (sequence, tile of the sequence, its first column in v8t)
    int64_t g = blockIdx.x, s0, pstart = 0;
    int len, j;
    if (a.cu_seqlens == nullptr) {
        const int nt = (a.max_seqlen + 63) / 64;
        const int seq = (int)(g / nt);
        if (seq >= a.num_seqs) return;
        j = (int)(g % nt);
        s0 = (int64_t)seq * a.max_seqlen;
        len = a.max_seqlen;
        pstart = (int64_t)seq * nt * 64;
    } else {
        int seq = 0;
        for (; seq < a.num_seqs; ++seq) {
            const int ls = a.cu_seqlens[seq + 1] - a.cu_seqlens[seq];
            const int nt = (ls + 63) / 64;
            if (g < nt) break;
            g -= nt;
            pstart += (int64_t)nt * 64;
        }
        if (seq >= a.num_seqs) return;
        j = (int)g;
        s0 = a.cu_seqlens[seq];
        len = a.cu_seqlens[seq + 1] - a.cu_seqlens[seq];
    }
    const int n = min(64, len - 64 * j);   // keys in this tile (>= 1)
    const Mul iq = {1.f, fp8::q_multiplier(a.amax[head], a.amax[a.heads + head])};
    const Mul ik = kv_multiplier(a.amax[a.heads + head]);
    const Mul iv = kv_multiplier(a.amax[2 * a.heads + head]);
    for (int i = threadIdx.x; i < HD * 64 / 16; i += kThreads) reinterpret_cast<uint4*>(vt)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * (HD / 8); idx += kThreads) {
        const int w = idx / (HD / 8), c = idx % (HD / 8);
        if (w >= n) continue;
        const int64_t chunk = ((s0 + 64 * j + w) * a.heads + head) * (HD / 8) + c;
        reinterpret_cast<uint2*>(a.q8)[chunk] = quant8(reinterpret_cast<const uint4*>(a.q)[chunk], iq);
        reinterpret_cast<uint2*>(a.k8)[chunk] = quant8(reinterpret_cast<const uint4*>(a.k)[chunk], ik);
        const uint2 vq = quant8(reinterpret_cast<const uint4*>(a.v)[chunk], iv);
        const int col = vt_col(w);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vt[(8 * c + e) * 64 + col] = (uint8_t)(vq.x >> (8 * e));
            vt[(8 * c + 4 + e) * 64 + col] = (uint8_t)(vq.y >> (8 * e));
        }
    }
    __syncthreads();
    // the tile's 128 rows of 64 bytes
    uint8_t* dst = reinterpret_cast<uint8_t*>(a.v8t) + (int64_t)head * HD * a.ldv + pstart + 64 * (int64_t)j;
    for (int i = threadIdx.x; i < HD * 4; i += kThreads) {
        const int d = i >> 2, q = i & 3;
        *reinterpret_cast<uint4*>(dst + (int64_t)d * a.ldv + 16 * q) = reinterpret_cast<const uint4*>(vt)[i];
    }
}

}  // namespace

hipError_t launch_quant_fp8(const QuantFp8Args& a, hipStream_t s) {
    hipLaunchKernelGGL(amax_clear_kernel, dim3(1), dim3(256), 0, s, a.amax, 3 * a.heads);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g1((unsigned)((a.tokens + kAmaxTokens - 1) / kAmaxTokens), (unsigned)a.heads);
    hipLaunchKernelGGL(amax_kernel, g1, dim3(kThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // tiles: sum over sequences of ceil(len / 64) <= tokens / 64 + num_seqs
    const int64_t tiles = a.cu_seqlens == nullptr ? (int64_t)a.num_seqs * ((a.max_seqlen + 63) / 64)
                                                  : a.tokens / 64 + a.num_seqs;
    hipLaunchKernelGGL(quant_kernel, dim3((unsigned)tiles, (unsigned)a.heads), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace dit
