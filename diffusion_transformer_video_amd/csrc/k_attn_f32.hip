// Full-precision (fp32) attention for gfx950 on the vector ALUs.
//
// o = softmax(q k^T / sqrt(d_head)) v per (sequence, head), bidirectional
// ("Por que e absurdamente dificil gerar um filme inteiro usando IA", section
// "Matematica por tras"; scale from "DiT, Flow Matching e 3D Attention",
// section "3D-RoPE e atencao espaco-temporal").
//
// fp32 activations are a small-workload path (the tiny block), kept in full
// fp32 so results stay within 1e-4 of the exact softmax: one thread owns one
// query row (q and the output accumulator in registers), key/value tiles are
// staged through LDS and read as broadcasts, and the softmax is evaluated
// online per key tile with exact expf. Queries and keys may come from separate
// packed sets (a sequence's keys in their own block); the row log-sum-exp of the
// scaled scores is m + ln l.
#include <math.h>

#include "dit_device.hpp"
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kQ = 64;   // queries per block (one wave)
constexpr int kK = 16;   // keys per LDS tile

template <int HD>
__global__ __launch_bounds__(kQ) void attn_f32_kernel(AttnArgs a) {
    __shared__ float ks[kK][HD];
    __shared__ float vs[kK][HD];
    const int head = blockIdx.y;
    const int seq = blockIdx.z;
    int64_t s0, s1, k0, k1;   // query rows / key rows of the sequence
    if (a.cu_seqlens == nullptr) {
        s0 = (int64_t)seq * a.max_seqlen;
        s1 = s0 + a.max_seqlen;
        k0 = (int64_t)seq * a.max_seqlen_k;
        k1 = k0 + a.max_seqlen_k;
    } else {
        s0 = a.cu_seqlens[seq];
        s1 = a.cu_seqlens[seq + 1];
        k0 = a.cu_seqlens_k[seq];
        k1 = a.cu_seqlens_k[seq + 1];
    }
    const int64_t len = s1 - s0, klen = k1 - k0;
    const int64_t q0 = (int64_t)blockIdx.x * kQ;
    if (q0 >= len) return;
    const int64_t qi = q0 + threadIdx.x;
    const bool active = qi < len;
    const int64_t ld = (int64_t)a.heads * HD;   // token stride in floats
    const float* Q = reinterpret_cast<const float*>(a.q) + s0 * ld + (int64_t)head * HD;
    const float* K = reinterpret_cast<const float*>(a.k) + k0 * ld + (int64_t)head * HD;
    const float* V = reinterpret_cast<const float*>(a.v) + k0 * ld + (int64_t)head * HD;

    float q[HD], o[HD];
    const int64_t qrow = active ? qi : 0;
#pragma unroll
    for (int d = 0; d < HD; ++d) {
        q[d] = Q[qrow * ld + d] * a.scale;
        o[d] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    for (int64_t kt = 0; kt < klen; kt += kK) {
        const int nk = (int)((klen - kt) < kK ? (klen - kt) : kK);
        __syncthreads();
        for (int idx = threadIdx.x; idx < kK * HD; idx += kQ) {
            const int r = idx / HD, d = idx % HD;
            const int64_t kr = kt + (r < nk ? r : 0);
            ks[r][d] = K[kr * ld + d];
            vs[r][d] = V[kr * ld + d];
        }
        __syncthreads();
        float s[kK];
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < kK; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int d = 0; d < HD; ++d) acc = fmaf(q[d], ks[r][d], acc);
            s[r] = (r < nk) ? acc : -INFINITY;
            mt = fmaxf(mt, s[r]);
        }
        const float mn = fmaxf(m, mt);
        const float corr = expf(m - mn);   // m = -inf on the first tile -> 0
        l *= corr;
#pragma unroll
        for (int d = 0; d < HD; ++d) o[d] *= corr;
#pragma unroll
        for (int r = 0; r < kK; ++r) {
            const float p = expf(s[r] - mn);
            l += p;
#pragma unroll
            for (int d = 0; d < HD; ++d) o[d] = fmaf(p, vs[r][d], o[d]);
        }
        m = mn;
    }
    if (active) {
        float* O = reinterpret_cast<float*>(a.o) + s0 * ld + (int64_t)head * HD;
        // no keys: the empty sum gives o = 0 and lse = -inf
        const float inv = klen > 0 ? 1.0f / l : 0.0f;
#pragma unroll
        for (int d = 0; d < HD; ++d) O[qi * ld + d] = o[d] * inv;
        if (a.lse != nullptr) a.lse[(s0 + qi) * a.heads + head] = klen > 0 ? m + logf(l) : -INFINITY;
    }
}

}  // namespace

hipError_t launch_attn3d_f32(const AttnArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.max_seqlen + kQ - 1) / kQ), (unsigned)a.heads,
                    (unsigned)a.num_seqs);
    if (a.head_dim == 64)
        hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(kQ), 0, s, a);
    else
        hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(kQ), 0, s, a);
    return hipGetLastError();
}

}  // namespace dit
