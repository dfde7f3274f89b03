// Flow-matching training-side kernels for gfx950: the straight-path interpolant
// and the conditional flow-matching loss ("DiT, Flow Matching e 3D Attention",
// section "Flow Matching e Rectified Flow"):
//   x_t = (1 - t) x_0 + t x_1                       (one flow time per row)
//   L   = | u_theta(x_t, t) - (x_1 - x_0) |^2        (squared norm per sample)
//
// Both read the latent once (HBM-bound, a few MB to tens of MB per call).
// Interpolant: a flat stream of 8-value chunks; x_t is formed as
// fma(t, x1, (1 - t) x0), so t = 0 and t = 1 return x0 and x1 exactly.
// Loss: 8 lanes share a token (each walks every 8th chunk of its channels),
// their partial sums meet in three xor shuffles in a fixed order, and the
// token's squared norm is stored; a second launch sums each row's tokens in one
// block (fixed per-thread order, then an LDS tree), so the result does not
// depend on scheduling.
#include "dit_device.hpp"
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerToken = 8;

template <bool BF16>
__global__ __launch_bounds__(kThreads) void interpolant_kernel(InterpArgs a) {
    const int nchunk = a.channels >> 3;
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= a.tokens * nchunk) return;
    const float t = a.t_rows[(idx / nchunk) / a.tokens_per_row];
    float x0[8], x1[8], o[8];
    Vec8<BF16>::load(a.x0, idx, x0);
    Vec8<BF16>::load(a.x1, idx, x1);
    const float s = 1.0f - t;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = fmaf(t, x1[e], s * x0[e]);
    Vec8<BF16>::store(a.xt, idx, o);
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void cfm_token_kernel(CfmArgs a) {
    const int nchunk = a.channels >> 3;
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t tok = g / kLanesPerToken;
    const int sub = (int)(g % kLanesPerToken);
    float acc = 0.f;
    if (tok < a.tokens) {
        for (int c = sub; c < nchunk; c += kLanesPerToken) {
            const int64_t idx = tok * nchunk + c;
            float u[8], x0[8], x1[8];
            Vec8<BF16>::load(a.u, idx, u);
            Vec8<BF16>::load(a.x0, idx, x0);
            Vec8<BF16>::load(a.x1, idx, x1);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = u[e] - (x1[e] - x0[e]);
                acc = fmaf(d, d, acc);
            }
        }
    }
    // the 8 lanes of a token are consecutive lanes of one wave (8 divides 64)
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (tok < a.tokens && sub == 0) a.loss_tok[tok] = acc;
}

// Per-row sums of the token losses: one block of kRowThreads per row; each thread
// keeps kRowAcc independent partial sums (kRowAcc loads in flight), added in a
// fixed order, then a fixed LDS tree -- deterministic. (A single long row, as at
// the 480P workload, is the latency-bound case: one serial load chain per
// thread took 36 us for 32,760 values.)
constexpr int kRowThreads = 1024;
constexpr int kRowAcc = 8;

__global__ __launch_bounds__(kRowThreads) void cfm_row_kernel(CfmArgs a) {
    __shared__ float red[kRowThreads];
    const int64_t row = blockIdx.x;
    const int64_t t0 = row * a.tokens_per_row, n = a.tokens_per_row;
    float acc[kRowAcc];
#pragma unroll
    for (int j = 0; j < kRowAcc; ++j) acc[j] = 0.f;
    for (int64_t base = 0; base < n; base += (int64_t)kRowThreads * kRowAcc) {
#pragma unroll
        for (int j = 0; j < kRowAcc; ++j) {
            const int64_t i = base + (int64_t)j * kRowThreads + threadIdx.x;
            if (i < n) acc[j] += a.loss_tok[t0 + i];
        }
    }
    float sum = acc[0];
#pragma unroll
    for (int j = 1; j < kRowAcc; ++j) sum += acc[j];
    red[threadIdx.x] = sum;
    __syncthreads();
    for (int w = kRowThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) a.loss_rows[row] = red[0];
}

}  // namespace

hipError_t launch_interpolant(const InterpArgs& a, bool bf16, hipStream_t s) {
    const int64_t n = a.tokens * (a.channels >> 3);
    const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
    if (bf16)
        hipLaunchKernelGGL(interpolant_kernel<true>, grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(interpolant_kernel<false>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_cfm_loss(const CfmArgs& a, bool bf16, hipStream_t s) {
    const int64_t n = a.tokens * kLanesPerToken;
    const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
    if (bf16)
        hipLaunchKernelGGL(cfm_token_kernel<true>, grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(cfm_token_kernel<false>, grid, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.loss_rows == nullptr) return e;
    const int64_t rows = a.tokens / a.tokens_per_row;
    hipLaunchKernelGGL(cfm_row_kernel, dim3((unsigned)rows), dim3(kRowThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace dit
