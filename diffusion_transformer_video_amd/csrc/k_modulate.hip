// Fused LayerNorm + adaLN-Zero modulation for gfx950.
//
// y = gamma[row] * (x - mean) / sqrt(var + eps) + beta[row] per token row
// ("DiT, Flow Matching e 3D Attention", section "A ruptura da U-Net", block
// equations). HBM-bound: one read of x, one write of y.
//
// One wave owns one token row. Each lane holds CPL chunks of 8 values in
// registers in their storage format (bf16 stays packed: 4 VGPRs per 8 values,
// which keeps occupancy high), so the row is read from HBM exactly once; mean
// and variance are two exact passes over the registers with DPP wave
// reductions. gamma/beta rows are shared by every token of a sample/frame and
// are served from cache.
#include "dit_device.hpp"
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kWaves = 4;

template <bool BF16, int CPL>
__global__ __launch_bounds__(64 * kWaves) void modulate_kernel(
    void* __restrict__ y, const void* __restrict__ x, const float* __restrict__ gamma,
    const float* __restrict__ beta, int64_t tokens, int d_model, int64_t tokens_per_row,
    float eps) {
    const int lane = threadIdx.x & 63;
    const int64_t tok = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (tok >= tokens) return;
    const int nchunk = d_model >> 3;
    const int64_t row_chunk = tok * nchunk;

    // the row stays in registers in its storage format (one HBM read)
    Packed8<BF16> v[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunk) v[i].load(x, row_chunk + c); else v[i].zero();
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        float f[8];
        v[i].unpack(f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += f[e];
    }
    const float inv_d = 1.0f / (float)d_model;
    const float mean = wave_sum(s) * inv_d;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) v[i].refresh();
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        if (lane + 64 * i < nchunk) {
            float f[8];
            v[i].unpack(f);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float dlt = f[e] - mean;
                ss += dlt * dlt;
            }
        }
    }
    const float var = wave_sum(ss) * inv_d;
    const float rstd = 1.0f / sqrtf(var + eps);

    const int64_t prow = (tok / tokens_per_row) * nchunk;
#pragma unroll
    for (int i = 0; i < CPL; ++i) v[i].refresh();
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunk) {
            float f[8], g[8], b[8], o[8];
            v[i].unpack(f);
            load_f32x8(gamma, prow + c, g);
            load_f32x8(beta, prow + c, b);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = fmaf(g[e], (f[e] - mean) * rstd, b[e]);
            Vec8<BF16>::store(y, row_chunk + c, o);
        }
    }
}

template <bool BF16>
hipError_t launch_t(const ModulateArgs& a, hipStream_t s) {
    const int nchunk = a.d_model / 8;
    const int cpl = (nchunk + 63) / 64;
    const dim3 grid((unsigned)((a.tokens + kWaves - 1) / kWaves));
    const dim3 block(64 * kWaves);
#define DIT_MOD_CASE(N)                                                                     \
    if (cpl <= N) {                                                                         \
        hipLaunchKernelGGL((modulate_kernel<BF16, N>), grid, block, 0, s, a.y, a.x, a.gamma, \
                           a.beta, a.tokens, a.d_model, a.tokens_per_row, a.eps);           \
        return hipGetLastError();                                                           \
    }
    DIT_MOD_CASE(1)
    DIT_MOD_CASE(2)
    DIT_MOD_CASE(4)
    DIT_MOD_CASE(6)
    DIT_MOD_CASE(8)
    DIT_MOD_CASE(10)
    DIT_MOD_CASE(12)
    DIT_MOD_CASE(16)
#undef DIT_MOD_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_adaln_modulate(const ModulateArgs& a, bool bf16, hipStream_t s) {
    return bf16 ? launch_t<true>(a, s) : launch_t<false>(a, s);
}

}  // namespace dit
