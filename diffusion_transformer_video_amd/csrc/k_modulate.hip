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
// reductions. gamma/beta rows are shared by every token of a sample/frame: for
// wide bf16 rows a block of kWavesL waves (kWavesL consecutive tokens) stages the
// parameter row it shares in LDS once, so the parameter rows leave the cache
// once per kWavesL tokens instead of once per token; elsewhere they are served
// from cache per token. Large batches of such rows split each row over two
// waves (modulate_pair_kernel).
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

constexpr int kWavesL = 8;

// Same per-row arithmetic as modulate_kernel; gamma/beta of the block's tokens
// come from LDS when all kWavesL tokens use one parameter row (decided per
// block, so the branch is uniform), else from global memory per token. The x
// loads are issued before the staging loads and the barrier, so they overlap.
template <bool BF16, int CPL>
__global__ __launch_bounds__(64 * kWavesL) void modulate_lds_kernel(
    void* __restrict__ y, const void* __restrict__ x, const float* __restrict__ gamma,
    const float* __restrict__ beta, int64_t tokens, int d_model, int64_t tokens_per_row,
    float eps) {
    extern __shared__ float4 gb_lds[];   // [2][d_model / 4]: gamma then beta
    const int lane = threadIdx.x & 63;
    const int64_t tok0 = (int64_t)blockIdx.x * kWavesL;
    const int64_t tok = tok0 + (threadIdx.x >> 6);
    const int nchunk = d_model >> 3;
    const int64_t row_chunk = tok * nchunk;
    const bool live = tok < tokens;

    // unconditional loads (chunk 0 for idle lanes and rows past the end, never
    // used): loads under a divergent branch are not kept in flight together
    Packed8<BF16> v[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        v[i].load_or_first(x, row_chunk + c, live && c < nchunk);
    }
    const int64_t last = (tok0 + kWavesL < tokens ? tok0 + kWavesL : tokens) - 1;
    const int64_t prow0 = tok0 / tokens_per_row;
    const bool shared_row = (last / tokens_per_row) == prow0;
    if (shared_row) {
        const float4* g4 = reinterpret_cast<const float4*>(gamma + prow0 * d_model);
        const float4* b4 = reinterpret_cast<const float4*>(beta + prow0 * d_model);
        const int n4 = d_model >> 2;
        for (int i = threadIdx.x; i < n4; i += 64 * kWavesL) {
            gb_lds[i] = g4[i];
            gb_lds[n4 + i] = b4[i];
        }
    }
    __syncthreads();
    if (!live) return;

    float s = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        if (lane + 64 * i < nchunk) {
            float f[8];
            v[i].unpack(f);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += f[e];
        }
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
    const int64_t prow = tok / tokens_per_row;
#pragma unroll
    for (int i = 0; i < CPL; ++i) v[i].refresh();
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunk) {
            float f[8], g[8], b[8], o[8];
            v[i].unpack(f);
            if (shared_row) {
                const float4 g0 = gb_lds[2 * c], g1 = gb_lds[2 * c + 1];
                const float4 b0 = gb_lds[2 * nchunk + 2 * c], b1 = gb_lds[2 * nchunk + 2 * c + 1];
                g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
                g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
                b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w;
                b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
            } else {
                load_f32x8(gamma, prow * nchunk + c, g);
                load_f32x8(beta, prow * nchunk + c, b);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = fmaf(g[e], (f[e] - mean) * rstd, b[e]);
            Vec8<BF16>::store(y, row_chunk + c, o);
        }
    }
}

// Large batches of wide bf16 rows: each row split over a pair of waves (half the
// row each, so a wave streams half as much), kRows2 rows per block; the two
// partial sums of each pass meet in LDS, and the shared parameter row is
// staged in LDS as in modulate_lds_kernel. The mean and variance sums add the
// two halves' wave sums, so their rounding differs from the one-wave kernel's.
constexpr int kRows2 = 8;   // rows per block, two waves per row
template <bool BF16, int CPL>
__global__ __launch_bounds__(64 * 2 * kRows2) void modulate_pair_kernel(
    void* __restrict__ y, const void* __restrict__ x, const float* __restrict__ gamma,
    const float* __restrict__ beta, int64_t tokens, int d_model, int64_t tokens_per_row, float eps) {
    extern __shared__ float4 gb_lds[];
    __shared__ float red[2][2 * kRows2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t tok0 = (int64_t)blockIdx.x * kRows2;
    const int64_t tok = tok0 + (wave >> 1);
    const int half = wave & 1;
    const int nchunk = d_model >> 3;
    const int hch = (nchunk + 1) >> 1;
    const int cb = half * hch, ce = half ? nchunk : hch;
    const int64_t row_chunk = tok * nchunk;
    const bool live = tok < tokens;
    Packed8<BF16> v[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = cb + lane + 64 * i;
        if (live && c < ce) v[i].load(x, row_chunk + c); else v[i].zero();
    }
    const int64_t last = (tok0 + kRows2 < tokens ? tok0 + kRows2 : tokens) - 1;
    const int64_t prow0 = tok0 / tokens_per_row;
    const bool shared_row = (last / tokens_per_row) == prow0;
    if (shared_row) {
        const float4* g4 = reinterpret_cast<const float4*>(gamma + prow0 * d_model);
        const float4* b4 = reinterpret_cast<const float4*>(beta + prow0 * d_model);
        const int n4 = d_model >> 2;
        for (int i = threadIdx.x; i < n4; i += 64 * 2 * kRows2) {
            gb_lds[i] = g4[i];
            gb_lds[n4 + i] = b4[i];
        }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        float f[8];
        v[i].unpack(f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += f[e];
    }
    s = wave_sum(s);
    if (lane == 0) red[0][wave] = s;
    __syncthreads();
    const float inv_d = 1.0f / (float)d_model;
    const float mean = (red[0][wave & ~1] + red[0][wave | 1]) * inv_d;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) v[i].refresh();
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        if (cb + lane + 64 * i < ce) {
            float f[8];
            v[i].unpack(f);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float dlt = f[e] - mean;
                ss += dlt * dlt;
            }
        }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[1][wave] = ss;
    __syncthreads();
    const float var = (red[1][wave & ~1] + red[1][wave | 1]) * inv_d;
    const float rstd = 1.0f / sqrtf(var + eps);
    if (!live) return;
    const int64_t prow = tok / tokens_per_row;
#pragma unroll
    for (int i = 0; i < CPL; ++i) v[i].refresh();
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = cb + lane + 64 * i;
        if (c < ce) {
            float f[8], g[8], b[8], o[8];
            v[i].unpack(f);
            if (shared_row) {
                const float4 g0 = gb_lds[2 * c], g1 = gb_lds[2 * c + 1];
                const float4 b0 = gb_lds[2 * nchunk + 2 * c], b1 = gb_lds[2 * nchunk + 2 * c + 1];
                g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
                g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
                b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w;
                b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
            } else {
                load_f32x8(gamma, prow * nchunk + c, g);
                load_f32x8(beta, prow * nchunk + c, b);
            }
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
    // 16K+ rows of 2048+ bf16 values: two waves per row (one wave streaming a
    // whole 6-10 KB row reached 57-72% of HBM bandwidth at the 480P and packed-
    // frame workloads, pairs 72-75%; a batch of 8K rows is too few for blocks of
    // 16 waves, there the one-wave kernel stays ahead)
    if constexpr (BF16) if (nchunk >= 256 && a.tokens >= 16384) {
        const int cpl2 = ((nchunk + 1) / 2 + 63) / 64;
        const dim3 grid2((unsigned)((a.tokens + kRows2 - 1) / kRows2));
        const size_t lds2 = (size_t)a.d_model * 2 * sizeof(float);   // <= 64 KB
#define DIT_MODP_CASE(N)                                                                             \
        if (cpl2 <= N) {                                                                             \
            hipLaunchKernelGGL((modulate_pair_kernel<BF16, N>), grid2, dim3(64 * 2 * kRows2), lds2, s, \
                               a.y, a.x, a.gamma, a.beta, a.tokens, a.d_model, a.tokens_per_row,    \
                               a.eps);                                                               \
            return hipGetLastError();                                                                \
        }
        DIT_MODP_CASE(2)
        DIT_MODP_CASE(3)
        DIT_MODP_CASE(4)
        DIT_MODP_CASE(5)
        DIT_MODP_CASE(6)
        DIT_MODP_CASE(8)
#undef DIT_MODP_CASE
    }
    if constexpr (BF16) if (nchunk >= 256) {   // rows of 2048+ bf16 values: LDS-staged parameters
        const dim3 grid((unsigned)((a.tokens + kWavesL - 1) / kWavesL));
        const size_t lds = (size_t)a.d_model * 2 * sizeof(float);   // <= 64 KB
#define DIT_MODL_CASE(N)                                                                          \
        if (cpl <= N) {                                                                           \
            hipLaunchKernelGGL((modulate_lds_kernel<BF16, N>), grid, dim3(64 * kWavesL), lds, s,  \
                               a.y, a.x, a.gamma, a.beta, a.tokens, a.d_model, a.tokens_per_row, \
                               a.eps);                                                            \
            return hipGetLastError();                                                             \
        }
        DIT_MODL_CASE(4)
        DIT_MODL_CASE(6)
        DIT_MODL_CASE(8)
        DIT_MODL_CASE(10)
        DIT_MODL_CASE(12)
        DIT_MODL_CASE(16)
#undef DIT_MODL_CASE
    }
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
