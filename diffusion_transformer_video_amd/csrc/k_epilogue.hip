// Gated residual and rectified-flow Euler update for gfx950, optionally in one
// launch.
//
// Residual ("DiT, Flow Matching e 3D Attention", section "A ruptura da U-Net"):
//   x_out[tok][c] = x[tok][c] + alpha[row][c] * branch[tok][c]
// Euler ("Flow Matching e Rectified Flow" section of the same page):
//   z_out[tok][c] = z[tok][c] + dt_rows[row] * u[tok][c]
// and, with dt scaled by 1/2, the first stage of the midpoint sampler the same
// section names beside Euler.
//
// Both are HBM-bound streams (6 bytes per bf16 element). The residual runs as
// short column strips: a thread owns one 8-column chunk of kTokPerThread
// consecutive tokens (loads issued up front, kept in storage format) and reads
// the alpha chunk (a per-sample / per-frame row) once per strip; threads are
// numbered chunk-fastest over (strip, chunk). More threads with fewer loads each
// stream faster than long strips. The Euler part is a flat stream
// of 8-value chunks. In the fused launch the first blocks run the residual and
// the remaining blocks the Euler update: two disjoint passes, one launch.
#include "dit_device.hpp"
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerThread = 2;   // 8 per thread ran at 62-70% of HBM, 1-2 at 70-77%
constexpr int kEulerChunksPerThread = 2;

template <bool BF16>
__device__ __forceinline__ void residual_block(const ResidualArgs& r, int64_t blk) {
    const int nchunk = r.d_model >> 3;
    // flat index over (token group of kTokPerThread, column chunk), chunk fastest
    const int64_t fi = blk * kThreads + threadIdx.x;
    const int64_t ngroups = (r.tokens + kTokPerThread - 1) / kTokPerThread;
    if (fi >= ngroups * nchunk) return;
    const int c = (int)(fi % nchunk);
    const int64_t tok0 = (fi / nchunk) * kTokPerThread;
    Packed8<BF16> xv[kTokPerThread], bv[kTokPerThread];   // loads in flight, storage format
#pragma unroll
    for (int t = 0; t < kTokPerThread; ++t) {
        const int64_t tok = tok0 + t;
        if (tok < r.tokens) {
            xv[t].load(r.x, tok * nchunk + c);
            bv[t].load(r.branch, tok * nchunk + c);
        }
    }
    int64_t cur_row = -1;
    float al[8];
#pragma unroll
    for (int t = 0; t < kTokPerThread; ++t) {
        const int64_t tok = tok0 + t;
        if (tok < r.tokens) {
            const int64_t row = tok / r.tokens_per_row;
            if (row != cur_row) {
                load_f32x8(r.alpha, row * nchunk + c, al);
                cur_row = row;
            }
            float xf[8], bf[8], o[8];
            xv[t].unpack(xf);
            bv[t].unpack(bf);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = fmaf(al[e], bf[e], xf[e]);
            Vec8<BF16>::store(r.x_out, tok * nchunk + c, o);
        }
    }
}

template <bool BF16>
__device__ __forceinline__ void euler_block(const EulerArgs& e, int64_t blk) {
    const int nchunk = e.channels >> 3;
    const int64_t total = e.tokens * nchunk;
    const int64_t base = blk * (kThreads * kEulerChunksPerThread) + threadIdx.x;
    Packed8<BF16> zv[kEulerChunksPerThread], uv[kEulerChunksPerThread];
#pragma unroll
    for (int i = 0; i < kEulerChunksPerThread; ++i) {
        const int64_t idx = base + (int64_t)i * kThreads;
        if (idx < total) {
            zv[i].load(e.z, idx);
            uv[i].load(e.u, idx);
        }
    }
#pragma unroll
    for (int i = 0; i < kEulerChunksPerThread; ++i) {
        const int64_t idx = base + (int64_t)i * kThreads;
        if (idx < total) {
            const float dt = e.dt_rows[(idx / nchunk) / e.tokens_per_row] * e.dt_scale;
            float zf[8], uf[8], o[8];
            zv[i].unpack(zf);
            uv[i].unpack(uf);
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] = fmaf(dt, uf[k], zf[k]);
            Vec8<BF16>::store(e.z_out, idx, o);
        }
    }
}

int64_t residual_blocks(const ResidualArgs* r) {
    if (r == nullptr || r->tokens == 0) return 0;
    const int64_t nchunk = r->d_model >> 3;
    const int64_t ngroups = (r->tokens + kTokPerThread - 1) / kTokPerThread;
    return (ngroups * nchunk + kThreads - 1) / kThreads;
}

int64_t euler_blocks(const EulerArgs* e) {
    if (e == nullptr || e->tokens == 0) return 0;
    const int64_t total = e->tokens * (e->channels >> 3);
    const int64_t per = kThreads * kEulerChunksPerThread;
    return (total + per - 1) / per;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void epilogue_kernel(ResidualArgs r, EulerArgs e,
                                                            int64_t n_res_blocks) {
    const int64_t b = blockIdx.x;
    if (b < n_res_blocks)
        residual_block<BF16>(r, b);
    else
        euler_block<BF16>(e, b - n_res_blocks);
}

}  // namespace

hipError_t launch_epilogue(const ResidualArgs* r, const EulerArgs* e, bool bf16, hipStream_t s) {
    const int64_t nr = residual_blocks(r);
    const int64_t ne = euler_blocks(e);
    if (nr + ne == 0) return hipSuccess;
    ResidualArgs rr = r ? *r : ResidualArgs{};
    EulerArgs ee = e ? *e : EulerArgs{};
    const dim3 grid((unsigned)(nr + ne));
    if (bf16)
        hipLaunchKernelGGL(epilogue_kernel<true>, grid, dim3(kThreads), 0, s, rr, ee, nr);
    else
        hipLaunchKernelGGL(epilogue_kernel<false>, grid, dim3(kThreads), 0, s, rr, ee, nr);
    return hipGetLastError();
}

}  // namespace dit
