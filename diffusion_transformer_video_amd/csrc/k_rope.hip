// 3D rotary position embedding, in place on q and k, for gfx950.
//
// "DiT, Flow Matching e 3D Attention", section "3D-RoPE e atencao
// espaco-temporal": d_head = d_t + d_h + d_w; each slice turns coordinate pairs
// by angles driven by its own grid coordinate (frame t', row h', column w'),
// and the same rotation R_3D(t', h', w') is applied to q and k of every head.
//
// HBM-bound: q and k are each read and written once (8 bytes per bf16 element
// of q when both are rotated). One wave owns up to kHeadsPerWave heads of one
// token (a token's heads are split evenly over ceil(heads / kHeadsPerWave)
// waves: a wave streaming a whole 24- or 40-head token row reached only 59-64%
// of HBM bandwidth, 8-head shares 63-70%). The integer token -> (sequence, t',
// h', w') map is computed once per wave; each lane owns one 8-value chunk of
// the head vector (4 pairs) and evaluates the 4 pair angles once, then rotates
// that chunk in each of the wave's heads of q and k (64 / (head_dim/8) heads
// per pass, so a pass is one contiguous, coalesced span of the token row).
#include "dit_device.hpp"
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kWaves = 8;
constexpr int kUnroll = 2;
constexpr int kHeadsPerWave = 8;

__device__ __forceinline__ void rotate8(float (&f)[8], const float (&cs)[4], const float (&sn)[4]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float x0 = f[2 * p], x1 = f[2 * p + 1];
        f[2 * p] = x0 * cs[p] - x1 * sn[p];
        f[2 * p + 1] = x0 * sn[p] + x1 * cs[p];
    }
}

template <bool BF16>
__global__ __launch_bounds__(64 * kWaves) void rope3d_kernel(RopeArgs a) {
    const int lane = threadIdx.x & 63;
    const int split = (a.heads + kHeadsPerWave - 1) / kHeadsPerWave;   // waves per token
    const int64_t wv = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int64_t tok = wv / split;
    const int part = (int)(wv - tok * split);
    if (tok >= a.tokens) return;

    // token -> position within its sequence
    int64_t n;
    if (a.cu_seqlens == nullptr) {
        const int64_t L = (int64_t)a.grid_t * a.grid_h * a.grid_w;
        n = tok % L;
    } else {
        int lo = 0, hi = a.num_seqs;  // largest s with cu[s] <= tok
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if ((int64_t)a.cu_seqlens[mid] <= tok) lo = mid; else hi = mid;
        }
        n = tok - (int64_t)a.cu_seqlens[lo];
    }
    const int64_t hw = (int64_t)a.grid_h * a.grid_w;
    const int pt = (int)(n / hw);
    const int ph = (int)((n / a.grid_w) % a.grid_h);
    const int pw = (int)(n % a.grid_w);
    if (a.pos_out != nullptr && lane == 0 && part == 0) {
        a.pos_out[3 * tok + 0] = pt;
        a.pos_out[3 * tok + 1] = ph;
        a.pos_out[3 * tok + 2] = pw;
    }

    const int cph = a.head_dim >> 3;      // chunks per head (divides 64)
    const int hpp = 64 / cph;             // heads per pass
    const int c = lane % cph;
    const int hsub = lane / cph;

    float cs[4], sn[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int dim = 8 * c + 2 * p;
        int pos, j, da;
        if (dim < a.d_t) {
            pos = pt; j = dim >> 1; da = a.d_t;
        } else if (dim < a.d_t + a.d_h) {
            pos = ph; j = (dim - a.d_t) >> 1; da = a.d_h;
        } else {
            pos = pw; j = (dim - a.d_t - a.d_h) >> 1; da = a.d_w;
        }
        const float theta = exp2f(-(float)(2 * j) / (float)da * a.log2_base);
        sincosf((float)pos * theta, &sn[p], &cs[p]);
    }

    const int64_t tok_chunk = tok * (int64_t)a.heads * cph;
    // this wave's heads [hb, he); kUnroll passes at a time: all their loads are
    // issued before the first rotation, so each lane keeps 2 * kUnroll 16-byte
    // loads in flight
    const int hb = (a.heads * part) / split, he = (a.heads * (part + 1)) / split;
    for (int h0 = hb + hsub; h0 < he; h0 += kUnroll * hpp) {
        Packed8<BF16> qv[kUnroll], kv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int h = h0 + u * hpp;
            if (h < he) {
                const int64_t idx = tok_chunk + (int64_t)h * cph + c;
                qv[u].load(a.q, idx);
                if (a.k != nullptr) kv[u].load(a.k, idx);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int h = h0 + u * hpp;
            if (h < he) {
                const int64_t idx = tok_chunk + (int64_t)h * cph + c;
                float f[8];
                qv[u].unpack(f);
                rotate8(f, cs, sn);
                Vec8<BF16>::store(a.q, idx, f);
                if (a.k != nullptr) {
                    kv[u].unpack(f);
                    rotate8(f, cs, sn);
                    Vec8<BF16>::store(a.k, idx, f);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_rope3d(const RopeArgs& a, bool bf16, hipStream_t s) {
    const int64_t waves = a.tokens * ((a.heads + kHeadsPerWave - 1) / kHeadsPerWave);
    if (waves > (int64_t)0x7fffffff * kWaves) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves));
    const dim3 block(64 * kWaves);
    if (bf16)
        hipLaunchKernelGGL(rope3d_kernel<true>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(rope3d_kernel<false>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace dit
