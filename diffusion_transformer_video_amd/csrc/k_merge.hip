// Partial-attention merge for gfx950: fold one partial result into a running
// accumulator.
//
// Ring attention ("DiT, Flow Matching e 3D Attention", section "Engenharia de
// inferencia e paralelismo de contexto: Ulysses, Ring Attention e FP8") attends
// a GPU's queries to one key/value block per ring step. With each block's
// output o_b normalised by its own exponential sum and lse_b = ln of that sum,
// two partials over disjoint key sets combine exactly:
//   lse = ln(e^lse_acc + e^lse_b)
//   o   = e^(lse_acc - lse) o_acc + e^(lse_b - lse) o_b
// A row whose sets are both empty (lse = -inf on both sides) stays o = 0,
// lse = -inf. The accumulator is fp32, so a ring of any length rounds each
// partial once (when it was stored) and the sum never in bf16.
//
// HBM-bound: per element, the fp32 accumulator is read and written and the
// partial read once (10 bytes with a bf16 partial). A thread owns one 8-value
// chunk; the chunks of a (token, head) row lie in one wave (64 is a multiple of
// head_dim / 8), so every lane reads the row's old lse_acc before the row's
// first lane stores the new one.
#include <math.h>

#include "dit_device.hpp"
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kThreads = 256;

template <bool BF16>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
    const int cpr = a.head_dim >> 3;   // chunks per row: 8 or 16
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t row = gid / cpr;
    if (row >= a.rows) return;
    const float la = a.lse_acc[row], lb = a.lse_b[row];
    float oa[8], ob[8], res[8];
    load_f32x8(a.o_acc, gid, oa);
    if constexpr (BF16)
        load_bf16x8_cached(a.o_b, gid, ob);
    else
        load_f32x8(reinterpret_cast<const float*>(a.o_b), gid, ob);
    const float m = fmaxf(la, lb);
    float lnew;
    if (m == -INFINITY) {
#pragma unroll
        for (int e = 0; e < 8; ++e) res[e] = 0.f;
        lnew = -INFINITY;
    } else {
        const float wa = expf(la - m), wb = expf(lb - m);   // one of them is 1
        const float sum = wa + wb;
        const float ca = wa / sum, cb = wb / sum;
#pragma unroll
        for (int e = 0; e < 8; ++e) res[e] = fmaf(ca, oa[e], cb * ob[e]);
        lnew = m + logf(sum);
    }
    f32x4* out = reinterpret_cast<f32x4*>(a.o_acc) + 2 * gid;
    out[0] = f32x4{res[0], res[1], res[2], res[3]};
    out[1] = f32x4{res[4], res[5], res[6], res[7]};
    if (gid % cpr == 0) a.lse_acc[row] = lnew;
}

}  // namespace

hipError_t launch_attn_merge(const MergeArgs& a, bool bf16, hipStream_t s) {
    const int64_t chunks = a.rows * (a.head_dim / 8);
    const dim3 grid((unsigned)((chunks + kThreads - 1) / kThreads));
    if (bf16)
        hipLaunchKernelGGL(merge_kernel<true>, grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(merge_kernel<false>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace dit
