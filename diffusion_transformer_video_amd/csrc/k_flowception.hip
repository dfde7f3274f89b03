// Flowception frame insertion and per-frame schedule for gfx950.
//
// "Flowception: Temporally Expansive Flow Matching for Video Generation"
// (technical summary, section 2): during sampling new frames are inserted
// between the existing ones; each starts as unit Gaussian noise with its own
// local time reset to 0, while the existing frames keep theirs. Here counts[f]
// new frames go right after existing frame f, taking the given noise frames in
// order; the packed batch (sequences of frames, tokens_per_frame token rows
// each) is rebuilt with new sequence offsets.
//
// Two launches, no scratch memory:
//   plan -- one block scans the counts (chunks of 1024 frames with a running
//           carry) and writes, per output frame, its local time and its source
//           (existing frame f, or -1 - n for noise frame n), and the new token
//           offsets of the sequences (each frame finds, by binary search, the
//           sequences that start at it).
//   copy -- one thread per 16-byte (bf16) / 32-byte (fp32) chunk of the output
//           latent reads its frame's source and copies from the latent or the
//           noise: a coalesced, HBM-bound gather.
// Schedule: dt_f = min(dt_max, 1 - t_f) and t_f += dt_f; a frame whose step is
// clipped lands on exactly 1 (1 - t_f is exact for t_f >= 1/2).
#include "dit_device.hpp"
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kThreads = 256;

__global__ __launch_bounds__(kPlanThreads) void insert_plan_kernel(InsertArgs a) {
    __shared__ int64_t wsum[kPlanThreads / 64];
    __shared__ int64_t carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) carry_s = 0;
    // counts are device data the host cannot check: mark every output frame
    // "no source" first, so frames the counts fail to cover are zero-filled by
    // the copy, and no write below goes past frames_out
    for (int64_t o = tid; o < a.frames_out; o += kPlanThreads) {
        a.src_out[o] = INT32_MIN;
        a.t_out[o] = 0.0f;
    }
    __syncthreads();
    const int64_t tpf = a.tokens_per_frame;
    for (int64_t base = 0; base < a.frames; base += kPlanThreads) {
        const int64_t f = base + tid;
        const int64_t c = f < a.frames ? (int64_t)a.counts[f] : 0;
        // inclusive scan of c over the wave, then over the waves of the block
        int64_t x = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int64_t y = __shfl_up(x, d);
            if (lane >= d) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        int64_t before = 0;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        const int64_t ex = carry_s + before + x - c;   // noise frames placed before frame f
        if (f < a.frames && f + ex >= 0 && f + ex < a.frames_out) {
            const int64_t o = f + ex;                   // output position of frame f
            a.t_out[o] = a.t_frames[f];
            a.src_out[o] = (int32_t)f;
            for (int64_t j = 0; j < c && o + 1 + j < a.frames_out; ++j) {   // c < 0: no iteration
                a.t_out[o + 1 + j] = 0.0f;
                a.src_out[o + 1 + j] = (int32_t)(-1 - (ex + j));
            }
            // sequences that start at frame f (several if some are empty)
            const int64_t key = f * tpf;
            int lo = 0, hi = a.num_seqs + 1;   // first s with cu[s] >= key
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if ((int64_t)a.cu_seqlens[mid] < key) lo = mid + 1; else hi = mid;
            }
            for (int s = lo; s <= a.num_seqs && (int64_t)a.cu_seqlens[s] == key; ++s)
                a.cu_out[s] = (int32_t)(o * tpf);
        }
        __syncthreads();   // every wave has read wsum and carry_s
        if (tid == 0) {
            int64_t tot = 0;
            for (int w = 0; w < kPlanThreads / 64; ++w) tot += wsum[w];
            carry_s += tot;
        }
        __syncthreads();
    }
    // sequences that start at the end (the closing offset, and empty ones there)
    if (tid == 0) {
        const int64_t key = a.frames * tpf;
        for (int s = a.num_seqs; s >= 0 && (int64_t)a.cu_seqlens[s] == key; --s)
            a.cu_out[s] = (int32_t)(a.frames_out * tpf);
    }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void insert_copy_kernel(InsertArgs a) {
    const int nchunk = a.channels >> 3;
    const int64_t per_frame = (int64_t)a.tokens_per_frame * nchunk;
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= a.frames_out * per_frame) return;
    const int64_t o = idx / per_frame, r = idx - o * per_frame;
    const int32_t s = a.src_out[o];
    const void* src = s >= 0 ? a.z : a.noise;
    const int64_t sf = s >= 0 ? s : -1 - (int64_t)s;
    const int64_t sidx = sf * per_frame + r;
    if (sf >= (s >= 0 ? a.frames : a.frames_out - a.frames)) {   // no valid source: zeros
        if constexpr (BF16) {
            __builtin_nontemporal_store(u32x4{0, 0, 0, 0}, reinterpret_cast<u32x4*>(a.z_out) + idx);
        } else {
            f32x4* q = reinterpret_cast<f32x4*>(a.z_out) + 2 * idx;
            q[0] = f32x4{0.f, 0.f, 0.f, 0.f};
            q[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        return;
    }
    if constexpr (BF16) {
        const u32x4 v = reinterpret_cast<const u32x4*>(src)[sidx];
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(a.z_out) + idx);
    } else {
        const f32x4* p = reinterpret_cast<const f32x4*>(src) + 2 * sidx;
        f32x4* q = reinterpret_cast<f32x4*>(a.z_out) + 2 * idx;
        const f32x4 v0 = p[0], v1 = p[1];
        __builtin_nontemporal_store(v0, q);
        __builtin_nontemporal_store(v1, q + 1);
    }
}

__global__ __launch_bounds__(kThreads) void schedule_kernel(float* dt_out, float* t, int64_t frames, float dt_max) {
    const int64_t f = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (f >= frames) return;
    const float tf = t[f];
    const float dt = fminf(dt_max, 1.0f - tf);
    dt_out[f] = dt;
    t[f] = tf + dt;
}

}  // namespace

hipError_t launch_insert_frames(const InsertArgs& a, bool bf16, hipStream_t s) {
    hipLaunchKernelGGL(insert_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = a.frames_out * a.tokens_per_frame * (a.channels >> 3);
    const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
    if (bf16)
        hipLaunchKernelGGL(insert_copy_kernel<true>, grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(insert_copy_kernel<false>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_frame_schedule(float* dt_out, float* t, int64_t frames, float dt_max, hipStream_t s) {
    hipLaunchKernelGGL(schedule_kernel, dim3((unsigned)((frames + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                       dt_out, t, frames, dt_max);
    return hipGetLastError();
}

}  // namespace dit
