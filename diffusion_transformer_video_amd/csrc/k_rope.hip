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
// h', w') map is computed once per wave in scalar registers; each lane owns one
// 8-value chunk of the head vector (4 pairs) and evaluates the 4 pair rotations
// once, then rotates that chunk in each of the wave's heads of q and k
// (64 / (head_dim/8) heads per pass, so a pass is one contiguous, coalesced
// span of the token row). Angles are formed in turns, pos * theta / (2 pi) with
// theta from a float64 table per block, whose fraction is exact, and fed to the
// hardware sine and cosine of turns (max error 1.3e-7 on [0, 1), measured over
// 2^24 points): more accurate than float32 sincosf of pos * theta, whose
// argument already carries the rounding of theta and of the product, and 283
// instead of 616 vector instructions per wave (the library sincosf's range
// reduction and 64-bit index division), which leaves the vector ALU a third
// busy instead of three quarters.
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

// Token -> (t', h', w') of its sequence: 32-bit scalar arithmetic (NARROW, when
// tokens * waves-per-token and the frame size fit in 31 bits), else 64-bit.
template <bool NARROW>
__device__ __forceinline__ void token_position(const RopeArgs& a, int64_t tok, int& pt, int& ph, int& pw) {
    int64_t n;
    if (a.cu_seqlens == nullptr) {
        const int64_t L = (int64_t)a.grid_t * a.grid_h * a.grid_w;
        n = NARROW ? (int64_t)((uint32_t)tok % (uint32_t)L) : tok % L;
    } else {
        int lo = 0, hi = a.num_seqs;  // largest s with cu[s] <= tok (uniform: scalar loads)
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if ((int64_t)a.cu_seqlens[mid] <= tok) lo = mid; else hi = mid;
        }
        n = tok - (int64_t)a.cu_seqlens[lo];
    }
    if constexpr (NARROW) {
        const uint32_t hw = (uint32_t)a.grid_h * (uint32_t)a.grid_w, m = (uint32_t)n;
        const uint32_t t = m / hw, r = m - t * hw, h = r / (uint32_t)a.grid_w;
        pt = (int)t; ph = (int)h; pw = (int)(r - h * (uint32_t)a.grid_w);
    } else {
        const int64_t hw = (int64_t)a.grid_h * a.grid_w;
        pt = (int)(n / hw);
        ph = (int)((n / a.grid_w) % a.grid_h);
        pw = (int)(n % a.grid_w);
    }
}

// One wave rotates up to kHeadsPerWave heads of one token (its share of the
// token's heads). The pair frequencies of the head vector are computed once per
// block in float64 (theta_j = base^(-2j/d_axis), as revolutions per unit
// position), so each lane only forms pos * f, takes the fraction (exact) and
// evaluates sine and cosine of that many turns with the hardware sin/cos.
template <bool BF16, bool NARROW>
__global__ __launch_bounds__(64 * kWaves) void rope3d_kernel(RopeArgs a) {
    __shared__ float4 freq4[32];   // up to 128 pairs: revolutions per unit position
    const int lane = threadIdx.x & 63;
    if ((int)threadIdx.x < (a.head_dim >> 1)) {
        const int P = threadIdx.x, e1 = a.d_t >> 1, e2 = (a.d_t + a.d_h) >> 1;
        int j, da;
        if (P < e1) {
            j = P; da = a.d_t;
        } else if (P < e2) {
            j = P - e1; da = a.d_h;
        } else {
            j = P - e2; da = a.d_w;
        }
        const double turns = exp2(-(double)(2 * j) / (double)da * a.log2_base) * 0.15915494309189533577;
        reinterpret_cast<float*>(freq4)[P] = (float)turns;
    }
    __syncthreads();

    const int split = (a.heads + kHeadsPerWave - 1) / kHeadsPerWave;   // waves per token
    const int64_t wv = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    int64_t tok;
    int part;
    if constexpr (NARROW) {
        const uint32_t t = (uint32_t)wv / (uint32_t)split;
        tok = t;
        part = (int)((uint32_t)wv - t * (uint32_t)split);
    } else {
        tok = wv / split;
        part = (int)(wv - tok * split);
    }
    if (tok >= a.tokens) return;
    int pt, ph, pw;
    token_position<NARROW>(a, tok, pt, ph, pw);
    if (a.pos_out != nullptr && lane == 0 && part == 0) {
        a.pos_out[3 * tok + 0] = pt;
        a.pos_out[3 * tok + 1] = ph;
        a.pos_out[3 * tok + 2] = pw;
    }

    const int cph = a.head_dim >> 3;      // chunks per head (divides 64)
    const int hpp = 64 / cph;             // heads per pass
    const int c = lane % cph;
    const int hsub = lane / cph;

    const float4 f4 = freq4[c];           // the lane's 4 pairs: 8c .. 8c+7
    const float fq[4] = {f4.x, f4.y, f4.z, f4.w};
    float cs[4], sn[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int dim = 8 * c + 2 * p;
        const int pos = dim < a.d_t ? pt : (dim < a.d_t + a.d_h ? ph : pw);
        const float turns = __builtin_amdgcn_fractf((float)pos * fq[p]);
        sn[p] = __builtin_amdgcn_sinf(turns);
        cs[p] = __builtin_amdgcn_cosf(turns);
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
            const int64_t idx = tok_chunk + (int64_t)h * cph + c;
            qv[u].load_or_first(a.q, idx, h < he);
            if (a.k != nullptr) kv[u].load_or_first(a.k, idx, h < he);
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

template <bool BF16>
void launch_t(const RopeArgs& a, dim3 grid, dim3 block, bool narrow, hipStream_t s) {
    if (narrow)
        hipLaunchKernelGGL((rope3d_kernel<BF16, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((rope3d_kernel<BF16, false>), grid, block, 0, s, a);
}

}  // namespace

hipError_t launch_rope3d(const RopeArgs& a, bool bf16, hipStream_t s) {
    const int64_t waves = a.tokens * ((a.heads + kHeadsPerWave - 1) / kHeadsPerWave);
    if (waves > (int64_t)0x7fffffff * kWaves) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves));
    const dim3 block(64 * kWaves);
    // 32-bit token arithmetic when the wave index, the token index and the frame
    // size all fit in 31 bits
    const bool narrow = waves + kWaves < ((int64_t)1 << 31) && (int64_t)a.grid_h * a.grid_w < ((int64_t)1 << 31) &&
                        (a.cu_seqlens != nullptr || (int64_t)a.grid_t * a.grid_h * a.grid_w < ((int64_t)1 << 31));
    if (bf16)
        launch_t<true>(a, grid, block, narrow, s);
    else
        launch_t<false>(a, grid, block, narrow, s);
    return hipGetLastError();
}

}  // namespace dit
