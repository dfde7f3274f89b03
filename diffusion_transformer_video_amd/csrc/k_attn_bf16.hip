// Flash-style bf16 attention on gfx950 matrix cores (MFMA).
//
// o = softmax(q k^T / sqrt(d_head)) v per (sequence, head), bidirectional, over
// packed variable-length sequences ("Por que e absurdamente dificil gerar um
// filme inteiro usando IA", section "Matematica por tras"; the 1/sqrt(d_head)
// scale on rotated q, k from "DiT, Flow Matching e 3D Attention", section
// "3D-RoPE e atencao espaco-temporal"). The two products are the only dense
// contractions of the block's attention half and run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
// Work decomposition
//   * A block of NW waves owns 32*NW queries of one (sequence, head); each wave
//     owns 32 queries. Blocks are numbered so that consecutive work items land
//     on the same XCD (the dispatcher deals blocks round-robin over the 8 XCDs),
//     which keeps the blocks that share one head's K/V on one L2.
//   * Scores are computed transposed, S^T = K Q^T (32 keys x 32 queries per
//     MFMA tile). In the 32x32 accumulator layout a lane then holds 16 keys of a
//     single query, so the row max/sum is a per-lane reduction plus one
//     exchange with the lane 32 apart, and the probabilities are already in the
//     B-operand layout of the second product O^T += V^T P^T (the contraction
//     slots are a fixed permutation of the keys, applied to V^T when it is
//     staged).
//   * Q stays in VGPRs for the whole key loop (it is the B operand of S^T).
//   * K tiles (64 keys) are staged into LDS row-major with a 16-byte row pad;
//     V tiles are transposed on the way in (register 4x8 transpose) into
//     [d][key'] with the same slot permutation, so both operands are single
//     16-byte LDS reads per lane. Two LDS buffers: the global loads of tile
//     j+1 are in flight while tile j is consumed; one barrier per tile.
//   * Online softmax in the exp2 domain with the 1/sqrt(d) scale folded into
//     one fma. The running max is only raised (and O, l rescaled) when a new
//     tile maximum exceeds it by more than 2^8 -- a wave-uniform branch -- so
//     the rescale multiply is skipped on almost every tile; p stays <= 2^8.
//   * Only the last key tile of a sequence carries a mask; rows past the end of
//     the sequence are clamped on load and never stored.
#include <math.h>

#include "dit_device.hpp"
#include "dit_internal.h"

namespace dit {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLazyRescale = 8.0f;   // log2 headroom before the max is raised

template <int HD, int NW>
struct Cfg {
    static constexpr int NT = 64 * NW;         // threads per block
    static constexpr int BQ = 32 * NW;         // queries per block
    static constexpr int BK = 64;              // keys per tile
    static constexpr int KSTR = HD * 2 + 16;   // bytes per K row in LDS
    static constexpr int VSTR = BK * 2 + 16;   // bytes per V^T row in LDS
    static constexpr int KBYTES = BK * KSTR;
    static constexpr int VBYTES = HD * VSTR;
    static constexpr int BUF = KBYTES + VBYTES;
    static constexpr int LDS = 2 * BUF;
    static constexpr int NKK = HD / 16;        // k-steps of the S^T product
    static constexpr int NDT = HD / 32;        // 32-wide d tiles of O^T
    static constexpr int CPR = HD / 8;         // 16-byte chunks per row
    static constexpr int KCH = BK * CPR / NT;  // K chunks per thread per tile
    static constexpr int VK = (BK / 4) * CPR >= NT ? 4 : 2;   // keys per V unit
    static constexpr int VUN = (BK / VK) * CPR / NT;           // V units per thread
    static_assert(KCH >= 1 && KCH * NT == BK * CPR, "K staging must tile evenly");
    static_assert(VUN >= 1 && VUN * NT == (BK / VK) * CPR, "V staging must tile evenly");
    // staging registers of one tile (ext vectors stay in VGPRs; C arrays may not)
    typedef uint32_t KStage __attribute__((ext_vector_type(4 * KCH)));
    typedef uint32_t VStage __attribute__((ext_vector_type(4 * VUN * VK)));
};

// Position of key `k` (0..BK-1) inside a V^T row: within each group of 16 keys,
// bits 2 and 3 of the offset are swapped, so that the 8 contraction slots of
// lane group g for MFMA step t are the 8 consecutive positions 16t + 8g .. +7.
__device__ __forceinline__ int vt_pos(int k) {
    const int o = k & 15;
    return (k & ~15) | (((o >> 2) & 1) << 3) | (((o >> 3) & 1) << 2) | (o & 3);
}

template <int HD, int NW>
__device__ __forceinline__ void load_tile(const uint4* __restrict__ Kg, const uint4* __restrict__ Vg,
                                          int64_t ld16, int64_t len, int tid, int j,
                                          typename Cfg<HD, NW>::KStage& kst,
                                          typename Cfg<HD, NW>::VStage& vst) {
    using C = Cfg<HD, NW>;
    const int64_t kbase = (int64_t)j * C::BK;
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
        const int u = tid + C::NT * i;
        const int row = u / C::CPR, c = u % C::CPR;
        int64_t kr = kbase + row;
        kr = kr < len ? kr : len - 1;
        const uint4 t = Kg[kr * ld16 + c];
        kst[4 * i + 0] = t.x; kst[4 * i + 1] = t.y; kst[4 * i + 2] = t.z; kst[4 * i + 3] = t.w;
    }
#pragma unroll
    for (int i = 0; i < C::VUN; ++i) {
        const int u = tid + C::NT * i;
        const int c = u % C::CPR, kgp = u / C::CPR;
#pragma unroll
        for (int r = 0; r < C::VK; ++r) {
            int64_t kr = kbase + kgp * C::VK + r;
            kr = kr < len ? kr : len - 1;
            const uint4 t = Vg[kr * ld16 + c];
            const int o = 4 * (i * C::VK + r);
            vst[o + 0] = t.x; vst[o + 1] = t.y; vst[o + 2] = t.z; vst[o + 3] = t.w;
        }
    }
}

template <int HD, int NW>
__device__ __forceinline__ void store_tile(char* smem, int tid, int buf,
                                           const typename Cfg<HD, NW>::KStage& kst,
                                           const typename Cfg<HD, NW>::VStage& vst) {
    using C = Cfg<HD, NW>;
    char* Kb = smem + buf * C::BUF;
    char* Vb = Kb + C::KBYTES;
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
        const int u = tid + C::NT * i;
        const int row = u / C::CPR, c = u % C::CPR;
        *reinterpret_cast<uint4*>(Kb + row * C::KSTR + c * 16) =
            make_uint4(kst[4 * i + 0], kst[4 * i + 1], kst[4 * i + 2], kst[4 * i + 3]);
    }
#pragma unroll
    for (int i = 0; i < C::VUN; ++i) {
        const int u = tid + C::NT * i;
        const int c = u % C::CPR, kgp = u / C::CPR;
        const int pos = vt_pos(kgp * C::VK);
        // word p of the 16-byte row r of this unit: dims c*8 + 2p, c*8 + 2p + 1
#define VW(r, p) vst[4 * (i * C::VK + (r)) + (p)]
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int d = c * 8 + 2 * p;
            char* dst_e = Vb + d * C::VSTR + pos * 2;
            char* dst_o = dst_e + C::VSTR;
            if constexpr (C::VK == 4) {
                uint2 ev, od;
                ev.x = (VW(0, p) & 0xffffu) | (VW(1, p) << 16);
                ev.y = (VW(2, p) & 0xffffu) | (VW(3, p) << 16);
                od.x = (VW(0, p) >> 16) | (VW(1, p) & 0xffff0000u);
                od.y = (VW(2, p) >> 16) | (VW(3, p) & 0xffff0000u);
                *reinterpret_cast<uint2*>(dst_e) = ev;
                *reinterpret_cast<uint2*>(dst_o) = od;
            } else {
                *reinterpret_cast<uint32_t*>(dst_e) = (VW(0, p) & 0xffffu) | (VW(1, p) << 16);
                *reinterpret_cast<uint32_t*>(dst_o) = (VW(0, p) >> 16) | (VW(1, p) & 0xffff0000u);
            }
        }
#undef VW
    }
}

template <int HD, int NW>
__global__ __launch_bounds__(64 * NW, 2) void attn_bf16_kernel(AttnArgs a, int nqt) {
    using C = Cfg<HD, NW>;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];

    // ---- block -> (sequence, head, query tile), XCD-contiguous numbering
    const int total = (int)gridDim.x;
    const int b = (int)blockIdx.x;
    const int per = total / 8, rem = total % 8;
    const int xcd = b % 8, idx = b / 8;
    const int w = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int qt = w % nqt;
    const int head = (w / nqt) % a.heads;
    const int seq = w / (nqt * a.heads);

    int64_t s0, len;
    if (a.cu_seqlens == nullptr) {
        s0 = (int64_t)seq * a.max_seqlen;
        len = a.max_seqlen;
    } else {
        s0 = a.cu_seqlens[seq];
        len = (int64_t)a.cu_seqlens[seq + 1] - s0;
    }
    const int64_t q0 = (int64_t)qt * C::BQ;
    if (q0 >= len) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int64_t ld16 = (int64_t)a.heads * C::CPR;   // token stride in 16-byte chunks
    const uint4* Qg = reinterpret_cast<const uint4*>(a.q) + s0 * ld16 + (int64_t)head * C::CPR;
    const uint4* Kg = reinterpret_cast<const uint4*>(a.k) + s0 * ld16 + (int64_t)head * C::CPR;
    const uint4* Vg = reinterpret_cast<const uint4*>(a.v) + s0 * ld16 + (int64_t)head * C::CPR;

    // ---- Q (B operand of S^T = K Q^T): lane holds query l32, d = 16kk + 8g .. +7
    const int64_t my_q = q0 + wave * 32 + l32;
    const int64_t qrow = my_q < len ? my_q : len - 1;
    bf16x8 qreg[C::NKK];
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk)
        qreg[kk] = __builtin_bit_cast(bf16x8, Qg[qrow * ld16 + 2 * kk + g]);

    f32x16 O[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
    float m_run = -INFINITY;   // running max in the scaled log2 domain
    float l_run = 0.f;         // this lane's partial row sum (its 16 keys per tile)

    typename C::KStage kst;
    typename C::VStage vst;
    const int ntiles = (int)((len + C::BK - 1) / C::BK);

    load_tile<HD, NW>(Kg, Vg, ld16, len, tid, 0, kst, vst);
    store_tile<HD, NW>(smem, tid, 0, kst, vst);
    __syncthreads();

    const float c = a.scale_log2;
    for (int j = 0; j < ntiles; ++j) {
        const int buf = j & 1;
        const bool more = (j + 1) < ntiles;
        if (more) load_tile<HD, NW>(Kg, Vg, ld16, len, tid, j + 1, kst, vst);

        const char* Kb = smem + buf * C::BUF;
        const char* Vb = Kb + C::KBYTES;

        // ---- S^T = K Q^T for 2 blocks of 32 keys
        f32x16 S0, S1;
#pragma unroll
        for (int r = 0; r < 16; ++r) { S0[r] = 0.f; S1[r] = 0.f; }
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk) {
            const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(Kb + l32 * C::KSTR + kk * 32 + g * 16);
            const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(Kb + (32 + l32) * C::KSTR + kk * 32 + g * 16);
            S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[kk], S0, 0, 0, 0);
            S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[kk], S1, 0, 0, 0);
        }

        // ---- mask keys past the sequence end (last tile only)
        if (!more) {
            const int64_t kbase = (int64_t)j * C::BK;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kofs = 8 * (r >> 2) + 4 * g + (r & 3);
                if (kbase + kofs >= len) S0[r] = -INFINITY;
                if (kbase + 32 + kofs >= len) S1[r] = -INFINITY;
            }
        }

        // ---- online softmax (exp2 domain, lazy max)
        float mx = fmaxf(S0[0], S1[0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(S0[r], S1[r]));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mxs = mx * c;
        if (__builtin_amdgcn_ballot_w64(mxs > m_run + kLazyRescale) != 0) {
            const float m_new = fmaxf(m_run, mxs);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;
            m_run = m_new;
        }
        // probabilities -> bf16 B operands: key block kb, MFMA step t (8 keys each)
        auto exp_pack = [&](const f32x16& S, int t) -> bf16x8 {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = __builtin_amdgcn_exp2f(fmaf(S[8 * t + e], c, -m_run));
                l_run += p[e];
            }
            uint4 wv;
            wv.x = pack_bf16x2(p[0], p[1]); wv.y = pack_bf16x2(p[2], p[3]);
            wv.z = pack_bf16x2(p[4], p[5]); wv.w = pack_bf16x2(p[6], p[7]);
            return __builtin_bit_cast(bf16x8, wv);
        };
        const bf16x8 P00 = exp_pack(S0, 0), P01 = exp_pack(S0, 1);
        const bf16x8 P10 = exp_pack(S1, 0), P11 = exp_pack(S1, 1);

        // ---- O^T += V^T P^T
        const char* Vrow = Vb + l32 * C::VSTR + 16 * g;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
            const char* vr = Vrow + dt * 32 * C::VSTR;
            const bf16x8 v00 = *reinterpret_cast<const bf16x8*>(vr + 0);
            const bf16x8 v01 = *reinterpret_cast<const bf16x8*>(vr + 32);
            const bf16x8 v10 = *reinterpret_cast<const bf16x8*>(vr + 64);
            const bf16x8 v11 = *reinterpret_cast<const bf16x8*>(vr + 96);
            O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v00, P00, O[dt], 0, 0, 0);
            O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v01, P01, O[dt], 0, 0, 0);
            O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v10, P10, O[dt], 0, 0, 0);
            O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v11, P11, O[dt], 0, 0, 0);
        }

        if (more) store_tile<HD, NW>(smem, tid, buf ^ 1, kst, vst);
        __syncthreads();
    }

    // ---- normalise and store: lane holds query l32, d = 32dt + 8(r/4) + 4g + r%4
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.0f / l_tot;
    if (my_q < len) {
        uint2* Og = reinterpret_cast<uint2*>(reinterpret_cast<uint4*>(a.o) + (s0 + my_q) * ld16 +
                                             (int64_t)head * C::CPR);
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                uint2 wv;
                wv.x = pack_bf16x2(O[dt][4 * rg + 0] * inv, O[dt][4 * rg + 1] * inv);
                wv.y = pack_bf16x2(O[dt][4 * rg + 2] * inv, O[dt][4 * rg + 3] * inv);
                Og[(dt * 32 + 8 * rg + 4 * g) / 4] = wv;
            }
        }
    }
}

template <int HD, int NW>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
    using C = Cfg<HD, NW>;
    const int nqt = (a.max_seqlen + C::BQ - 1) / C::BQ;
    const int64_t total = (int64_t)nqt * a.heads * a.num_seqs;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_bf16_kernel<HD, NW>), dim3((unsigned)total), dim3(C::NT), 0, s, a, nqt);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn3d_bf16(const AttnArgs& a, hipStream_t s) {
    if (a.head_dim == 64) return launch_t<64, 4>(a, s);
    return launch_t<128, 4>(a, s);
}

}  // namespace dit
