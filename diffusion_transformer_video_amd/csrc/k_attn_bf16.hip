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
    static constexpr int ROWB = HD * 2;        // bytes per K / V row in LDS (no padding)
    static constexpr int CPR = HD / 8;         // 16-byte chunks per row
    static constexpr int RPB = 1024 / ROWB;    // rows per 1 KB block (one wave-wide load)
    static constexpr int KBYTES = BK * ROWB;
    static constexpr int BUF = 2 * KBYTES;     // K tile + V tile
    // double buffered: two separate LDS objects, so the compiler can tell that
    // the loads streaming into one never alias the reads of the other
    static constexpr int NBLK = KBYTES / 1024; // 1 KB blocks per K (or V) tile
    static constexpr int LPW = NBLK / NW;      // K (and V) block loads per wave per tile
    static constexpr int NKK = HD / 16;        // k-steps of the S^T product
    static constexpr int NDT = HD / 32;        // 32-wide d tiles of O^T
    static_assert(LPW >= 1 && LPW * NW == NBLK, "tile loads must split evenly over the waves");
    static_assert(CPR == 8 || CPR == 16, "head_dim 64 or 128");
};

// LDS swizzles (16-byte chunk granularity; rows are unpadded so whole 1 KB
// blocks arrive by direct global->LDS loads in lane order).
//  K: chunk c of row r sits at c ^ kswz(r). The K operand read of 16 lanes takes
//     16 consecutive rows at one logical chunk; the XOR spreads them over all
//     64 banks.
//  V: chunk c of key row r sits at c ^ vswz(r). A transposed read takes 4
//     consecutive key rows x 32 bytes per 16 lanes (64 bytes per 32 lanes); the
//     XOR moves the 4 rows onto disjoint chunk groups.
template <int CPR>
__device__ __forceinline__ int kswz(int r) { return (r / (16 / CPR)) & (CPR - 1); }
template <int CPR>
__device__ __forceinline__ int vswz(int r) { return 4 * ((r / (16 / CPR)) % (CPR / 4)); }

// Max / sum of x over the lane pair (l, l ^ 32): v_permlane32_swap exchanges the
// upper half of the first operand with the lower half of the second, so with
// both operands = x the two results hold (own, partner) in some order per lane.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Issue the direct global->LDS loads of one K/V tile (keys kbase..kbase+63 of
// the sequence) into LDS buffer `dst`. Wave w moves 1 KB blocks w, w+NW, ... of
// K and of V; in a block, lane L carries row RPB*blk + L/CPR, physical chunk
// L%CPR (hence logical chunk (L%CPR) ^ swizzle(row)). FULL: every row is inside
// the sequence and the per-lane offset is loop-invariant (rows step by the
// scalar offset); otherwise rows past the end are clamped to the last row.
template <int HD, int NW, bool FULL>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                           char* dst, int wave, int lane, uint32_t ldb,
                                           uint32_t kbase, uint32_t rows_left,
                                           uint32_t koff, uint32_t voff) {
    using C = Cfg<HD, NW>;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
        const int blk = wave + NW * i;
        const uint32_t row_step = (uint32_t)(C::RPB * NW * i);   // rows added by block i
        uint32_t ko = koff, vo = voff, so = (kbase + row_step) * ldb;
        if (!FULL) {
            const uint32_t r0 = (uint32_t)(C::RPB * wave + lane / C::CPR) + row_step;
            const uint32_t r = r0 < rows_left ? r0 : rows_left - 1;
            const uint32_t pc = (uint32_t)(lane % C::CPR);
            ko = r * ldb + ((pc ^ (uint32_t)kswz<C::CPR>((int)r0)) * 16);
            vo = r * ldb + ((pc ^ (uint32_t)vswz<C::CPR>((int)r0)) * 16);
            so = kbase * ldb;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(dst + blk * 1024), 16, (int)ko, (int)so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(dst + C::KBYTES + blk * 1024), 16, (int)vo,
                                                 (int)so, 0, 0);
    }
}

template <int HD, int NW>
__device__ __forceinline__ void issue_tile_any(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                               char* dst, int wave, int lane, uint32_t ldb,
                                               uint32_t kbase, uint32_t len, uint32_t koff, uint32_t voff) {
    if (kbase + Cfg<HD, NW>::BK <= len)
        issue_tile<HD, NW, true>(rk, rv, dst, wave, lane, ldb, kbase, len - kbase, koff, voff);
    else
        issue_tile<HD, NW, false>(rk, rv, dst, wave, lane, ldb, kbase, len - kbase, koff, voff);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// V^T operand for one MFMA step: 4 consecutive keys at Vaddr and 4 more 8 keys
// later (the two halves of the lane's 8 contraction slots), transposed on read.
__device__ __forceinline__ bf16x8 vt_operand(const char* Vaddr, int second) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(Vaddr));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(Vaddr + second));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Online-softmax update for one 32-key block of S^T (this lane: one query, 16
// keys) followed by its two MFMA steps of O^T += V^T P^T. The running max is only
// raised when the block max exceeds it by more than 2^kLazyRescale (wave-uniform
// branch, rare after the first block). Probabilities are rounded to bf16 for the
// MFMA, and the row sum accumulates exactly those rounded values (v_dot2 with
// ones), so the normalisation uses the weights the product used.
//
// vt[dt] points at this lane's V^T source for d tile dt, key block 0, step 0 of
// the current buffer; key block kb / step t / second half add
// (32kb + 16t + 8h) rows.
template <int HD, int NW, bool MASK>
__device__ __forceinline__ void block_softmax_pv(f32x16& S, const char* const (&vt)[Cfg<HD, NW>::NDT],
                                                 int kb, f32x16 (&O)[Cfg<HD, NW>::NDT], float& m_run,
                                                 float& l_run, float c, int g, int kofs0, int len) {
    using C = Cfg<HD, NW>;
    if constexpr (MASK) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (kofs0 + 8 * (r >> 2) + 4 * g + (r & 3) >= len) S[r] = -INFINITY;
    }
    float mx = __builtin_fmaxf(S[0], __builtin_fmaxf(S[1], S[2]));
#pragma unroll
    for (int r = 3; r < 15; r += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(S[r], S[r + 1]));
    mx = __builtin_fmaxf(mx, S[15]);
    const float mxs = pair_max(mx) * c;
    if (__builtin_amdgcn_ballot_w64(mxs > m_run + kLazyRescale) != 0) {
        const float m_new = __builtin_fmaxf(m_run, mxs);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;
        m_run = m_new;
    }
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(S[8 * t + 2 * e], c, -m_run));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(S[8 * t + 2 * e + 1], c, -m_run));
            w[e] = pack_bf16x2(p0, p1);
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e]), ones, l_run, false);
        }
        const bf16x8 P = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
            const bf16x8 v = vt_operand(vt[dt] + (32 * kb + 16 * t) * C::ROWB, 8 * C::ROWB);
            O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, P, O[dt], 0, 0, 0);
        }
    }
}

// One key tile of 64 keys in LDS buffer `buf`: S^T = K Q^T (two 32-key blocks)
// on MFMA, then per block the online softmax and O^T += V^T P^T on MFMA, so the
// second block's softmax can overlap the first block's products.
// kaddr[kk]: this lane's K operand address for k-step kk (row l32 of key block 0)
// in buffer 0; MASK: the tile may extend past the sequence end.
template <int HD, int NW, bool MASK>
__device__ __forceinline__ void tile_step(const char* bufp, const int (&kaddr)[Cfg<HD, NW>::NKK],
                                          const int (&vaddr)[Cfg<HD, NW>::NDT],
                                          const bf16x8 (&qreg)[Cfg<HD, NW>::NKK],
                                          f32x16 (&O)[Cfg<HD, NW>::NDT], float& m_run, float& l_run,
                                          float c, int g, int kbase, int len) {
    using C = Cfg<HD, NW>;
    f32x16 S0, S1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { S0[r] = 0.f; S1[r] = 0.f; }
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(bufp + kaddr[kk]);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(bufp + kaddr[kk] + 32 * C::ROWB);
        S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[kk], S0, 0, 0, 0);
        S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[kk], S1, 0, 0, 0);
    }
    const char* vt[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) vt[dt] = bufp + vaddr[dt];
    block_softmax_pv<HD, NW, MASK>(S0, vt, 0, O, m_run, l_run, c, g, kbase, len);
    block_softmax_pv<HD, NW, MASK>(S1, vt, 1, O, m_run, l_run, c, g, kbase + 32, len);
}

template <int HD, int NW>
__global__ __launch_bounds__(64 * NW, 2) void attn_bf16_kernel(AttnArgs a, int nqt) {
    using C = Cfg<HD, NW>;
    __shared__ __attribute__((aligned(1024))) char smem0[C::BUF];
    __shared__ __attribute__((aligned(1024))) char smem1[C::BUF];

    // ---- block -> (sequence, head, query tile), XCD-contiguous numbering
    const int total = (int)gridDim.x;
    const int b = (int)blockIdx.x;
    const int per = total / 8, rem = total % 8;
    const int xcd = b % 8, idx = b / 8;
    const int w = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    // the divisions run on the vector ALU; the results are block-uniform
    const int qt = __builtin_amdgcn_readfirstlane(w % nqt);
    const int head = __builtin_amdgcn_readfirstlane((w / nqt) % a.heads);
    const int seq = __builtin_amdgcn_readfirstlane(w / (nqt * a.heads));

    int64_t s0;
    int len;
    if (a.cu_seqlens == nullptr) {
        s0 = (int64_t)seq * a.max_seqlen;
        len = a.max_seqlen;
    } else {
        // uniform per block: keep them in SGPRs so the buffer descriptors are scalar
        const int c0 = __builtin_amdgcn_readfirstlane(a.cu_seqlens[seq]);
        const int c1 = __builtin_amdgcn_readfirstlane(a.cu_seqlens[seq + 1]);
        s0 = c0;
        len = c1 - c0;
    }
    const int q0 = qt * C::BQ;
    if (q0 >= len) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const uint32_t ldb = (uint32_t)a.heads * HD * 2;   // token stride in bytes
    const int64_t base = (s0 * a.heads + head) * (int64_t)HD;   // element offset of (s0, head, 0)
    const uint32_t span = (uint32_t)len * ldb;        // bytes of this sequence (< 2^31, host-checked)
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const __bf16*>(a.q) + base), (short)0, span, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const __bf16*>(a.k) + base), (short)0, span, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const __bf16*>(a.v) + base), (short)0, span, 0x00020000);

    // ---- per-lane, loop-invariant offsets
    // direct loads: lane carries row RPB*wave + lane/CPR of each of its blocks
    const int lrow = C::RPB * wave + lane / C::CPR;
    const int pc = lane % C::CPR;
    const uint32_t koff = (uint32_t)lrow * ldb + (uint32_t)((pc ^ kswz<C::CPR>(lrow)) * 16);
    const uint32_t voff = (uint32_t)lrow * ldb + (uint32_t)((pc ^ vswz<C::CPR>(lrow)) * 16);
    // K operand (A of S^T): row l32, logical chunk 2kk + g
    int kaddr[C::NKK];
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk)
        kaddr[kk] = l32 * C::ROWB + (((2 * kk + g) ^ kswz<C::CPR>(l32)) * 16);
    // V^T operand (A of O^T): 16-lane group hg = lane/16 covers d = 32dt + 16(hg%2) + i
    // (i = lane%16); its source lanes point at key row 4g + i/4 (+ block offsets),
    // 4 dims starting at 32dt + 16(hg%2) + 4(i%4).
    int vaddr[C::NDT];
    {
        const int i16 = lane & 15, hg = lane >> 4;
        const int vrow = 4 * g + i16 / 4;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
            const int d0 = 32 * dt + 16 * (hg & 1) + 4 * (i16 & 3);   // first dim of the 8-byte piece
            const int chunk = (d0 / 8) ^ vswz<C::CPR>(vrow);
            vaddr[dt] = C::KBYTES + vrow * C::ROWB + chunk * 16 + (d0 % 8) * 2;
        }
    }

    // ---- Q (B operand of S^T = K Q^T): lane holds query l32, d = 16kk + 8g .. +7
    const int my_q = q0 + wave * 32 + l32;
    const uint32_t qrow = (uint32_t)(my_q < len ? my_q : len - 1);
    bf16x8 qreg[C::NKK];
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk)
        qreg[kk] = __builtin_bit_cast(bf16x8, bload(rq, qrow * ldb + (2 * kk + g) * 16, 0));

    f32x16 O[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
    float m_run = -INFINITY;   // running max in the scaled log2 domain
    float l_run = 0.f;         // this lane's partial row sum (its 16 keys per tile)
    const float c = a.scale_log2;
    const int ntiles = (len + C::BK - 1) / C::BK;

    issue_tile_any<HD, NW>(rk, rv, smem0, wave, lane, ldb, 0, (uint32_t)len, koff, voff);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // tile j+1 streams into one buffer while tile j is consumed from the other;
    // unrolled by two so each buffer is a distinct object at every access
    for (int j = 0;;) {
        if (j + 1 >= ntiles) {
            tile_step<HD, NW, true>(smem0, kaddr, vaddr, qreg, O, m_run, l_run, c, g, j * C::BK, len);
            break;
        }
        issue_tile_any<HD, NW>(rk, rv, smem1, wave, lane, ldb, (uint32_t)(j + 1) * C::BK, (uint32_t)len,
                               koff, voff);
        tile_step<HD, NW, false>(smem0, kaddr, vaddr, qreg, O, m_run, l_run, c, g, j * C::BK, len);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        ++j;
        if (j + 1 >= ntiles) {
            tile_step<HD, NW, true>(smem1, kaddr, vaddr, qreg, O, m_run, l_run, c, g, j * C::BK, len);
            break;
        }
        issue_tile_any<HD, NW>(rk, rv, smem0, wave, lane, ldb, (uint32_t)(j + 1) * C::BK, (uint32_t)len,
                               koff, voff);
        tile_step<HD, NW, false>(smem1, kaddr, vaddr, qreg, O, m_run, l_run, c, g, j * C::BK, len);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        ++j;
    }

    // ---- normalise and store: lane holds query l32, d = 32dt + 8(r/4) + 4g + r%4
    const float inv = 1.0f / pair_sum(l_run);   // lanes l and l^32 summed disjoint keys
    if (my_q < len) {
        uint2* Og = reinterpret_cast<uint2*>(reinterpret_cast<__bf16*>(a.o) + base +
                                             (int64_t)my_q * a.heads * HD);
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
