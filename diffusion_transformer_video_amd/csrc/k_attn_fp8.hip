// FP8 (OCP E4M3) attention on gfx950 matrix cores: both products on
// v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulation.
//
// o = softmax(q k^T / sqrt(d_head)) v per (sequence, head) on the dequantised
// values ("Por que e absurdamente dificil gerar um filme inteiro usando IA",
// section "Matematica por tras"; the 8-bit quantisation of "DiT, Flow Matching e
// 3D Attention", section "Engenharia de inferencia e paralelismo de contexto:
// Ulysses, Ring Attention e FP8"). Inputs are the codes and per-head amax values
// written by the quantisation kernel (k_quant_fp8.hip). q's scale makes the
// score scale (both dequantisation scales times log2(e) / sqrt(d)) a power of
// two 2^n (dit_fp8.hpp), applied by the score product's E8M0 block scales: the
// product's output is already the base-2 exponent of the softmax. v's scale
// amax / 448 goes into the final normalisation.
//
// Same organisation as the bf16 kernel (8 waves x 32 queries per block, 64-key
// tiles through 3-deep LDS rings loaded with direct HBM -> LDS loads, one
// barrier per tile, transposed scores S^T = K Q^T so a lane holds 32 keys of one
// query), with 8-bit operands:
//   * one 32x32x64 product consumes 64 head dims (S) or 64 keys (O), so a tile
//     takes 4 + 4 products per wave instead of 16 + 16, and moves half the LDS
//     bytes;
//   * operand bytes pair up by (lane half, byte index) in both A and B (probed),
//     so lane half h of the scores holds keys {32b + 8q + 4h + i}; V is stored
//     transposed with exactly those keys at columns 32h + 16b + 4q + i, and
//     the probabilities go from the score registers into the B operand with
//     no lane exchange and no transposing read;
//   * probabilities are 2^(s - m + 6) with an integer running max m, raised to
//     the ceiling of a tile max that exceeds it by more than 2: the largest
//     weight lies in [2^5, 2^8] (E4M3 holds up to 448). The shift is applied by
//     the conversion to E4M3: v_cvt_scalef32_pk_fp8_f32 divides by 2^(m - 6)
//     (only the scale's exponent is used; probed: round to nearest even), so
//     a score costs one exponential and half a conversion, no arithmetic. That
//     needs 2^s itself in float32 range, i.e. m in [-100, 120] for every query
//     of the block; an item whose max leaves that range is recomputed with the
//     shift subtracted before the exponential (2^(s - m), conversion scale
//     2^-6);
//   * the exponentials take about as many cycles per tile as the products (one
//     per score, each costing about two vector-ALU issue slots in a throughput
//     probe), so the vector ALU is the bound and the rest of the softmax is
//     kept off it: the row sums are one more product per tile, against a
//     constant operand whose row 0 is 1.0 (they add the same E4M3
//     probabilities the output product uses); the tile loop is unrolled over
//     the lcm of the 3-slot rings and the 2 score register sets, so LDS slot
//     addresses are immediate offsets and no score register is copied.
#include <math.h>

#include "dit_attn_common.hpp"
#include "dit_device.hpp"
#include "dit_fp8.hpp"
#include "dit_internal.h"

namespace dit {
namespace {

using namespace attn;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

constexpr int HD = 128, NW = 8, BK = 64, ST = 3;
constexpr int BQ = 32 * NW;          // queries per block
constexpr int TILEB = BK * HD;       // bytes of a K tile (64 rows x 128) or a V^T tile (128 rows x 64)
constexpr float kLazy = 2.0f;        // log2 headroom before the max is raised
constexpr float kPOffset = 6.0f;     // exp2 offset of the probabilities
constexpr float kE4M3Max = 448.0f;
constexpr float kFastMin = -100.0f, kFastMax = 120.0f;   // running max range of the unshifted exponentials

// LDS swizzles of 16-byte chunks: K rows have 8 chunks, V^T rows 4. A 16-lane
// group of an operand read takes 16 consecutive rows at one logical chunk; the
// XOR spreads them over all 64 banks.
__device__ __forceinline__ int kswz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int vswz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ i32x8 lds_op(uint32_t a0, uint32_t a1) {
    const u32x4 x = *(lds_u32x4*)(uintptr_t)a0;
    const u32x4 y = *(lds_u32x4*)(uintptr_t)a1;
    const i32x8 r = {(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
    return r;
}

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);   // e4m3 x e4m3, scale 1
}
// the same with the E8M0 block scale 2^(sb - 127) on B
__device__ __forceinline__ f32x16 mfma8s(const i32x8& a, const i32x8& b, const f32x16& c, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// max of the lane's 32 scores, a left-to-right chain (it compiles to 3-input
// maxima). No inline asm here: these reads follow the products closely, and the
// compiler inserts the wait states a vector read of a matrix-core result needs
// only before instructions it knows.
__device__ __forceinline__ float max32(const f32x16 (&S)[2]) {
    float a = __builtin_fmaxf(S[0][0], S[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) a = __builtin_fmaxf(__builtin_fmaxf(a, S[0][r]), S[1][r]);
    return a;
}

struct State {
    i32x4 rk, rv;
    int wave, lane, g, len, ntiles;
    uint32_t ldk, koff, voff;
    uint32_t kaddr[4];   // K operand chunk addresses in ring slot 0: (step i, chunk t) -> 2i + t
    uint32_t vaddr[2];   // V^T operand chunk addresses in ring slot 0, d block 0
    i32x8 qreg[2];       // Q (B operand of S^T) for head dims 0..63 and 64..127
    i32x8 ones;          // A operand whose row 0 is E4M3 1.0 at all 64 keys, rows 1..31 zero
    f32x16 O[4];
    f32x16 L;            // row sums: row 0 of L = ones x P (lanes of half 0, register 0)
    float m_run;         // running max (an integer, or -inf before the first tile)
    bool fast;           // wave-uniform: the unshifted exponentials are in range (max_update)
    int scb;             // E8M0 block scale of the score product's Q operand: 2^n
};

// K tile (keys kbase..kbase+63): wave w moves rows 8w..8w+7 (1 KB); lane L
// carries row 8w + L/8 at physical chunk L%8.
__device__ __forceinline__ void issue_k(const State& p, char* dst, uint32_t kbase) {
    const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(dst) + 1024 * p.wave);
    if (kbase + BK <= (uint32_t)p.len) {
        dma16(p.rk, lbase, p.koff, kbase * p.ldk);
    } else {   // last tile: rows past the end repeat the last row (masked later)
        const uint32_t r0 = (uint32_t)(8 * p.wave + p.lane / 8);
        const uint32_t rows_left = (uint32_t)p.len - kbase;
        const uint32_t r = r0 < rows_left ? r0 : rows_left - 1;
        dma16(p.rk, lbase, r * p.ldk + (uint32_t)(((p.lane % 8) ^ kswz((int)r0)) * 16), kbase * p.ldk);
    }
}

// V^T tile j: wave w moves rows 16w..16w+15 (1 KB); lane L carries row
// 16w + L/4 at physical chunk L%4. The sequence is padded to whole tiles.
__device__ __forceinline__ void issue_v(const State& p, char* dst, uint32_t j) {
    const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(dst) + 1024 * p.wave);
    dma16(p.rv, lbase, p.voff, 64 * j);
}

// The operand addresses are a per-lane part plus a slot offset that is a
// compile-time constant in the unrolled loop; the offset belongs in the LDS
// instruction's offset field. A local copy of the per-lane part, redefined by an
// empty asm (no instruction) in the same block as the reads, keeps the compiler
// from computing the sums elsewhere (hoisted out of the loop, each in a register
// of its own, or in a block before the reads where they cannot fold).
template <int N>
__device__ __forceinline__ void local_addrs(uint32_t (&a)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(a[i]));
}

__device__ __forceinline__ void s_tile(State& p, uint32_t slot_off, f32x16 (&S)[2]) {
    uint32_t (&ka)[4] = p.kaddr;
    local_addrs(ka);
#pragma unroll
    for (int r = 0; r < 16; ++r) { S[0][r] = 0.f; S[1][r] = 0.f; }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const uint32_t off = slot_off + kb * 32 * HD;
            S[kb] = mfma8s(lds_op(ka[2 * i] + off, ka[2 * i + 1] + off), p.qreg[i], S[kb], p.scb);
        }
}

__device__ __forceinline__ void mask_tile(f32x16 (&S)[2], int g, int kbase, int len) {
    // keys of the tile that exist; redefined here by an empty asm so that the 32
    // compares stay in this (once per sequence) branch: the last tile's index is
    // loop-invariant, and hoisted compares would hold 64 scalar registers per
    // unrolled step
    int rem = len - kbase;
    asm volatile("" : "+s"(rem));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int k = 8 * (r >> 2) + 4 * g + (r & 3);
        if (k >= rem) S[0][r] = -INFINITY;
        if (k + 32 >= rem) S[1][r] = -INFINITY;
    }
}

// raise the running max (rescaling O and l) to the ceiling of the tile max when
// that exceeds it by more than kLazy -- a wave-uniform branch. The factor is a
// power of two (integer maxima), so the rescale is exact. p.fast: every query
// of the wave has its max in [kFastMin, kFastMax], where the unshifted
// exponentials stay in float32 range.
__device__ __forceinline__ void max_update(State& p, const f32x16 (&S)[2]) {
    const float mxs = pair_max(max32(S));
    if (__builtin_amdgcn_ballot_w64(mxs > p.m_run + kLazy) != 0) {
        const float m_new = __builtin_fmaxf(p.m_run, __builtin_ceilf(mxs));
        const float alpha = __builtin_amdgcn_exp2f(p.m_run - m_new);
#pragma unroll
        for (int r = 0; r < 16; ++r) p.L[r] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) p.O[dt][r] *= alpha;
        p.m_run = m_new;
        p.fast = __builtin_amdgcn_ballot_w64(!(m_new >= kFastMin && m_new <= kFastMax)) == 0;
    }
}

// probabilities of the tile in S as the B operand of O^T += V^T P^T (byte
// 16b + r of the lane's 32 = score S[b][r]): E4M3(2^S / 2^(m - 6)) (FAST), or
// with the shift subtracted first, E4M3(2^(S - m) / 2^-6) -- the same values
// wherever the first form is in range
template <bool FAST>
__device__ __forceinline__ i32x8 probs(const State& p, const f32x16 (&S)[2]) {
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    // 2^(m - 6) (m - 6 in [-106, 114] when FAST: a normal float), or 2^-6
    const float pscale = FAST ? __int_as_float(((int)p.m_run - (int)kPOffset + 127) << 23) : 0x1p-6f;
    int w[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * t + e;
            v[e] = __builtin_amdgcn_exp2f(FAST ? S[j >> 4][j & 15] : S[j >> 4][j & 15] - p.m_run);
        }
        // the first conversion fills bytes 0-1 and keeps bytes 2-3 of its first
        // operand, which the second one overwrites: any register will do, and
        // v[0]'s (dead after it) spares a zeroing move
        s16x2 d = __builtin_bit_cast(s16x2, v[0]);
        d = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(d, v[0], v[1], pscale, false);
        d = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(d, v[2], v[3], pscale, true);
        w[t] = __builtin_bit_cast(int, d);
    }
    const i32x8 r = {w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7]};
    return r;
}

// P(j) from Sin and S(j+1) into Sout (the products are independent of the
// exponentials, which the compiler interleaves with them), in the wave's mode.
// The markers at both ends of each arm (empty asm, no instruction) keep the
// common products from being hoisted or sunk out of the arms, away from the
// exponentials they overlap.
__device__ __forceinline__ i32x8 probs_and_scores(State& p, const f32x16 (&Sin)[2], uint32_t kslot,
                                                  f32x16 (&Sout)[2]) {
    i32x8 P;
    if (p.fast) {
        asm volatile("; fast probabilities");
        P = probs<true>(p, Sin);
        s_tile(p, kslot, Sout);
        asm volatile("; fast probabilities end");
    } else {
        asm volatile("; shifted probabilities");
        P = probs<false>(p, Sin);
        s_tile(p, kslot, Sout);
        asm volatile("; shifted probabilities end");
    }
    return P;
}

__device__ __forceinline__ void pv_tile(State& p, uint32_t slot_off, const i32x8& P) {
    uint32_t (&va)[2] = p.vaddr;
    local_addrs(va);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        const uint32_t off = slot_off + dt * 32 * BK;
        p.O[dt] = mfma8(lds_op(va[0] + off, va[1] + off), P, p.O[dt]);
    }
    p.L = mfma8(p.ones, P, p.L);
}

// K and V^T tile rings in LDS (one kernel in this file uses them); addressed
// directly, so every slot address is a compile-time constant
__shared__ __attribute__((aligned(1024))) char kring[ST][TILEB];
__shared__ __attribute__((aligned(1024))) char vring[ST][TILEB];


// Step j (j = J mod 6) of the key loop: Sin holds S(j); K(j+1), V(j) are resident
// in slots (J+1) % 3, J % 3. Issues K(j+3), V(j+2); leaves S(j+1) in Sout.
template <int J>
__device__ __forceinline__ void step(State& p, int j, const f32x16 (&Sin)[2], f32x16 (&Sout)[2]) {
    const int kn = j + 3, vn = j + 2;
    const bool ik = kn < p.ntiles, iv = vn < p.ntiles;
    if (ik) issue_k(p, kring[(J + 3) % ST], (uint32_t)kn * BK);
    if (iv) issue_v(p, vring[(J + 2) % ST], (uint32_t)vn);
    const i32x8 P = probs_and_scores(p, Sin, ((J + 1) % ST) * TILEB, Sout);
    pv_tile(p, (J % ST) * TILEB, P);
    if (j + 1 == p.ntiles - 1) mask_tile(Sout, p.g, (j + 1) * BK, p.len);
    max_update(p, Sout);
    // the next step reads K(j+2), V(j+1), issued one step earlier; this step's
    // own loads (completing in issue order) may stay in flight
    if (ik)
        asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if (iv)
        asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

// The same step with run-time slots, S(j) -> S(j+1) in place (the fewer than
// six steps after the unrolled passes)
__device__ __forceinline__ void step_rt(State& p, int j, f32x16 (&S)[2]) {
    const int kn = j + 3, vn = j + 2;
    const bool ik = kn < p.ntiles, iv = vn < p.ntiles;
    if (ik) issue_k(p, kring[kn % ST], (uint32_t)kn * BK);
    if (iv) issue_v(p, vring[vn % ST], (uint32_t)vn);
    f32x16 Sn[2];
    const i32x8 P = probs_and_scores(p, S, (uint32_t)((j + 1) % ST) * TILEB, Sn);
    S[0] = Sn[0];
    S[1] = Sn[1];
    pv_tile(p, (uint32_t)(j % ST) * TILEB, P);
    if (j + 1 == p.ntiles - 1) mask_tile(S, p.g, (j + 1) * BK, p.len);
    max_update(p, S);
    if (ik)
        asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if (iv)
        asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

__global__ __launch_bounds__(64 * NW, 1) void attn_fp8_kernel(AttnFp8Args a, int nqt) {

    BlockWork bw;
    if (!decode_block(a.cu_seqlens, a.cu_seqlens, a.num_seqs, a.max_seqlen, a.max_seqlen, a.heads, nqt, BQ, bw))
        return;
    const int head = bw.head, len = bw.len;
    const int q0 = bw.qt * BQ;
    if (q0 >= len) return;
    // first column of the sequence in v8t: sequences padded to whole tiles
    int64_t pstart;
    if (a.cu_seqlens == nullptr) {
        pstart = (int64_t)bw.seq * ((a.max_seqlen + BK - 1) / BK) * BK;
    } else {
        pstart = 0;
        for (int s = 0; s < bw.seq; ++s) {
            const int ls = __builtin_amdgcn_readfirstlane(a.cu_seqlens[s + 1] - a.cu_seqlens[s]);
            pstart += (int64_t)((ls + BK - 1) / BK) * BK;
        }
    }

    State p;
    const int tid = thread_index();
    p.lane = tid & 63;
    p.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    p.g = p.lane >> 5;
    const int l32 = p.lane & 31;
    p.len = len;
    p.ntiles = (len + BK - 1) / BK;
    p.ldk = (uint32_t)a.heads * HD;   // token stride of q8 / k8 in bytes
    const int64_t base = (bw.s0 * a.heads + head) * (int64_t)HD;
    const uint32_t span = (uint32_t)len * p.ldk;
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void*)(reinterpret_cast<const uint8_t*>(a.q8) + base), (short)0, span,
                                          0x00020000);
    p.rk = make_rsrc(reinterpret_cast<const uint8_t*>(a.k8) + base, span);
    p.rv = make_rsrc(reinterpret_cast<const uint8_t*>(a.v8t) + (int64_t)head * HD * a.ldv + pstart,
                     (uint32_t)(HD * a.ldv - pstart));
    {
        const int kr = 8 * p.wave + p.lane / 8;
        p.koff = (uint32_t)kr * p.ldk + (uint32_t)(((p.lane % 8) ^ kswz(kr)) * 16);
        const int vr = 16 * p.wave + p.lane / 4;
        p.voff = (uint32_t)vr * (uint32_t)a.ldv + (uint32_t)(((p.lane % 4) ^ vswz(vr)) * 16);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
            p.kaddr[2 * i + t] = lds_addr(kring[0]) + (uint32_t)(l32 * HD + (((4 * i + 2 * p.g + t) ^ kswz(l32)) * 16));
#pragma unroll
    for (int t = 0; t < 2; ++t)
        p.vaddr[t] = lds_addr(vring[0]) + (uint32_t)(l32 * BK + (((2 * p.g + t) ^ vswz(l32)) * 16));

    // ---- Q: lane holds query q0 + 32 wave + l32, head dims 64i + 32g .. +31
    const int my_q = q0 + 32 * p.wave + l32;
    {
        const uint32_t qrow = (uint32_t)(my_q < len ? my_q : len - 1);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint4 x = bload(rq, qrow * p.ldk + 64 * i + 32 * p.g, 0);
            const uint4 y = bload(rq, qrow * p.ldk + 64 * i + 32 * p.g + 16, 0);
            const i32x8 r = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
            p.qreg[i] = r;
        }
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) p.O[dt][r] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) p.L[r] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) p.ones[t] = l32 == 0 ? 0x38383838 : 0;   // E4M3 1.0 = 0x38
    p.m_run = -INFINITY;
    p.fast = false;   // set with the first tile's max
    p.scb = 127 + fp8::score_exponent(a.amax[head], a.amax[a.heads + head]);   // score scale 2^n
    const float sv = a.amax[2 * a.heads + head] / kE4M3Max;

    // ---- prologue: K(0), V(0), K(1) resident; S(0) and its max; then the loads a
    // step -1 would have issued (K(2), V(1))
    issue_k(p, kring[0], 0);
    issue_v(p, vring[0], 0);
    if (p.ntiles > 1) issue_k(p, kring[1], BK);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    f32x16 Sa[2], Sb[2];
    s_tile(p, 0, Sa);
    if (p.ntiles == 1) mask_tile(Sa, p.g, 0, len);
    max_update(p, Sa);
    __syncthreads();   // all reads of K(0) done before its slot is refilled
    if (p.ntiles > 2) issue_k(p, kring[2], 2 * BK);
    if (p.ntiles > 1) issue_v(p, vring[1], 1);

    // ---- steady state: passes of six steps (slots and score sets alternate with
    // compile-time indices, S(j) back in Sa after each pass), then the rest
    const int steps = p.ntiles - 1;
    int j = 0;
    for (; j + 6 <= steps; j += 6) {
        step<0>(p, j, Sa, Sb);
        step<1>(p, j + 1, Sb, Sa);
        step<2>(p, j + 2, Sa, Sb);
        step<3>(p, j + 3, Sb, Sa);
        step<4>(p, j + 4, Sa, Sb);
        step<5>(p, j + 5, Sb, Sa);
    }
    for (; j < steps; ++j) step_rt(p, j, Sa);
    {
        const i32x8 P = p.fast ? probs<true>(p, Sa) : probs<false>(p, Sa);
        pv_tile(p, (uint32_t)((p.ntiles - 1) % ST) * TILEB, P);
    }

    // ---- normalise and store: lane holds query my_q, d = 32dt + 8(r/4) + 4g + r%4;
    // the row sum is row 0 of L (half 0); half 1's register 0 holds row 4 (zero)
    const float inv = sv / pair_sum(p.L[0]);
    // the sequence's rows of o for this head as a range-checked buffer: rows past
    // its end store to kDropOffset (no lane-divergent branch)
    const uint32_t ostride = (uint32_t)a.heads * HD * 2;   // bytes per token row of o
    const __amdgpu_buffer_rsrc_t ro = out_rsrc(reinterpret_cast<__bf16*>(a.o) + base, (uint32_t)len * ostride);
    const uint32_t rowoff = (uint32_t)my_q * ostride;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            uint2 wv;
            wv.x = pack_bf16x2(p.O[dt][4 * rg + 0] * inv, p.O[dt][4 * rg + 1] * inv);
            wv.y = pack_bf16x2(p.O[dt][4 * rg + 2] * inv, p.O[dt][4 * rg + 3] * inv);
            bstore8(ro, wv, my_q < len ? rowoff + (uint32_t)(dt * 32 + 8 * rg + 4 * p.g) * 2 : kDropOffset);
        }
}

}  // namespace

hipError_t launch_attn3d_fp8(const AttnFp8Args& a, hipStream_t s) {
    const int nqt = (a.max_seqlen + BQ - 1) / BQ;
    const int64_t total = (int64_t)nqt * a.heads * a.num_seqs;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_fp8_kernel, dim3((unsigned)total), dim3(64 * NW), 0, s, a, nqt);
    return hipGetLastError();
}

}  // namespace dit
