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
// Design
//   * A block of NW waves owns 32*NW queries of one (sequence, head); each wave
//     owns 32 queries. Work items are numbered head-major over the exact query
//     tiles of all packed sequences (longest first) and remapped so that
//     consecutive items land on the same XCD (the dispatcher deals blocks
//     round-robin over the 8 XCDs): every XCD gets whole heads of every
//     sequence, and its concurrent blocks share one head's K/V in its L2.
//   * Scores are computed transposed, S^T = K Q^T (32 keys x 32 queries per
//     MFMA tile). In the 32x32 accumulator layout a lane then holds 16 keys of a
//     single query, so the row max/sum is a per-lane reduction plus one
//     exchange with the lane 32 apart, and the probabilities are already in the
//     B-operand layout of the second product O^T += V^T P^T: the contraction
//     slots of a lane are two runs of 4 consecutive keys, which is exactly what
//     one transposed LDS read (ds_read_b64_tr_b16) returns from row-major V.
//   * Q stays in VGPRs for the whole key loop (it is the B operand of S^T).
//   * K and V tiles (64 keys) move HBM -> LDS with direct loads
//     (buffer_load_dwordx4 ... lds): no staging registers and no register
//     transpose. Rows are unpadded; XOR chunk swizzles keep the K operand reads
//     and the transposed V reads free of bank conflicts.
//   * Software pipeline: the K stream runs one tile ahead of V. Iteration j
//     holds S(j) in registers and, in one straight-line block, computes the
//     softmax of S(j) on the vector ALU while the matrix cores compute
//     S(j+1) = K(j+1) Q^T, then O += V(j) P(j). With 8 waves the K and V tiles
//     sit in three-slot LDS rings (96 KB): step j reads K(j+1) and V(j), K(j+2)
//     and V(j+1) have landed, K(j+3) and V(j+2) are being loaded (with 4 waves,
//     two-slot rings and one tile ahead). The loop is unrolled over six steps,
//     so every ring slot offset is a compile-time constant. The loads are
//     issued from inline asm and waited for explicitly, so the compiler never
//     stalls a read of one tile on the loads of later tiles in flight. One
//     barrier per tile.
//   * Online softmax in the exp2 domain with the 1/sqrt(d) scale folded into
//     one fma. The running max is only raised (and O, l rescaled) when a new
//     tile maximum exceeds it by more than 2^8 -- a wave-uniform branch -- so
//     the rescale multiply is skipped on almost every tile; p stays <= 2^8.
//     The row sum accumulates the bf16-rounded probabilities the product uses.
//   * Only the last key tile of a sequence carries a mask; rows past the end of
//     the sequence are clamped on load and never stored.
//   * Two launch forms run the same per-item code: one block per work item, or
//     (use_persistent below) one persistent block per compute unit drawing items
//     from per-XCD queues with stealing (the XCDs run at different clocks under
//     this load), whose last round is cut along the keys into pieces merged by
//     the last piece to finish (see dit_attn_common.hpp).
#include <math.h>

#define DIT_ATTN_PERSISTENT
#include "dit_attn_common.hpp"
#include "dit_device.hpp"
#include "dit_internal.h"

namespace dit {
namespace {

using namespace attn;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr float kLazyRescale = 8.0f;   // log2 headroom before the max is raised
// The persistent launch (per-XCD queues, split tail) is used from 4 work items
// per resident block (the queues even out the XCDs' clock differences), and from
// 2 when a one-block-per-item launch would leave its last round less than 90%
// full (the split tail fills it). Measured against the persistent launch
// without the split tail: 720P +2%, one GPU's Ulysses share (2.5 items per
// block) +8%, 480P within 1%; the image workload (3 whole rounds) runs 9% faster
// with one block per item than persistent.
//
// Only on the whole chip (256 CUs, 8 XCDs): the queues are per XCD and a split
// item's pieces are only taken on their own XCD (their partials never leave its
// L2), so every XCD must run blocks of the launch. A partitioned device (fewer
// XCDs) runs one block per item.
__host__ __forceinline__ bool use_persistent(int64_t grid, int64_t resident, int cus) {
    if (cus != 256 || resident < 8) return false;
    if (grid >= 4 * resident) return true;
    const int64_t last = grid % resident;
    return grid >= 2 * resident && last != 0 && 10 * last < 9 * resident;
}

template <int HD, int NW>
struct Cfg {
    static constexpr int BK = 64;              // keys per tile
    static constexpr int ROWB = HD * 2;        // bytes per K / V row in LDS (no padding)
    static constexpr int CPR = HD / 8;         // 16-byte chunks per row
    static constexpr int RPB = 1024 / ROWB;    // rows per 1 KB block (one wave-wide load)
    static constexpr int TILEB = BK * ROWB;    // bytes of one K (or V) tile
    static constexpr int NBLK = TILEB / 1024;  // 1 KB blocks per tile
    static constexpr int LPW = NBLK / NW;      // block loads per wave per tile
    // LDS ring depth per stream: with 8 waves (one block per CU) three K and three V
    // tiles fit (96 KB) and both streams run two tiles ahead; with 4 waves (two
    // blocks per CU) two of each (64 KB per block) and one tile ahead.
    static constexpr int ST = NW >= 8 ? 3 : 2;
    static constexpr int NKK = HD / 16;        // k-steps of the S^T product
    static constexpr int NDT = HD / 32;        // 32-wide d tiles of O^T
    static_assert(LPW >= 1 && LPW * NW == NBLK, "tile loads must split evenly over the waves");
    static_assert(CPR == 8 || CPR == 16, "head_dim 64 or 128");
};

// LDS swizzles (16-byte chunk granularity).
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

typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 16-byte LDS read at byte address a + OFF (OFF folds into the instruction)
template <int OFF>
__device__ __forceinline__ bf16x8 lds_read16(uint32_t a) {
    return *(lds_bf16x8*)(uintptr_t)(a + OFF);
}

// Direct global->LDS loads of one K or V tile (keys kbase..kbase+63 of the
// sequence) into the LDS tile at `dst`. Wave w moves 1 KB blocks w, w+NW, ...; in
// a block, lane L carries row RPB*blk + L/CPR at physical chunk L%CPR, i.e. the
// logical chunk (L%CPR) ^ swizzle(row), folded into the per-lane offset `off`.
// FULL: every row is inside the sequence; the offset is loop-invariant and the
// tile and block bases ride in the scalar offset. Otherwise rows past the end are
// clamped to the last row (their scores are masked / probabilities are 0).
template <int HD, int NW, bool FULL, bool ISV>
__device__ __forceinline__ void issue(const i32x4& rs, uint32_t lbase, int wave, int lane,
                                      uint32_t ldb, uint32_t kbase, uint32_t rows_left, uint32_t off) {
    using C = Cfg<HD, NW>;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
        const int blk = wave + NW * i;
        const uint32_t row_step = (uint32_t)(C::RPB * NW * i);
        uint32_t vo = off, so = (kbase + row_step) * ldb;
        if (!FULL) {
            const uint32_t r0 = (uint32_t)(C::RPB * wave + lane / C::CPR) + row_step;
            const uint32_t r = r0 < rows_left ? r0 : rows_left - 1;
            const uint32_t pc = (uint32_t)(lane % C::CPR);
            const uint32_t sw = ISV ? (uint32_t)vswz<C::CPR>((int)r0) : (uint32_t)kswz<C::CPR>((int)r0);
            vo = r * ldb + (pc ^ sw) * 16;
            so = kbase * ldb;
        }
        dma16(rs, __builtin_amdgcn_readfirstlane(lbase + blk * 1024), vo, so);
    }
}

template <int HD, int NW, bool ISV>
__device__ __forceinline__ void issue_any(const i32x4& rs, uint32_t lbase, int wave, int lane,
                                          uint32_t ldb, uint32_t kbase, uint32_t len, uint32_t off) {
    if (kbase + Cfg<HD, NW>::BK <= len)
        issue<HD, NW, true, ISV>(rs, lbase, wave, lane, ldb, kbase, len - kbase, off);
    else
        issue<HD, NW, false, ISV>(rs, lbase, wave, lane, ldb, kbase, len - kbase, off);
}

// K operands of one tile: for k-step kk and key block kb, this lane's 16 bytes
// (row 32kb + l32, logical chunk 2kk + g). All are read up front so their LDS
// latency hides behind the softmax of the previous tile.
template <int HD, int NW>
__device__ __forceinline__ void k_fetch(uint32_t kb, const uint32_t (&kaddr)[Cfg<HD, NW>::NKK],
                                        bf16x8 (&ka)[2 * Cfg<HD, NW>::NKK]) {
    using C = Cfg<HD, NW>;
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
        const uint32_t a = kaddr[kk] + kb;
        ka[2 * kk] = lds_read16<0>(a);
        ka[2 * kk + 1] = lds_read16<32 * C::ROWB>(a);
    }
}

// S^T = K Q^T for both 32-key blocks and all QB query blocks of this wave: each
// K operand read from LDS feeds QB products.
template <int HD, int NW, int QB>
__device__ __forceinline__ void s_mfma(const bf16x8 (&ka)[2 * Cfg<HD, NW>::NKK],
                                       const bf16x8 (&qreg)[QB][Cfg<HD, NW>::NKK], f32x16 (&S)[QB][2]) {
    using C = Cfg<HD, NW>;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) { S[qb][0][r] = 0.f; S[qb][1][r] = 0.f; }
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            S[qb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[2 * kk], qreg[qb][kk], S[qb][0], 0, 0, 0);
            S[qb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[2 * kk + 1], qreg[qb][kk], S[qb][1], 0, 0, 0);
        }
}

// S^T as above with the K operands read from LDS just before use (no prefetch
// registers; with QB = 2 every read already feeds two products).
template <int HD, int NW, int QB>
__device__ __forceinline__ void s_tile(uint32_t kb, const uint32_t (&kaddr)[Cfg<HD, NW>::NKK],
                                       const bf16x8 (&qreg)[QB][Cfg<HD, NW>::NKK], f32x16 (&S)[QB][2]) {
    using C = Cfg<HD, NW>;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) { S[qb][0][r] = 0.f; S[qb][1][r] = 0.f; }
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
        const uint32_t a = kaddr[kk] + kb;
        const bf16x8 a0 = lds_read16<0>(a);
        const bf16x8 a1 = lds_read16<32 * C::ROWB>(a);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            S[qb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[qb][kk], S[qb][0], 0, 0, 0);
            S[qb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[qb][kk], S[qb][1], 0, 0, 0);
        }
    }
}

// Keys >= len of the tile starting at kbase get score -inf (last tile only).
template <int QB>
__device__ __forceinline__ void mask_tile(f32x16 (&S)[QB][2], int g, int kbase, int len) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int k = kbase + 8 * (r >> 2) + 4 * g + (r & 3);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            if (k >= len) S[qb][0][r] = -INFINITY;
            if (k + 32 >= len) S[qb][1][r] = -INFINITY;
        }
    }
}

// a left-to-right chain: it compiles to 3-input maxima (a balanced tree of
// pairs does not)
__device__ __forceinline__ float max32(const f32x16& S0, const f32x16& S1) {
    float mx = __builtin_fmaxf(S0[0], S1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = __builtin_fmaxf(__builtin_fmaxf(mx, S0[r]), S1[r]);
    return mx;
}

// Online-softmax bookkeeping of one tile for one query block: the scaled tile
// max (tile_max), then raise the running max (and rescale O and l) only if the
// tile max exceeds it by more than 2^kLazyRescale (raise_max; wave-uniform
// branch).
__device__ __forceinline__ float tile_max(const f32x16& S0, const f32x16& S1, float c) {
    return pair_max(max32(S0, S1)) * c;
}

template <int NDT>
__device__ __forceinline__ void raise_max(float mxs, f32x16 (&O)[NDT], float& m_run, float& l_run) {
    if (__builtin_amdgcn_ballot_w64(mxs > m_run + kLazyRescale) != 0) {
        const float m_new = __builtin_fmaxf(m_run, mxs);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;
        m_run = m_new;
    }
}

// Probabilities of 8 scores -> one bf16x8 B operand.
__device__ __forceinline__ bf16x8 probs8(const f32x16& S, int t, float c, float m_run) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(S[8 * t + 2 * e], c, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(S[8 * t + 2 * e + 1], c, -m_run));
        w[e] = pack_bf16x2(p0, p1);
    }
    return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

// Row-sum contribution of one B operand: the rounded bf16 values (v_dot2 with
// ones), i.e. exactly the weights the product used.
__device__ __forceinline__ void rowsum8(const bf16x8& P, float& l_run) {
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    const uint4 w = __builtin_bit_cast(uint4, P);
    l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), ones, l_run, false);
    l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), ones, l_run, false);
    l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), ones, l_run, false);
    l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), ones, l_run, false);
}

// V^T operand for one MFMA step: 4 consecutive keys at byte address a + OFF and 4
// more 8 keys (SECOND bytes) later -- the two halves of the lane's 8 contraction
// slots -- transposed on read.
template <int OFF, int SECOND>
__device__ __forceinline__ bf16x8 vt_operand(uint32_t a) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(a + OFF));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(a + OFF + SECOND));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// O^T += V^T P^T for one 16-key MFMA step (KB, T) of a tile, for every query block:
// each V^T operand read from LDS feeds QB products. vb[dt]: this lane's V^T source
// address for d tile dt, first step, in the current V tile; step (KB, T) adds
// 32 KB + 16 T rows (a constant offset).
template <int HD, int NW, int QB, int KB, int T>
__device__ __forceinline__ void pv_step(const uint32_t (&vb)[Cfg<HD, NW>::NDT], const bf16x8 (&P)[QB][4],
                                        f32x16 (&O)[QB][Cfg<HD, NW>::NDT]) {
    using C = Cfg<HD, NW>;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
        const bf16x8 v = vt_operand<(32 * KB + 16 * T) * C::ROWB, 8 * C::ROWB>(vb[dt]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            O[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, P[qb][2 * KB + T], O[qb][dt], 0, 0, 0);
    }
}

template <int HD, int NW, int QB>
__device__ __forceinline__ void pv_tile(uint32_t vread, const uint32_t (&vaddr)[Cfg<HD, NW>::NDT],
                                        const bf16x8 (&P)[QB][4], f32x16 (&O)[QB][Cfg<HD, NW>::NDT]) {
    using C = Cfg<HD, NW>;
    uint32_t vb[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) vb[dt] = vaddr[dt] + vread;
    pv_step<HD, NW, QB, 0, 0>(vb, P, O);
    pv_step<HD, NW, QB, 0, 1>(vb, P, O);
    pv_step<HD, NW, QB, 1, 0>(vb, P, O);
    pv_step<HD, NW, QB, 1, 1>(vb, P, O);
}

// Per-block state threaded through the pipeline.
template <int HD, int NW, int QB>
struct Pipe {
    using C = Cfg<HD, NW>;
    i32x4 rk, rv;
    int wave, lane, g, len, qlen, ntiles;   // len: keys of the sequence; qlen: its queries
    uint32_t ldb, koff, voff;
    uint32_t kring, vring;      // LDS addresses of the K and V tile rings
    uint32_t kaddr[C::NKK];     // K operand addresses in ring slot 0 (ring base included)
    uint32_t vaddr[C::NDT];     // V^T operand addresses in ring slot 0
    bf16x8 qreg[QB][C::NKK];
    f32x16 O[QB][C::NDT];
    float m_run[QB], l_run[QB];
    float c;
};

// Running-max update for the tile held in S (before its probabilities are formed).
template <int HD, int NW, int QB>
__device__ __forceinline__ void max_update(Pipe<HD, NW, QB>& p, const f32x16 (&S)[QB][2]) {
    using C = Cfg<HD, NW>;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
        raise_max<C::NDT>(tile_max(S[qb][0], S[qb][1], p.c), p.O[qb], p.m_run[qb], p.l_run[qb]);
}

// bf16 probabilities P[qb][2kb + t] of the tile held in S (running max already
// raised for it).
template <int HD, int NW, int QB>
__device__ __forceinline__ void probs_tile(const Pipe<HD, NW, QB>& p, const f32x16 (&S)[QB][2],
                                           bf16x8 (&P)[QB][4]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int t = 0; t < 2; ++t) P[qb][2 * kb + t] = probs8(S[qb][kb], t, p.c, p.m_run[qb]);
}

template <int HD, int NW, int QB>
__device__ __forceinline__ void rowsum_tile(Pipe<HD, NW, QB>& p, const bf16x8 (&P)[QB][4]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) rowsum8(P[qb][i], p.l_run[qb]);
}

// One pipeline step for tile j (Sin = S(j) in registers with the running max
// already raised for it; K(j+1) and V(j) resident): stream K(j+ST) and V(j+ST-1)
// into their ring slots; P(j) on the vector ALU while the matrix cores compute
// S(j+1) = K(j+1) Q^T into Sout; O += V(j) P(j) while the vector ALU forms the
// row sums of P(j) and the max of S(j+1) (masked first when it is the last
// tile, LAST) -- so the rarely taken rescale branch comes after all of the
// step's products are issued and never splits them from the softmax work;
// finally wait for the tiles the next step needs and publish them with a
// barrier. Requires j+1 < ntiles. kslot / vslot: byte offsets of ring slots
// (j+1) % ST and j % ST; compile-time constants in the unrolled loop, where they
// fold into the LDS instructions' offset fields.
template <int HD, int NW, int QB, bool LAST>
__device__ __forceinline__ void pipe_step(Pipe<HD, NW, QB>& p, int j, const f32x16 (&Sin)[QB][2],
                                          f32x16 (&Sout)[QB][2], uint32_t kslot, uint32_t vslot,
                                          uint32_t kslot_next, uint32_t vslot_next) {
    using C = Cfg<HD, NW>;
    const int kn = j + C::ST, vn = j + C::ST - 1;   // tiles streamed in this step
    const bool issue_k = kn < p.ntiles, issue_v = vn < p.ntiles;
    if (issue_k)
        issue_any<HD, NW, false>(p.rk, p.kring + kslot_next, p.wave, p.lane, p.ldb, (uint32_t)kn * C::BK,
                                 (uint32_t)p.len, p.koff);
    if (issue_v)
        issue_any<HD, NW, true>(p.rv, p.vring + vslot_next, p.wave, p.lane, p.ldb, (uint32_t)vn * C::BK,
                                (uint32_t)p.len, p.voff);
    // the per-lane operand addresses, redefined here by an empty asm (no
    // instruction) at the head of the block that reads them: the slot offsets then
    // fold into the reads instead of every (address + offset) sum being hoisted out
    // of the loop into a register of its own
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) asm volatile("" : "+v"(p.kaddr[kk]));
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) asm volatile("" : "+v"(p.vaddr[dt]));
    bf16x8 P[QB][4];
    if constexpr (QB == 1 && NW == 4) {   // registers to spare: read all K operands first
        bf16x8 ka[2 * C::NKK];
        k_fetch<HD, NW>(kslot, p.kaddr, ka);
        probs_tile<HD, NW, QB>(p, Sin, P);
        s_mfma<HD, NW, QB>(ka, p.qreg, Sout);   // S(j+1): independent of the exps above
    } else {
        probs_tile<HD, NW, QB>(p, Sin, P);
        s_tile<HD, NW, QB>(kslot, p.kaddr, p.qreg, Sout);   // S(j+1): independent of the exps above
    }
    pv_tile<HD, NW, QB>(vslot, p.vaddr, P, p.O);
    rowsum_tile<HD, NW, QB>(p, P);
    if constexpr (LAST) mask_tile<QB>(Sout, p.g, (j + 1) * C::BK, p.len);
    float mxs[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mxs[qb] = tile_max(Sout[qb][0], Sout[qb][1], p.c);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) raise_max<C::NDT>(mxs[qb], p.O[qb], p.m_run[qb], p.l_run[qb]);
    // the next step reads K(j+2) and V(j+1): with a 2-deep ring they were issued in
    // this step, with a 3-deep ring in the previous one, so this step's own loads
    // (completing in issue order) may stay in flight
    if constexpr (C::ST == 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
        static_assert(C::LPW == 2, "3-deep ring wait counts assume two loads per stream per wave");
        if (issue_k)
            asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else if (issue_v)
            asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();   // everyone's loads have landed; all reads of tile j are done
}

// Step j of the unrolled loop: J = j mod 6 (a multiple of the ring depth and of
// the two score register sets) fixes the ring slots at compile time.
template <int HD, int NW, int QB, int J>
__device__ __forceinline__ void pipe_step_u(Pipe<HD, NW, QB>& p, int j, const f32x16 (&Sin)[QB][2],
                                            f32x16 (&Sout)[QB][2]) {
    using C = Cfg<HD, NW>;
    pipe_step<HD, NW, QB, false>(p, j, Sin, Sout, ((J + 1) % C::ST) * C::TILEB, (J % C::ST) * C::TILEB,
                                 ((J + C::ST) % C::ST) * C::TILEB, ((J + C::ST - 1) % C::ST) * C::TILEB);
}

// Step j with run-time ring slots, S(j) -> S(j+1) in place (the steps after the
// unrolled passes, and the last one, which masks).
template <int HD, int NW, int QB, bool LAST>
__device__ __forceinline__ void pipe_step_rt(Pipe<HD, NW, QB>& p, int j, f32x16 (&S)[QB][2]) {
    using C = Cfg<HD, NW>;
    const uint32_t ks = __builtin_amdgcn_readfirstlane(((j + 1) % C::ST) * C::TILEB);
    const uint32_t vs = __builtin_amdgcn_readfirstlane((j % C::ST) * C::TILEB);
    const uint32_t kn = __builtin_amdgcn_readfirstlane(((j + C::ST) % C::ST) * C::TILEB);
    const uint32_t vn = __builtin_amdgcn_readfirstlane(((j + C::ST - 1) % C::ST) * C::TILEB);
    f32x16 Sn[QB][2];
    pipe_step<HD, NW, QB, LAST>(p, j, S, Sn, ks, vs, kn, vn);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) { S[qb][0] = Sn[qb][0]; S[qb][1] = Sn[qb][1]; }
}

// Final tile (S = S(j) in registers, running max raised for it; V(j) at LDS
// address vread).
template <int HD, int NW, int QB>
__device__ __forceinline__ void pipe_last(Pipe<HD, NW, QB>& p, const f32x16 (&S)[QB][2], uint32_t vread) {
    bf16x8 P[QB][4];
    probs_tile<HD, NW, QB>(p, S, P);
    pv_tile<HD, NW, QB>(vread, p.vaddr, P, p.O);
    rowsum_tile<HD, NW, QB>(p, P);
}

// One work item: the BQ = 32 QB NW queries of query tile bw.qt of one (sequence,
// head) against all of the sequence's keys, through the block's K / V tile rings
// in LDS. QB = query blocks of 32 per wave. QB = 2 halves the LDS operand traffic
// per flop but needs about 450 registers, i.e. one wave per SIMD (VGPRs + AGPRs);
// QB = 1 runs two waves per SIMD. tid: the thread's index in the block.
template <int HD, int NW, int QB>
__device__ __forceinline__ void attn_item(const AttnArgs& a, const attn::BlockWork& bw,
                                          char (&kbuf)[Cfg<HD, NW>::ST][Cfg<HD, NW>::TILEB],
                                          char (&vbuf)[Cfg<HD, NW>::ST][Cfg<HD, NW>::TILEB], int tid,
                                          attn::SplitPartial* part = nullptr) {
    using C = Cfg<HD, NW>;
    constexpr int BQ = 32 * QB * NW;   // queries per block
    const int head = bw.head, qt = bw.qt, len = bw.len, klen = bw.klen;
    const int64_t s0 = bw.s0, k0 = bw.k0;
    const int q0 = qt * BQ;
    if (q0 >= len) return;
    if (klen == 0) {   // no keys: o = 0, lse = -inf (the empty sum)
        for (int i = tid; i < BQ; i += 64 * NW) {
            const int qi = q0 + i;
            if (qi >= len) break;
            const int64_t row = (s0 + qi) * a.heads + head;
            uint4* Og = reinterpret_cast<uint4*>(reinterpret_cast<__bf16*>(a.o) + row * HD);
#pragma unroll
            for (int c = 0; c < HD / 8; ++c) Og[c] = make_uint4(0, 0, 0, 0);
            if (a.lse != nullptr) a.lse[row] = -INFINITY;
        }
        return;
    }

    Pipe<HD, NW, QB> p;
    p.lane = tid & 63;
    p.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    p.g = p.lane >> 5;
    const int l32 = p.lane & 31;
    p.len = klen;
    p.qlen = len;
    p.ntiles = (klen + C::BK - 1) / C::BK;
    p.ldb = (uint32_t)a.heads * HD * 2;   // token stride in bytes
    const int64_t base = (s0 * a.heads + head) * (int64_t)HD;   // element offset of (s0, head, 0)
    const int64_t kbase = (k0 * a.heads + head) * (int64_t)HD;  // element offset of (k0, head, 0)
    // bytes of this sequence's queries / keys (< 2^31, host-checked)
    const uint32_t qspan = (uint32_t)len * p.ldb, kspan = (uint32_t)klen * p.ldb;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const __bf16*>(a.q) + base), (short)0, qspan, 0x00020000);
    p.rk = make_rsrc(reinterpret_cast<const __bf16*>(a.k) + kbase, kspan);
    p.rv = make_rsrc(reinterpret_cast<const __bf16*>(a.v) + kbase, kspan);

    // ---- per-lane, loop-invariant offsets
    {
        // direct loads: lane carries row RPB*wave + lane/CPR of each of its blocks
        const int lrow = C::RPB * p.wave + p.lane / C::CPR;
        const int pc = p.lane % C::CPR;
        p.koff = (uint32_t)lrow * p.ldb + (uint32_t)((pc ^ kswz<C::CPR>(lrow)) * 16);
        p.voff = (uint32_t)lrow * p.ldb + (uint32_t)((pc ^ vswz<C::CPR>(lrow)) * 16);
    }
    p.kring = lds_addr(kbuf[0]);
    p.vring = lds_addr(vbuf[0]);
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk)
        p.kaddr[kk] = p.kring + (uint32_t)(l32 * C::ROWB + (((2 * kk + p.g) ^ kswz<C::CPR>(l32)) * 16));
    {
        // V^T operand (A of O^T): 16-lane group hg = lane/16 covers d = 32dt + 16(hg%2) + i
        // (i = lane%16); its source lanes point at key row 4g + i/4 (+ step offsets),
        // 4 dims starting at 32dt + 16(hg%2) + 4(i%4).
        const int i16 = p.lane & 15, hg = p.lane >> 4;
        const int vrow = 4 * p.g + i16 / 4;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
            const int d0 = 32 * dt + 16 * (hg & 1) + 4 * (i16 & 3);
            p.vaddr[dt] = p.vring + (uint32_t)(vrow * C::ROWB + ((d0 / 8) ^ vswz<C::CPR>(vrow)) * 16 + (d0 % 8) * 2);
        }
    }

    // ---- Q (B operand of S^T = K Q^T): block qb of this wave, lane holds query
    // q0 + 32(QB wave + qb) + l32, d = 16kk + 8g .. +7
    int my_q[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        my_q[qb] = q0 + 32 * (QB * p.wave + qb) + l32;
        const uint32_t qrow = (uint32_t)(my_q[qb] < len ? my_q[qb] : len - 1);
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk)
            p.qreg[qb][kk] = __builtin_bit_cast(bf16x8, bload(rq, qrow * p.ldb + (2 * kk + p.g) * 16, 0));
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) p.O[qb][dt][r] = 0.f;
        p.m_run[qb] = -INFINITY;   // running max in the scaled log2 domain
        p.l_run[qb] = 0.f;         // this lane's partial row sum (its 16 keys per tile)
    }
    p.c = a.scale_log2;

    // ---- prologue: K(0), V(0), K(1) resident; S(0); then the loads a step -1
    // would have issued (K(ST-1), V(ST-2)) for a 3-deep ring
    issue_any<HD, NW, false>(p.rk, p.kring, p.wave, p.lane, p.ldb, 0, (uint32_t)klen, p.koff);
    issue_any<HD, NW, true>(p.rv, p.vring, p.wave, p.lane, p.ldb, 0, (uint32_t)klen, p.voff);
    if (p.ntiles > 1)
        issue_any<HD, NW, false>(p.rk, p.kring + C::TILEB, p.wave, p.lane, p.ldb, C::BK, (uint32_t)klen, p.koff);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    f32x16 S[QB][2], Sb[QB][2];
    {
        bf16x8 ka[2 * C::NKK];
        k_fetch<HD, NW>(0, p.kaddr, ka);
        s_mfma<HD, NW, QB>(ka, p.qreg, S);
    }
    if (p.ntiles == 1) mask_tile<QB>(S, p.g, 0, klen);
    max_update<HD, NW, QB>(p, S);
    // every wave's reads of K(0) are done before step 0 streams into its slot
    __syncthreads();
    if constexpr (C::ST == 3) {
        if (p.ntiles > 2)
            issue_any<HD, NW, false>(p.rk, p.kring + 2 * C::TILEB, p.wave, p.lane, p.ldb, 2 * C::BK,
                                     (uint32_t)klen, p.koff);
        if (p.ntiles > 1)
            issue_any<HD, NW, true>(p.rv, p.vring + C::TILEB, p.wave, p.lane, p.ldb, C::BK, (uint32_t)klen,
                                    p.voff);
    }

    // ---- steady state: step j reads K(j+1), V(j) from ring slots (j+1) % ST, j % ST;
    // passes of six steps with compile-time slots (S(j) back in S after each
    // pass), the remaining steps with run-time slots, the masked last step
    int j = 0;
    for (; j + 6 <= p.ntiles - 2; j += 6) {
        pipe_step_u<HD, NW, QB, 0>(p, j, S, Sb);
        pipe_step_u<HD, NW, QB, 1>(p, j + 1, Sb, S);
        pipe_step_u<HD, NW, QB, 2>(p, j + 2, S, Sb);
        pipe_step_u<HD, NW, QB, 3>(p, j + 3, Sb, S);
        pipe_step_u<HD, NW, QB, 4>(p, j + 4, S, Sb);
        pipe_step_u<HD, NW, QB, 5>(p, j + 5, Sb, S);
    }
    for (; j < p.ntiles - 2; ++j) pipe_step_rt<HD, NW, QB, false>(p, j, S);
    if (p.ntiles > 1) pipe_step_rt<HD, NW, QB, true>(p, p.ntiles - 2, S);
    pipe_last<HD, NW, QB>(p, S, (uint32_t)((p.ntiles - 1) % C::ST) * C::TILEB);

    if (part != nullptr) {   // a piece of a split item: the unnormalised partial, m and l
        if constexpr (HD == attn::kSplitD && 32 * QB * NW == attn::kSplitQ) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int ql = 32 * (QB * p.wave + qb) + l32;   // query within the item
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg)
                        *reinterpret_cast<float4*>(&part->o[ql][dt * 32 + 8 * rg + 4 * p.g]) =
                            make_float4(p.O[qb][dt][4 * rg], p.O[qb][dt][4 * rg + 1], p.O[qb][dt][4 * rg + 2],
                                        p.O[qb][dt][4 * rg + 3]);
                const float l = pair_sum(p.l_run[qb]);
                if (p.g == 0) {
                    part->m[ql] = p.m_run[qb];
                    part->l[ql] = l;
                }
            }
        }
        return;
    }
    // ---- normalise and store: lane holds query my_q[qb], d = 32dt + 8(r/4) + 4g + r%4;
    // lanes l and l^32 summed disjoint keys of the same query.
    // The sequence's rows of o (and lse) for this head, as range-checked buffers:
    // rows past its end store to kDropOffset (no lane-divergent branch)
    const uint32_t ostride = (uint32_t)a.heads * HD * 2;   // bytes per token row of o
    const __amdgpu_buffer_rsrc_t ro =
        out_rsrc(reinterpret_cast<__bf16*>(a.o) + (s0 * a.heads + head) * HD, (uint32_t)len * ostride);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = pair_sum(p.l_run[qb]);
        const float inv = 1.0f / l;
        const bool live = my_q[qb] < len;
        const uint32_t rowoff = (uint32_t)my_q[qb] * ostride;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                uint2 wv;
                wv.x = pack_bf16x2(p.O[qb][dt][4 * rg + 0] * inv, p.O[qb][dt][4 * rg + 1] * inv);
                wv.y = pack_bf16x2(p.O[qb][dt][4 * rg + 2] * inv, p.O[qb][dt][4 * rg + 3] * inv);
                bstore8(ro, wv, live ? rowoff + (uint32_t)(dt * 32 + 8 * rg + 4 * p.g) * 2 : kDropOffset);
            }
        }
        // ln sum_keys exp(s) = ln 2 * (m + log2 l): scores were exponentiated as
        // exp2(s * log2(e) - m)
        if (a.lse != nullptr) {
            const __amdgpu_buffer_rsrc_t rl = out_rsrc(a.lse + s0 * a.heads + head, (uint32_t)len * a.heads * 4);
            bstore4(rl, (p.m_run[qb] + __log2f(l)) * 0.69314718055994531f,
                    live && p.g == 0 ? (uint32_t)my_q[qb] * a.heads * 4 : kDropOffset);
        }
    }
}

// One block per work item (the grid covers num_seqs x the longest sequence's
// query tiles; blocks past the real items exit).
template <int HD, int NW, int QB>
__global__ __launch_bounds__(64 * NW, (QB == 1 && NW == 4) ? 2 : 1) void attn_bf16_kernel(AttnArgs a, int nqt) {
    using C = Cfg<HD, NW>;
    __shared__ __attribute__((aligned(1024))) char kbuf[C::ST][C::TILEB];
    __shared__ __attribute__((aligned(1024))) char vbuf[C::ST][C::TILEB];
    attn::BlockWork bw;
    if (!attn::decode_block(a.cu_seqlens, a.cu_seqlens_k, a.num_seqs, a.max_seqlen, a.max_seqlen_k, a.heads, nqt,
                            32 * QB * NW, bw))
        return;
    attn_item<HD, NW, QB>(a, bw, kbuf, vbuf, thread_index());
}

// ---- Persistent launch (work queues and tail splitting: dit_attn_common.hpp)
struct AttnLaunch {
    AttnArgs a;
    int nqt, nblocks;
    uint32_t* queue;              // this launch's queue slot
    attn::SplitPartial* split;    // partial slots, or null: no tail splitting
    uint32_t* split_cnt;          // completion counters of the split items
};

// Merge of the s partials of one split item (slots slot0 .. slot0 + s - 1) into
// its output rows: per query, M = max m_p, L = sum l_p 2^(m_p - M),
// o = sum 2^(m_p - M) o_p / L, lse = ln 2 (M + log2 L); no keys at all (M = -inf)
// gives o = 0, lse = -inf. Two threads per query, 64 dims each.
template <int NW>
__device__ __forceinline__ void merge_pieces(const AttnArgs& a, const attn::BlockWork& bw,
                                             const attn::SplitPartial* parts, int s, int tid) {
    constexpr int D = attn::kSplitD;
    for (int t = tid; t < 2 * attn::kSplitQ; t += 64 * NW) {
        const int ql = t >> 1, h = t & 1;
        const int qi = bw.qt * attn::kSplitQ + ql;
        if (qi >= bw.len) continue;
        float M = -INFINITY;
        for (int pc = 0; pc < s; ++pc) M = __builtin_fmaxf(M, parts[pc].m[ql]);
        const int64_t row = (bw.s0 + qi) * a.heads + bw.head;
        uint4* Og = reinterpret_cast<uint4*>(reinterpret_cast<__bf16*>(a.o) + row * D) + h * (D / 16);
        if (M == -INFINITY) {
#pragma unroll
            for (int c = 0; c < D / 16; ++c) Og[c] = make_uint4(0, 0, 0, 0);
            if (a.lse != nullptr && h == 0) a.lse[row] = -INFINITY;
            continue;
        }
        float acc[D / 2];
#pragma unroll
        for (int i = 0; i < D / 2; ++i) acc[i] = 0.f;
        float L = 0.f;
        for (int pc = 0; pc < s; ++pc) {
            const float w = __builtin_amdgcn_exp2f(parts[pc].m[ql] - M);
            L = fmaf(w, parts[pc].l[ql], L);
            const float4* src = reinterpret_cast<const float4*>(&parts[pc].o[ql][h * (D / 2)]);
#pragma unroll
            for (int i = 0; i < D / 8; ++i) {
                const float4 v = src[i];
                acc[4 * i] = fmaf(w, v.x, acc[4 * i]);
                acc[4 * i + 1] = fmaf(w, v.y, acc[4 * i + 1]);
                acc[4 * i + 2] = fmaf(w, v.z, acc[4 * i + 2]);
                acc[4 * i + 3] = fmaf(w, v.w, acc[4 * i + 3]);
            }
        }
        const float inv = 1.0f / L;
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
            Og[c] = make_uint4(pack_bf16x2(acc[8 * c] * inv, acc[8 * c + 1] * inv),
                               pack_bf16x2(acc[8 * c + 2] * inv, acc[8 * c + 3] * inv),
                               pack_bf16x2(acc[8 * c + 4] * inv, acc[8 * c + 5] * inv),
                               pack_bf16x2(acc[8 * c + 6] * inv, acc[8 * c + 7] * inv));
        if (a.lse != nullptr && h == 0) a.lse[row] = (M + __log2f(L)) * 0.69314718055994531f;
    }
}

// Piece p of s of a split item covers key tiles p nt / s .. (p + 1) nt / s - 1
// (possibly none): narrow the item to those keys. Returns false for an empty
// piece, whose partial (m = -inf, l = 0) is written here.
template <int NW, int BK>
__device__ __forceinline__ bool piece_keys(attn::BlockWork& bw, const attn::Unit& un, attn::SplitPartial* part,
                                           int tid) {
    const int nt = (bw.klen + BK - 1) / BK;
    const int t0 = un.piece * nt / un.pieces, t1 = (un.piece + 1) * nt / un.pieces;
    const int k_lo = t0 * BK, k_hi = t1 * BK < bw.klen ? t1 * BK : bw.klen;
    if (k_hi > k_lo) {
        bw.k0 += k_lo;
        bw.klen = k_hi - k_lo;
        return true;
    }
    for (int q = tid; q < attn::kSplitQ; q += 64 * NW) {
        part->m[q] = -INFINITY;
        part->l[q] = 0.f;
    }
    return false;
}

// After a piece's partial is stored: if it is the item's last piece to finish,
// merge. The pieces of an item all run on one XCD (one L2): each wave waits for
// its partial stores to be acknowledged (by the L2) before the barrier, thread
// 0 then increments the item's counter; the last piece reads the partials after
// seeing the count (its L1 holds none of them: each slot is read once per
// launch, and the L1 is invalidated at every kernel start). The last piece
// clears the counter.
template <int NW>
__device__ __forceinline__ void piece_done(const AttnArgs& a, const attn::BlockWork& bw, const attn::Unit& un,
                                           attn::SplitPartial* split, uint32_t* split_cnt, int tid, int& s_flag) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // every wave's partial stores have completed
    if (tid == 0) {
        const uint32_t done = atomicAdd(&split_cnt[un.counter], 1u);
        s_flag = done == (uint32_t)(un.pieces - 1);
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(s_flag)) {
        merge_pieces<NW>(a, bw, split + (un.slot - un.piece), un.pieces, tid);
        if (tid == 0) __hip_atomic_store(&split_cnt[un.counter], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The kernel's argument block, as a constant-memory pointer redefined at each
// use (see the persistent loop), and the attention arguments read from it.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* kernargs() {
    uint64_t p = reinterpret_cast<uint64_t>(__builtin_amdgcn_kernarg_segment_ptr());
    asm volatile("" : "+s"(p));
    p = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p >> 32)) << 32) |
        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    return (const __attribute__((address_space(4))) T*)p;
}
__device__ __forceinline__ AttnArgs load_args(const __attribute__((address_space(4))) AttnLaunch* lp) {
    AttnArgs a;
    a.o = lp->a.o; a.q = lp->a.q; a.k = lp->a.k; a.v = lp->a.v;
    a.tokens = lp->a.tokens; a.heads = lp->a.heads; a.head_dim = lp->a.head_dim;
    a.cu_seqlens = lp->a.cu_seqlens; a.num_seqs = lp->a.num_seqs; a.max_seqlen = lp->a.max_seqlen;
    a.scale_log2 = lp->a.scale_log2; a.scale = lp->a.scale;
    a.cu_seqlens_k = lp->a.cu_seqlens_k; a.max_seqlen_k = lp->a.max_seqlen_k; a.lse = lp->a.lse;
    return a;
}

template <int HD, int NW, int QB>
__global__ __launch_bounds__(64 * NW, (QB == 1 && NW == 4) ? 2 : 1) void attn_bf16_persistent(AttnLaunch L) {
    using C = Cfg<HD, NW>;
    constexpr int BQ = 32 * QB * NW;
    __shared__ __attribute__((aligned(1024))) char kbuf[C::ST][C::TILEB];
    __shared__ __attribute__((aligned(1024))) char vbuf[C::ST][C::TILEB];
    __shared__ int s_item, s_unit, s_flag;
    typedef __attribute__((address_space(4))) const AttnLaunch* kernarg_ptr;   // constant memory: scalar loads

    const int total = attn::items_total(L.a.cu_seqlens, L.a.num_seqs, L.a.heads, L.nqt, BQ);
    for (;;) {
        // The launch arguments, the item count and the thread index are redefined
        // here for every item (empty asm, no instruction; the pointer is read back
        // through readfirstlane, since asm outputs count as divergent): otherwise
        // they and everything derived from them are computed once and held in
        // registers through every key loop, where the scalar registers are already
        // all in use. For the same reason nothing about the unit is kept across
        // the item: a split piece's completion re-derives it from the LDS copy.
        const kernarg_ptr lp = kernargs<AttnLaunch>();
        int tt = total, tid = thread_index();
        asm volatile("" : "+s"(tt), "+v"(tid));
        tt = __builtin_amdgcn_readfirstlane(tt);
        // blocks per XCD (the dispatcher deals blocks round-robin), and whether this
        // launch splits its tail (partial slots given, 256 queries x 128 dims per item)
        const int bpx = lp->nblocks / 8;
        const bool split =
            lp->split != nullptr && lp->nblocks % 8 == 0 && HD == attn::kSplitD && BQ == attn::kSplitQ;
        AttnArgs a = load_args(lp);

        __syncthreads();   // the previous item's LDS reads, and every wave's read of s_item, are done
        if (tid == 0) {
            int v, u;
            attn::next_unit(lp->queue, tt, bpx, split, attn::xcc_id(), v, u);
            s_item = v;
            s_unit = u;
        }
        __syncthreads();
        const int v = __builtin_amdgcn_readfirstlane(s_item);
        if (v < 0) break;
        {
            const attn::Unit un = attn::decode_unit(tt, bpx, split, v, __builtin_amdgcn_readfirstlane(s_unit));
            attn::BlockWork bw;
            attn::decode_item(un.item, a.cu_seqlens, a.cu_seqlens_k, a.num_seqs, a.max_seqlen, a.max_seqlen_k,
                              lp->nqt, BQ, tt, a.heads, bw);
            // a piece of a split item: its keys only, its partial into its slot
            attn::SplitPartial* part = un.pieces > 1 ? lp->split + un.slot : nullptr;
            const bool keys = part == nullptr || piece_keys<NW, Cfg<HD, NW>::BK>(bw, un, part, tid);
            if (keys) attn_item<HD, NW, QB>(a, bw, kbuf, vbuf, tid, part);
        }
        {
            const kernarg_ptr lq = kernargs<AttnLaunch>();
            int t2 = total, tid2 = thread_index();
            asm volatile("" : "+s"(t2), "+v"(tid2));
            t2 = __builtin_amdgcn_readfirstlane(t2);
            const bool split2 =
                lq->split != nullptr && lq->nblocks % 8 == 0 && HD == attn::kSplitD && BQ == attn::kSplitQ;
            const attn::Unit un = attn::decode_unit(t2, lq->nblocks / 8, split2, __builtin_amdgcn_readfirstlane(s_item),
                                                    __builtin_amdgcn_readfirstlane(s_unit));
            if (un.pieces > 1) {
                const AttnArgs a2 = load_args(lq);
                attn::BlockWork whole;
                attn::decode_item(un.item, a2.cu_seqlens, a2.cu_seqlens_k, a2.num_seqs, a2.max_seqlen,
                                  a2.max_seqlen_k, lq->nqt, BQ, t2, a2.heads, whole);
                piece_done<NW>(a2, whole, un, lq->split, lq->split_cnt, tid2, s_flag);
            }
        }
    }
    // the last block to finish clears this slot's counters for its next launch
    if (thread_index() == 0) {
        attn::queue_finish(L.queue, L.nblocks);
    }
}

// ---- Scratch of the allocation-free entry point (dit_attn3d_noalloc): one
// persistent-launch queue slot -- the 8 XCD counters and the finished-block
// count, a 64-byte line each, 576 bytes -- in a file-scope device array (one copy
// per device, kept until the process ends). The name is a host-side stand-in:
// host code uses only the per-device address that hipGetSymbolAddress returns.
// The counters count work items, so no input needs more than this. Every
// allocation-free call on a device shares the slot: calls that overlap on one
// device race (their blocks would draw each other's items).
constexpr int kScratchWords = 9 * attn::kQWords;
static __device__ __align__(256) uint32_t scratch[kScratchWords];

struct ScratchDevice {
    std::mutex mu;
    bool init = false;
    uint32_t* ptr = nullptr;
};
ScratchDevice g_scratch_dev[64];

// The current device's address of `scratch`, resolved on its first use.
hipError_t scratch_address(uint32_t*& out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    ScratchDevice& d = g_scratch_dev[dev];
    std::lock_guard<std::mutex> g(d.mu);
    if (!d.init) {
        e = hipGetSymbolAddress(reinterpret_cast<void**>(&d.ptr), HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        d.init = true;
    }
    out = d.ptr;
    return hipSuccess;
}

// Zeroes the queue slot before a launch (a kernel, not a memset node, so a
// captured graph clears it on every replay too).
__global__ void scratch_clear_kernel(uint32_t* q, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) q[i] = 0u;
}

// noalloc: persistent launches take their queue slot from `scratch` (no launch
// tracking, no split tail); otherwise from the tracked slots of
// dit_attn_common.hpp, with the split tail when its scratch is free.
template <int HD, int NW, int QB>
hipError_t launch_t(const AttnArgs& a, hipStream_t s, bool noalloc) {
    constexpr int BQ = 32 * QB * NW;
    const int nqt = (a.max_seqlen + BQ - 1) / BQ;
    const int64_t grid = (int64_t)nqt * a.heads * a.num_seqs;   // >= the number of items
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    int cus = 0;
    hipError_t e = attn::device_cus(cus);
    if (e != hipSuccess) return e;
    const int64_t resident = (int64_t)cus * ((QB == 1 && NW == 4) ? 2 : 1);   // blocks the chip holds at once
    auto per_item = [&]() -> hipError_t {
        hipLaunchKernelGGL((attn_bf16_kernel<HD, NW, QB>), dim3((unsigned)grid), dim3(64 * NW), 0, s, a, nqt);
        return hipGetLastError();
    };
    if (use_persistent(grid, resident, cus)) {
        // enough items per resident block for the queues (and the split tail) to
        // even out the XCDs
        if (noalloc) {
            uint32_t* q = nullptr;
            e = scratch_address(q);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(scratch_clear_kernel, dim3(1), dim3(64), 0, s, q, kScratchWords);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            const AttnLaunch L{a, nqt, (int)resident, q, nullptr, nullptr};
            hipLaunchKernelGGL((attn_bf16_persistent<HD, NW, QB>), dim3((unsigned)resident), dim3(64 * NW), 0, s, L);
            return hipGetLastError();
        }
        return attn::persistent_launch(
            s,
            [&](uint32_t* queue, attn::SplitPartial* split, uint32_t* split_cnt) -> hipError_t {
                const AttnLaunch L{a, nqt, (int)resident, queue, split, split_cnt};
                hipLaunchKernelGGL((attn_bf16_persistent<HD, NW, QB>), dim3((unsigned)resident), dim3(64 * NW), 0,
                                   s, L);
                return hipGetLastError();
            },
            per_item);
    }
    return per_item();
}

}  // namespace

hipError_t launch_attn3d_bf16(const AttnArgs& a, hipStream_t s) {
    if (a.head_dim == 64) return launch_t<64, 4, 1>(a, s, false);
    return launch_t<128, 8, 1>(a, s, false);
}

hipError_t launch_attn3d_bf16_noalloc(const AttnArgs& a, hipStream_t s) {
    if (a.head_dim == 64) return launch_t<64, 4, 1>(a, s, true);
    return launch_t<128, 8, 1>(a, s, true);
}

}  // namespace dit
