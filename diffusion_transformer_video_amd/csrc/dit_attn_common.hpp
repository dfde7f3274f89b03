// Pieces shared by the gfx950 attention kernels (bf16 and fp8): lane-pair
// reductions over the two halves of a wave, buffer loads and range-checked
// stores, the direct HBM -> LDS load, the numbering of work items (query tiles)
// and their XCD-aware dealing to blocks, and the per-XCD work queues of the
// persistent launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace dit {
namespace attn {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

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

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource (raw, 32-bit range checked) for `bytes` bytes at `p`.
__device__ __forceinline__ i32x4 make_rsrc(const void* p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const i32x4 r = {(int)(uint32_t)a, (int)(uint32_t)((a >> 32) & 0xffffu), (int)bytes, 0x00020000};
    return r;
}

// One wave-wide 16-byte-per-lane load HBM -> LDS: lane L's 16 bytes land at
// lds_addr + 16 L. Issued from inline asm so that the compiler does not treat
// the pending load as a possible writer of the LDS tiles being read meanwhile
// (it would then wait for it before every LDS read); completion is waited for
// explicitly (vmcnt) before the barrier that publishes the tile. M0 is saved and
// restored around the instruction. The asm has no register outputs.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(lds_ptr_t)(const_cast<void*>(p));   // LDS byte address
}

// Stores without a lane-divergent branch: a raw buffer store drops every access
// at or past the resource's record count, so a lane whose row lies past the
// sequence's end stores to kDropOffset instead of branching around the store. (A
// divergent branch around the output stores lets the compiler sink the last
// matrix-core products into it, where a product reads its operands from the
// active lanes only.)
constexpr uint32_t kDropOffset = 0xFFFFFFF0u;   // past any record count used with it

__device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t r, uint2 v, uint32_t off) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 d = {v.x, v.y};
    __builtin_amdgcn_raw_buffer_store_b64(d, r, (int)off, 0, 0);
}

__device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, float v, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, 0);
}

// raw buffer resource over `bytes` bytes at p (byte offsets, range-checked)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)bytes, 0x00020000);
}

// Thread and block indices straight from the hardware registers. (In kernels
// this large, the library functions behind threadIdx / blockIdx / gridDim are
// not inlined: each use became a call, which clobbers registers and costs
// spills.)
__device__ __forceinline__ int thread_index() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ unsigned block_index() { return __builtin_amdgcn_workgroup_id_x(); }

// Work item of one block: query tile qt of sequence seq, head head; the
// sequence's queries start at row s0 (len of them), its keys at row k0 (klen).
struct BlockWork {
    int head, seq, qt;
    int64_t s0, k0;
    int len, klen;
};

// Work items are numbered head-major over the exact query tiles (BQ queries) of
// every sequence (longest sequence first within a head). cu_q NULL: dense
// sequences of max_q queries. Returns the number of items (wave-uniform).
__device__ __forceinline__ int items_total(const int32_t* cu_q, int num_seqs, int heads, int nqt, int BQ) {
    if (cu_q == nullptr) return nqt * heads * num_seqs;   // the one-block-per-item launch's grid
    int total = 0;
    for (int s = 0; s < num_seqs; ++s) {
        const int ls = __builtin_amdgcn_readfirstlane(cu_q[s + 1] - cu_q[s]);
        total += (ls + BQ - 1) / BQ;
    }
    return total * heads;
}

// The items dealt to XCD x: [start, start + len). The dispatcher deals blocks
// round-robin over the 8 XCDs, so an XCD receives every 8th block; giving it a
// contiguous range of items hands it whole heads with all their sequences
// (balanced), and its concurrent blocks share one head's K/V in its L2.
__device__ __forceinline__ void xcd_slice(int total, int x, int& start, int& len) {
    const int per = total / 8, rem = total % 8;
    len = per + (x < rem ? 1 : 0);
    start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
}

// Item w -> (head, sequence, query tile) and the sequence's rows. Every decoded
// value is wave-uniform.
__device__ __forceinline__ void decode_item(int w, const int32_t* cu_q, const int32_t* cu_k, int num_seqs, int max_q,
                                            int max_k, int nqt, int BQ, int total, int heads, BlockWork& bw) {
    int seq, qt, head;
    int64_t s0, k0;   // first query row / first key row of the sequence
    int len, klen;    // its queries / keys
    if (cu_q == nullptr) {
        const int per_head = nqt * num_seqs;
        head = __builtin_amdgcn_readfirstlane(w / per_head);
        const int r = w - head * per_head;
        seq = __builtin_amdgcn_readfirstlane(r / nqt);
        qt = __builtin_amdgcn_readfirstlane(r - seq * nqt);
        s0 = (int64_t)seq * max_q;
        len = max_q;
        k0 = (int64_t)seq * max_k;
        klen = max_k;
    } else {
        const int per_head = total / heads;
        head = __builtin_amdgcn_readfirstlane(w / per_head);
        int r = __builtin_amdgcn_readfirstlane(w - head * per_head);
        // walk the sequences longest first (by queries; ties: lower index first);
        // num_seqs is small, so the O(n^2) rank walk is a handful of scalar steps
        seq = -1;
        qt = 0;
        int prev_len = 0x7fffffff, prev_idx = -1;
        for (int k = 0; k < num_seqs && seq < 0; ++k) {
            // next sequence in (length desc, index asc) order after (prev_len, prev_idx)
            int best = -1, best_len = -1;
            for (int s = 0; s < num_seqs; ++s) {
                const int ls = __builtin_amdgcn_readfirstlane(cu_q[s + 1] - cu_q[s]);
                const bool after = num_seqs > 32 ? s > prev_idx   // many sequences: index order
                                                   : ls < prev_len || (ls == prev_len && s > prev_idx);
                if (after && (num_seqs > 32 ? best < 0 : ls > best_len)) { best = s; best_len = ls; }
            }
            const int nt = (best_len + BQ - 1) / BQ;
            if (r < nt) { seq = best; qt = r; } else { r -= nt; prev_len = best_len; prev_idx = best; }
        }
        seq = __builtin_amdgcn_readfirstlane(seq);
        qt = __builtin_amdgcn_readfirstlane(qt);
        const int c0 = __builtin_amdgcn_readfirstlane(cu_q[seq]);
        const int c1 = __builtin_amdgcn_readfirstlane(cu_q[seq + 1]);
        s0 = c0;
        len = c1 - c0;
        const int d0 = __builtin_amdgcn_readfirstlane(cu_k[seq]);
        const int d1 = __builtin_amdgcn_readfirstlane(cu_k[seq + 1]);
        k0 = d0;
        klen = d1 - d0;
    }
    bw.head = head;
    bw.seq = seq;
    bw.qt = qt;
    bw.s0 = s0;
    bw.k0 = k0;
    bw.len = len;
    bw.klen = klen;
}

// One block per item: block b -> item, remapped so that consecutive items land on
// the same XCD (xcd_slice). Blocks past the real total (the grid is sized for
// num_seqs x the longest sequence) are dealt last and get false.
__device__ __forceinline__ bool decode_block(const int32_t* cu_q, const int32_t* cu_k, int num_seqs, int max_q,
                                             int max_k, int heads, int nqt, int BQ, BlockWork& w) {
    const int total = items_total(cu_q, num_seqs, heads, nqt, BQ);
    const int b = (int)block_index();
    if (b >= total) return false;
    int start, len;
    xcd_slice(total, b % 8, start, len);
    decode_item(start + b / 8, cu_q, cu_k, num_seqs, max_q, max_k, nqt, BQ, total, heads, w);
    return true;
}

// ---- Persistent launches: one block per resident slot (CU), looping over items.
// The XCDs of one chip run at different clocks under this load (their blocks'
// key loops differed by up to 10% within one launch), so a fixed 1/8 of the items
// per XCD leaves the fast XCDs idle at the end. In a persistent launch every XCD
// draws items from its own queue -- its xcd_slice range, in order, so that its
// concurrent blocks still share a head's K/V in its L2 -- and, once that is
// empty, from the other XCDs' queues. A queue is an item counter in device memory
// (device-scope atomics); the last block to finish clears the counters for the
// next launch that uses the same slot. Launches rotate over kQueueSlots slots, so
// concurrently running launches (other streams) use different counters as long
// as fewer than kQueueSlots of one kernel file are in flight on one device. The
// counters are per translation unit (anonymous namespace): each attention kernel
// file has its own.
constexpr int kQueueSlots = 64;
constexpr int kQWords = 16;   // one 64-byte line per counter

namespace {

__device__ uint32_t g_attn_queue[kQueueSlots][9 * kQWords];   // 8 XCD queues, then the finished-block count

// Per device: compute units, the counters' device address, the next slot.
struct QueueDevice {
    std::atomic<int> cus{0};
    std::atomic<uint32_t*> queue{nullptr};
    std::atomic<uint32_t> next_slot{0};
};
QueueDevice g_queue_dev[64];

// Host: the current device's compute-unit count and, when want_slot, a queue
// slot for one launch.
inline hipError_t queue_launch_info(int& cus, uint32_t*& queue_slot, bool want_slot) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    QueueDevice& d = g_queue_dev[dev];
    int n = d.cus.load(std::memory_order_relaxed);
    uint32_t* q = d.queue.load(std::memory_order_relaxed);
    if (n == 0 || q == nullptr) {
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        // the array's device address on this device (its name in host code is not it)
        e = hipGetSymbolAddress(reinterpret_cast<void**>(&q), HIP_SYMBOL(g_attn_queue));
        if (e != hipSuccess) return e;
        d.cus.store(n, std::memory_order_relaxed);
        d.queue.store(q, std::memory_order_relaxed);
    }
    cus = n;
    queue_slot = want_slot
                     ? q + (size_t)(d.next_slot.fetch_add(1, std::memory_order_relaxed) % kQueueSlots) * 9 * kQWords
                     : nullptr;
    return hipSuccess;
}

}  // namespace

// The XCD this wave runs on (HW_REG_XCC_ID).
__device__ __forceinline__ int xcc_id() {
    return (int)(__builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (31 << 11)) & 7);
}

// The next item for a block on XCD x: its own queue first, then the others in
// turn; -1 when every queue is empty. Counters may run past their range
// (harmless: they are cleared at the end of the launch).
__device__ __forceinline__ int next_item(uint32_t* q, int total, int x) {
    for (int t = 0; t < 8; ++t) {
        const int v = (x + t) & 7;
        int start, len;
        xcd_slice(total, v, start, len);
        if (len == 0) continue;
        const uint32_t i = atomicAdd(&q[v * kQWords], 1u);
        if (i < (uint32_t)len) return start + (int)i;
    }
    return -1;
}

// Called once per block (one thread) after its last item: the last block of the
// launch clears the slot's counters.
__device__ __forceinline__ void queue_finish(uint32_t* q, int nblocks) {
    __threadfence();
    if (atomicAdd(&q[8 * kQWords], 1u) == (uint32_t)(nblocks - 1))
        for (int i = 0; i < 9; ++i) __hip_atomic_store(&q[i * kQWords], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace attn
}  // namespace dit
