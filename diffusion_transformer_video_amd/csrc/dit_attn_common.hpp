// Pieces shared by the gfx950 attention kernels (bf16 and fp8): lane-pair
// reductions over the two halves of a wave, buffer loads and range-checked
// stores, the direct HBM -> LDS load, the numbering of work items (query tiles)
// and their XCD-aware dealing to blocks, and the per-XCD work queues of the
// persistent launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

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
__host__ __device__ __forceinline__ void xcd_slice(int total, int x, int& start, int& len) {
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

#ifdef DIT_ATTN_PERSISTENT   // the bf16 attention file only (it alone holds the device state below)
// ---- Persistent launches: one block per resident slot (CU), looping over items.
// The XCDs of one chip run at different clocks under this load (their blocks'
// key loops differed by up to 10% within one launch), so a fixed 1/8 of the items
// per XCD leaves the fast XCDs idle at the end. In a persistent launch every XCD
// draws work units from its own queue -- its xcd_slice range, in order, so that
// its concurrent blocks still share a head's K/V in its L2 -- and, once that is
// empty, from the other XCDs' queues. A queue is a unit counter in device memory
// (device-scope atomics); the last block to finish clears the counters for the
// next launch that uses the same slot.
//
// Tail splitting: the last T items of each XCD's range (the items of its last,
// partly filled round; a whole round when the range divides evenly) are split
// along the keys into s pieces each (split_plan), so the launch's last round
// runs pieces of 1/s of an item rather than whole items. A piece writes its
// partial result (unnormalised float32 o, running max m and row sum l per query)
// to a scratch slot; the last piece of an item to finish (a counter per split
// item) merges the s partials with the log-sum-exp rule and writes the item's
// output. Pieces are only taken from their own XCD's queue (other XCDs steal
// full items only), so a split item's pieces, their partials and the merge
// share one L2: a piece publishes its partial by waiting for its stores before
// its counter increment, with no L2 write-back or invalidation.
//
// Device state (file-scope device arrays, resolved per device with
// hipGetSymbolAddress; nothing is allocated at call time): kQueueSlots queue
// slots and one split scratch area. The host hands a slot to a launch only when
// the slot's previous launch was on the same stream (stream order) or has
// completed (an event recorded after it), and likewise the split scratch; a
// launch that finds no free slot, or runs under stream capture, takes the
// one-block-per-item form, which keeps no device state. The counters are per
// translation unit (anonymous namespace): each attention kernel file has its own.
constexpr int kQueueSlots = 64;
constexpr int kQWords = 16;      // one 64-byte line per counter
constexpr int kSplitC = 32;      // blocks per XCD the split plan is sized for (256 CUs)
constexpr int kSplitMaxS = 16;   // at most this many pieces per split item
constexpr int kSplitPieces = 8 * 2 * kSplitC;   // partial slots: T s <= 2 C per XCD
constexpr int kSplitQ = 256;     // queries per work item (the split path's block)
constexpr int kSplitD = 128;     // head dim of the split path
struct SplitPartial {            // one piece's partial result for its 256 queries
    float o[kSplitQ][kSplitD];   // sum_k 2^(s_k c - m) v_k (unnormalised)
    float m[kSplitQ];            // running max (scaled log2 domain)
    float l[kSplitQ];            // sum_k 2^(s_k c - m)
};

namespace {

__device__ uint32_t g_attn_queue[kQueueSlots][9 * kQWords];   // 8 XCD queues, then the finished-block count
__device__ __attribute__((aligned(256))) SplitPartial g_attn_split[kSplitPieces];
__device__ uint32_t g_attn_split_cnt[8 * kSplitC * kQWords];   // one counter (line) per split item

// Per device: device addresses of the arrays, and the launch tracking of the
// slots and the split scratch.
struct QueueDevice {
    std::mutex mu;
    bool init = false;
    uint32_t* queue = nullptr;
    SplitPartial* split = nullptr;
    uint32_t* split_cnt = nullptr;
    hipEvent_t ev[kQueueSlots + 1] = {};      // [kQueueSlots]: the split scratch
    hipStream_t last[kQueueSlots + 1] = {};
    bool used[kQueueSlots + 1] = {};
    uint32_t next = 0;
};
QueueDevice g_queue_dev[64];

inline hipError_t queue_device(QueueDevice*& out, int& dev) {
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    QueueDevice& d = g_queue_dev[dev];
    std::lock_guard<std::mutex> g(d.mu);   // first use may come from several threads
    if (!d.init) {
        // the arrays' device addresses on this device (their names in host code are not)
        e = hipGetSymbolAddress(reinterpret_cast<void**>(&d.queue), HIP_SYMBOL(g_attn_queue));
        if (e != hipSuccess) return e;
        e = hipGetSymbolAddress(reinterpret_cast<void**>(&d.split), HIP_SYMBOL(g_attn_split));
        if (e != hipSuccess) return e;
        e = hipGetSymbolAddress(reinterpret_cast<void**>(&d.split_cnt), HIP_SYMBOL(g_attn_split_cnt));
        if (e != hipSuccess) return e;
        // The events only tell the host that a launch has finished with its
        // counters and partials, which only kernels on this device read: no
        // system-scope release (with one, each record wrote the L2 back and held
        // the stream's next kernel ~10 us).
        for (int i = 0; i <= kQueueSlots; ++i) {
            e = hipEventCreateWithFlags(&d.ev[i], hipEventDisableTiming | hipEventDisableSystemFence);
            if (e != hipSuccess) return e;
        }
        d.init = true;
    }
    out = &d;
    return hipSuccess;
}

// Host: the current device's compute-unit count (an attribute query only, so a
// first call under stream capture creates nothing).
inline hipError_t device_cus(int& cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    return hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
}

// true if resource i may be used by a launch on `stream` now
inline bool resource_free(QueueDevice& d, int i, hipStream_t stream) {
    if (!d.used[i] || d.last[i] == stream) return true;
    return hipEventQuery(d.ev[i]) == hipSuccess;
}

// Host: run `launch(queue_slot, split, split_cnt)` for a persistent launch on
// `stream` with a free queue slot (and the split scratch if it is free, else
// null), recording the slot's event after it; or, under stream capture or when
// no slot is free, run `fallback()`. Serialised per device.
template <class Persistent, class Fallback>
inline hipError_t persistent_launch(hipStream_t stream, Persistent&& launch, Fallback&& fallback) {
    // under capture first: replays would share device counters, and the state
    // below (events, symbol addresses) is not created inside a capture
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) return fallback();
    QueueDevice* dp = nullptr;
    int dev = 0;
    e = queue_device(dp, dev);
    if (e != hipSuccess) return e;
    QueueDevice& d = *dp;
    std::lock_guard<std::mutex> g(d.mu);
    int slot = -1;
    for (int t = 0; t < kQueueSlots; ++t) {
        const int i = (int)((d.next + t) % kQueueSlots);
        if (resource_free(d, i, stream)) { slot = i; break; }
    }
    if (slot < 0) return fallback();   // kQueueSlots launches in flight on other streams
    d.next = (uint32_t)(slot + 1);
    const bool split = resource_free(d, kQueueSlots, stream);
    e = launch(d.queue + (size_t)slot * 9 * kQWords, split ? d.split : nullptr, split ? d.split_cnt : nullptr);
    if (e != hipSuccess) return e;
    e = hipEventRecord(d.ev[slot], stream);
    if (e != hipSuccess) return e;
    d.used[slot] = true;
    d.last[slot] = stream;
    if (split) {
        e = hipEventRecord(d.ev[kQueueSlots], stream);
        if (e != hipSuccess) return e;
        d.used[kQueueSlots] = true;
        d.last[kQueueSlots] = stream;
    }
    return hipSuccess;
}

}  // namespace

// The XCD this wave runs on (HW_REG_XCC_ID).
__device__ __forceinline__ int xcc_id() {
    return (int)(__builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (31 << 11)) & 7);
}

// Split plan of one XCD's range of len items for C blocks per XCD: the last T
// items are cut into s pieces (s = 1: no split). T = the items of the last,
// partly filled round; s in [2, 16] with T s <= 2C minimises the last round's
// length ceil(T s / C) / s (ties: fewer pieces). A range that divides evenly
// has its whole last round cut in halves: the XCDs' clock differences then
// even out, by stealing, at half-item granularity. Ranges shorter than 2
// rounds are left whole.
__host__ __device__ __forceinline__ void split_plan(int len, int C, bool enabled, int& T, int& s) {
    T = 0;
    s = 1;
    if (!enabled || C > kSplitC || C <= 0 || len < 2 * C) return;
    if (len % C == 0) {
        T = C;
        s = 2;
        return;
    }
    const int t = len % C;
    int best_s = 1, best_num = 1, best_den = 1;   // tail length best_num / best_den (s = 1: 1 round)
    for (int c = 2; c <= kSplitMaxS && t * c <= 2 * C; ++c) {
        const int num = (t * c + C - 1) / C;   // rounds of pieces
        if (num * best_den < best_num * c) { best_s = c; best_num = num; best_den = c; }
    }
    if (best_s > 1) { T = t; s = best_s; }
}

// Units of XCD x's queue: its full items, then T s pieces (piece-major).
__host__ __device__ __forceinline__ int xcd_units(int len, int T, int s) { return len - T + T * s; }

// The next unit for a block on XCD x: its own queue first, then the others in
// turn. Returns the owning XCD v and the unit index u in its range, or v = -1
// when every queue is empty. Counters may run past their range (harmless: they
// are cleared at the end of the launch).
__device__ __forceinline__ void next_unit(uint32_t* q, int total, int C, bool split, int x, int& v, int& u) {
    for (int t = 0; t < 8; ++t) {
        const int y = (x + t) & 7;
        int start, len, T, s;
        xcd_slice(total, y, start, len);
        if (len == 0) continue;
        split_plan(len, C, split, T, s);
        if (t == 0) {   // own queue: full items, then the pieces
            const uint32_t i = atomicAdd(&q[y * kQWords], 1u);
            if (i < (uint32_t)xcd_units(len, T, s)) { v = y; u = (int)i; return; }
            continue;
        }
        // another XCD's queue: full items only (compare-and-swap below its pieces).
        // A split item's pieces and their merge thus share one L2, so publishing
        // a partial needs no L2 write-back.
        const uint32_t avail = (uint32_t)(len - T);
        uint32_t c = __hip_atomic_load(&q[y * kQWords], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        while (c < avail) {
            const uint32_t old = atomicCAS(&q[y * kQWords], c, c + 1);
            if (old == c) { v = y; u = (int)c; return; }
            c = old;
        }
    }
    v = -1;
    u = -1;
}

// Unit u of XCD v -> item index, piece (p of s; s = 1: whole item), and for a
// piece its partial slot and counter index.
struct Unit {
    int item, piece, pieces, slot, counter;
};
__device__ __forceinline__ Unit decode_unit(int total, int C, bool split, int v, int u) {
    int start, len, T, s;
    xcd_slice(total, v, start, len);
    split_plan(len, C, split, T, s);
    Unit r;
    if (u < len - T) {
        r.item = start + u;
        r.piece = 0;
        r.pieces = 1;
        r.slot = r.counter = -1;
    } else {
        const int i = u - (len - T);
        const int it = i % T;
        r.piece = i / T;
        r.pieces = s;
        r.item = start + len - T + it;
        r.slot = v * 2 * kSplitC + it * s + r.piece;
        r.counter = (v * kSplitC + it) * kQWords;
    }
    return r;
}

// Called once per block (one thread) after its last unit: the last block of the
// launch clears the slot's counters.
__device__ __forceinline__ void queue_finish(uint32_t* q, int nblocks) {
    __threadfence();
    if (atomicAdd(&q[8 * kQWords], 1u) == (uint32_t)(nblocks - 1))
        for (int i = 0; i < 9; ++i) __hip_atomic_store(&q[i * kQWords], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
#endif  // DIT_ATTN_PERSISTENT

}  // namespace attn
}  // namespace dit
