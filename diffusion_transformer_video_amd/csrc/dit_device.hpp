// Device-side helpers shared by the gfx950 kernels: bf16 <-> fp32 packing,
// 16-byte vector loads/stores of 8 activation values, and wave reductions.
// Activation loads and stores are nontemporal: every activation the
// bandwidth-bound kernels touch is read once and written once per launch. The
// loads matter as much as the stores: a cached load allocates the line in the
// 256 MB memory-side cache, an in-place kernel (RoPE, the merge) then dirties
// it there, and the next kernel pays for writing those lines back (measured:
// modulate after RoPE 159 us instead of 117 us at the 480P video size; RoPE
// back to back 238 us, 214 us with nontemporal loads). Parameter rows (gamma,
// beta, alpha), which many tokens re-read, use cached loads (load_f32x8), and so
// does the merge, where nontemporal loads measured 6% slower.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// 8 consecutive activation values <-> 8 floats.
template <bool BF16>
struct Vec8;

template <>
struct Vec8<true> {
    __device__ __forceinline__ static void load(const void* base, int64_t idx8, float (&f)[8]) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + idx8);
        const uint4 w = make_uint4(v[0], v[1], v[2], v[3]);
        f[0] = bf16lo(w.x); f[1] = bf16hi(w.x); f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
        f[4] = bf16lo(w.z); f[5] = bf16hi(w.z); f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
    }
    __device__ __forceinline__ static void store(void* base, int64_t idx8, const float (&f)[8]) {
        uint4 w;
        w.x = pack_bf16x2(f[0], f[1]); w.y = pack_bf16x2(f[2], f[3]);
        w.z = pack_bf16x2(f[4], f[5]); w.w = pack_bf16x2(f[6], f[7]);
        // streaming output: nontemporal store (not kept in the caches)
        const u32x4 v = {w.x, w.y, w.z, w.w};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(base) + idx8);
    }
};

template <>
struct Vec8<false> {
    __device__ __forceinline__ static void load(const void* base, int64_t idx8, float (&f)[8]) {
        const f32x4* p = reinterpret_cast<const f32x4*>(base) + 2 * idx8;
        const f32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
        f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
        f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    }
    __device__ __forceinline__ static void store(void* base, int64_t idx8, const float (&f)[8]) {
        f32x4* p = reinterpret_cast<f32x4*>(base) + 2 * idx8;
        const f32x4 a = {f[0], f[1], f[2], f[3]};
        const f32x4 b = {f[4], f[5], f[6], f[7]};
        __builtin_nontemporal_store(a, p);
        __builtin_nontemporal_store(b, p + 1);
    }
};

// 8 bf16 values through the caches (the merge's partial: a nontemporal load
// measured slower there)
__device__ __forceinline__ void load_bf16x8_cached(const void* base, int64_t idx8, float (&f)[8]) {
    const uint4 w = reinterpret_cast<const uint4*>(base)[idx8];
    f[0] = bf16lo(w.x); f[1] = bf16hi(w.x); f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
    f[4] = bf16lo(w.z); f[5] = bf16hi(w.z); f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
}

__device__ __forceinline__ void load_f32x8(const float* base, int64_t idx8, float (&f)[8]) {
    const float4* p = reinterpret_cast<const float4*>(base) + 2 * idx8;
    const float4 a = p[0], b = p[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Sum over the 64 lanes of a wave; every lane receives the total. Lane exchanges
// within each row of 16 lanes use DPP (quad_perm xor 1, xor 2, row_half_mirror,
// row_mirror); the four row sums are then read with v_readlane.
__device__ __forceinline__ float wave_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// 8 activation values kept packed in registers (bf16: one uint4; fp32: two).
template <bool BF16>
struct Packed8;

template <>
struct Packed8<true> {
    uint4 w;
    __device__ __forceinline__ void load(const void* base, int64_t idx8) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + idx8);
        w = make_uint4(v[0], v[1], v[2], v[3]);
    }
    __device__ __forceinline__ void zero() { w = make_uint4(0, 0, 0, 0); }
    // Load of chunk idx8 if ok, else of chunk 0 (always in bounds; the caller
    // ignores it). Branch-free: a load under a lane-divergent branch whose other
    // side zeroes the registers makes the compiler wait for each such load
    // before the next is issued.
    __device__ __forceinline__ void load_or_first(const void* base, int64_t idx8, bool ok) {
        load(base, ok ? idx8 : 0);
    }
    // Empty asm that "redefines" the packed words: later passes unpack again
    // instead of the compiler keeping all unpacked floats live (emits nothing).
    __device__ __forceinline__ void refresh() { asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w)); }
    __device__ __forceinline__ void unpack(float (&f)[8]) const {
        f[0] = bf16lo(w.x); f[1] = bf16hi(w.x); f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
        f[4] = bf16lo(w.z); f[5] = bf16hi(w.z); f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
    }
};

template <>
struct Packed8<false> {
    float4 a, b;
    __device__ __forceinline__ void load(const void* base, int64_t idx8) {
        const f32x4* p = reinterpret_cast<const f32x4*>(base) + 2 * idx8;
        const f32x4 x = __builtin_nontemporal_load(p), y = __builtin_nontemporal_load(p + 1);
        a = make_float4(x[0], x[1], x[2], x[3]);
        b = make_float4(y[0], y[1], y[2], y[3]);
    }
    __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void load_or_first(const void* base, int64_t idx8, bool ok) {
        load(base, ok ? idx8 : 0);
    }
    __device__ __forceinline__ void refresh() {}
    __device__ __forceinline__ void unpack(float (&f)[8]) const {
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
};

}  // namespace dit
