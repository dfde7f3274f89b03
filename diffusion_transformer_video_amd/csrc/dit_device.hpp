// Device-side helpers shared by the gfx950 kernels: bf16 <-> fp32 packing,
// 16-byte vector loads/stores of 8 activation values, and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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
        const uint4 w = reinterpret_cast<const uint4*>(base)[idx8];
        f[0] = bf16lo(w.x); f[1] = bf16hi(w.x); f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
        f[4] = bf16lo(w.z); f[5] = bf16hi(w.z); f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
    }
    __device__ __forceinline__ static void store(void* base, int64_t idx8, const float (&f)[8]) {
        uint4 w;
        w.x = pack_bf16x2(f[0], f[1]); w.y = pack_bf16x2(f[2], f[3]);
        w.z = pack_bf16x2(f[4], f[5]); w.w = pack_bf16x2(f[6], f[7]);
        reinterpret_cast<uint4*>(base)[idx8] = w;
    }
};

template <>
struct Vec8<false> {
    __device__ __forceinline__ static void load(const void* base, int64_t idx8, float (&f)[8]) {
        const float4* p = reinterpret_cast<const float4*>(base) + 2 * idx8;
        const float4 a = p[0], b = p[1];
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
    __device__ __forceinline__ static void store(void* base, int64_t idx8, const float (&f)[8]) {
        float4* p = reinterpret_cast<float4*>(base) + 2 * idx8;
        p[0] = make_float4(f[0], f[1], f[2], f[3]);
        p[1] = make_float4(f[4], f[5], f[6], f[7]);
    }
};

__device__ __forceinline__ void load_f32x8(const float* base, int64_t idx8, float (&f)[8]) {
    const float4* p = reinterpret_cast<const float4*>(base) + 2 * idx8;
    const float4 a = p[0], b = p[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Sum over the 64 lanes of a wave; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace dit
