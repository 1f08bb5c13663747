// Device-side helpers shared by the gfx950 kernels of libgdn: element conversions and the
// MFMA fragment types. gfx950 only; 64-lane wavefronts.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// bf16 <-> fp32. bf16 is the top half of an fp32; rounding is to nearest, ties to even,
// and NaN stays NaN.
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// storage element types of q, k, v and o
struct BF16 {
    using T = uint16_t;
    static __device__ __forceinline__ float load(const T* p) { return bf2f(*p); }
    static __device__ __forceinline__ T from(float f) { return f2bf(f); }
};
struct F32 {
    using T = float;
    static __device__ __forceinline__ float load(const T* p) { return *p; }
    static __device__ __forceinline__ T from(float f) { return f; }
};

// 4 consecutive elements as fp32
__device__ __forceinline__ float4 load4(const uint16_t* p) {
    uint2 r = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
}
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }

__device__ __forceinline__ void store4(uint16_t* p, float4 x) {
    uint2 r;
    r.x = (uint32_t)f2bf(x.x) | ((uint32_t)f2bf(x.y) << 16);
    r.y = (uint32_t)f2bf(x.z) | ((uint32_t)f2bf(x.w) << 16);
    *reinterpret_cast<uint2*>(p) = r;
}
__device__ __forceinline__ void store4(float* p, float4 x) { *reinterpret_cast<float4*>(p) = x; }

}  // namespace gdn
