// Device-side helpers shared by the gfx950 kernels of libgdn: element conversions and the
// MFMA fragment types. gfx950 only; 64-lane wavefronts.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;

// bf16 <-> fp32. bf16 is the top half of an fp32. fp32 -> bf16 uses gfx950's conversion
// instruction (v_cvt_pk_bf16_f32: round to nearest even, two values per instruction).
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// two floats -> packed bf16 pair (low half = a)
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
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
    r.x = f2bf2(x.x, x.y);
    r.y = f2bf2(x.z, x.w);
    *reinterpret_cast<uint2*>(p) = r;
}
__device__ __forceinline__ void store4(float* p, float4 x) { *reinterpret_cast<float4*>(p) = x; }

// Raw buffer resource over `bytes` bytes at p (stride 0): loads past the end return zero and
// stores past the end are dropped by the hardware. Staging a ragged chunk through one needs no
// per-row branch, so all of a thread's row loads are issued back to back and stay in flight
// together (behind a branch the compiler waits for each load before the next).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int offset) {
    typedef int i32x4_t __attribute__((ext_vector_type(4)));
    const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 0);
    return uint4{(unsigned)v.x, (unsigned)v.y, (unsigned)v.z, (unsigned)v.w};
}
__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, int offset) {
    typedef int i32x2_t __attribute__((ext_vector_type(2)));
    const i32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, offset, 0, 0);
    return uint2{(unsigned)v.x, (unsigned)v.y};
}
__device__ __forceinline__ unsigned buffer_load4(__amdgpu_buffer_rsrc_t r, int offset) {
    return (unsigned)__builtin_amdgcn_raw_buffer_load_b32(r, offset, 0, 0);
}
// 4 consecutive elements from fp32 (bf16: 8 bytes, round to nearest even; fp32: 16 bytes)
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, int offset, float4 x, uint16_t) {
    typedef int i32x2_t __attribute__((ext_vector_type(2)));
    const i32x2_t v = {(int)f2bf2(x.x, x.y), (int)f2bf2(x.z, x.w)};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, offset, 0, 0);
}
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, int offset, float4 x, float) {
    typedef int i32x4_t __attribute__((ext_vector_type(4)));
    const i32x4_t v = {__float_as_int(x.x), __float_as_int(x.y), __float_as_int(x.z), __float_as_int(x.w)};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, offset, 0, 0);
}

}  // namespace gdn
