// MFMA fragment conventions for the gfx950 prefill kernels.
//
// A "fragment" is one 16-byte register quad per lane of a 64-lane wave (1 KB per wave) holding
// a 16 x KB operand block of v_mfma_f32_16x16x32_bf16 (KB = 32) or of four chained
// v_mfma_f32_16x16x4_f32 (KB = 16). Lane l = 16 j + m holds row m (A operand) or column m
// (B operand) and the KB/4 k-indices kofs(j, e), e = 0 .. KB/4 - 1.
//
// The k-order is chosen so that the fp32 accumulator of a 16 x 16 MFMA tile (lane 16 j + n
// holds rows 4 j .. 4 j + 3 of column n) converts to an operand fragment in registers with no
// data movement: for bf16 a fragment packs two row-adjacent accumulator tiles, for fp32 one.
// Because the hardware pairs element e of A's lane (j, m) with element e of B's lane (j, n),
// any k-order gives the exact product as long as both operands use the same one.
#pragma once
#include "gdn_device.h"

namespace gdn {

constexpr int CH = 64;  // chunk length in tokens

template <class E>
struct MM;

template <>
struct MM<BF16> {
    static constexpr int KB = 32;  // k extent of one fragment
    static constexpr int EPF = 8;  // elements per lane
    using frag = bf16x8;
    static __device__ __forceinline__ f32x4 mma(const frag& a, const frag& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // k offset (within the fragment's KB-block) of element e held by lane group j
    static __device__ __forceinline__ int kofs(int j, int e) { return e < 4 ? 4 * j + e : 12 + 4 * j + e; }
    static __device__ __forceinline__ frag pack(const float (&x)[8]) {
        const uint4 u = {f2bf2(x[0], x[1]), f2bf2(x[2], x[3]), f2bf2(x[4], x[5]), f2bf2(x[6], x[7])};
        return __builtin_bit_cast(frag, u);
    }
    // fragment of k-block kb from accumulator tiles t[2 kb], t[2 kb + 1], times s
    static __device__ __forceinline__ frag from_acc(const f32x4* t, int kb, float s = 1.f) {
        const float x[8] = {t[2 * kb][0] * s, t[2 * kb][1] * s, t[2 * kb][2] * s, t[2 * kb][3] * s,
                            t[2 * kb + 1][0] * s, t[2 * kb + 1][1] * s, t[2 * kb + 1][2] * s, t[2 * kb + 1][3] * s};
        return pack(x);
    }
};

template <>
struct MM<F32> {
    static constexpr int KB = 16;
    static constexpr int EPF = 4;
    using frag = f32x4;
    static __device__ __forceinline__ f32x4 mma(const frag& a, const frag& b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ int kofs(int j, int e) { return 4 * j + e; }
    static __device__ __forceinline__ frag pack(const float (&x)[4]) { return frag{x[0], x[1], x[2], x[3]}; }
    static __device__ __forceinline__ frag from_acc(const f32x4* t, int kb, float s = 1.f) {
        return frag{t[kb][0] * s, t[kb][1] * s, t[kb][2] * s, t[kb][3] * s};
    }
};

// 16-byte fragment store / load (lane-contiguous, 1 KB per fragment)
template <class F>
__device__ __forceinline__ void st_frag(void* base, int lane, const F& f) {
    *reinterpret_cast<F*>(static_cast<char*>(base) + lane * 16) = f;
}
template <class F>
__device__ __forceinline__ F ld_frag(const void* base, int lane) {
    return *reinterpret_cast<const F*>(static_cast<const char*>(base) + lane * 16);
}

// Fragment whose lane (j, m) takes row `rp` (row m of the operand, k contiguous in memory)
// at k = k0 + kofs(j, e), every element multiplied by `s`. rp == nullptr gives zeros.
template <class E>
__device__ __forceinline__ typename MM<E>::frag row_frag(const typename E::T* rp, int k0, int j, float s) {
    using M = MM<E>;
    float x[M::EPF];
    if (rp) {
        const float4 a = load4(rp + k0 + 4 * j);
        x[0] = a.x * s; x[1] = a.y * s; x[2] = a.z * s; x[3] = a.w * s;
        if constexpr (M::EPF == 8) {
            const float4 b = load4(rp + k0 + 16 + 4 * j);
            x[4] = b.x * s; x[5] = b.y * s; x[6] = b.z * s; x[7] = b.w * s;
        }
    } else {
#pragma unroll
        for (int e = 0; e < M::EPF; ++e) x[e] = 0.f;
    }
    return M::pack(x);
}

// Same, with a per-k scale sk[k] (k = k0 + kofs(j, e)) instead of one scalar.
template <class E>
__device__ __forceinline__ typename MM<E>::frag row_frag_ks(const typename E::T* rp, int k0, int j, const float* sk) {
    using M = MM<E>;
    float x[M::EPF];
    const float4 a = load4(rp + k0 + 4 * j);
    const float4 sa = *reinterpret_cast<const float4*>(sk + k0 + 4 * j);
    x[0] = a.x * sa.x; x[1] = a.y * sa.y; x[2] = a.z * sa.z; x[3] = a.w * sa.w;
    if constexpr (M::EPF == 8) {
        const float4 b = load4(rp + k0 + 16 + 4 * j);
        const float4 sb = *reinterpret_cast<const float4*>(sk + k0 + 16 + 4 * j);
        x[4] = b.x * sb.x; x[5] = b.y * sb.y; x[6] = b.z * sb.z; x[7] = b.w * sb.w;
    }
    return M::pack(x);
}

// Fragment from an fp32 row (LDS) at k = k0 + kofs(j, e).
template <class E>
__device__ __forceinline__ typename MM<E>::frag row_frag_f32(const float* rp, int k0, int j) {
    using M = MM<E>;
    float x[M::EPF];
    const float4 a = *reinterpret_cast<const float4*>(rp + k0 + 4 * j);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    if constexpr (M::EPF == 8) {
        const float4 b = *reinterpret_cast<const float4*>(rp + k0 + 16 + 4 * j);
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    return M::pack(x);
}

// Fragment of a row (k contiguous in memory) at k = k0 + kofs(j, e), taken as stored.
template <class E>
__device__ __forceinline__ typename MM<E>::frag row_frag_raw(const typename E::T* rp, int k0, int j) {
    if constexpr (MM<E>::EPF == 8) {
        const uint2 a = *reinterpret_cast<const uint2*>(rp + k0 + 4 * j);
        const uint2 b = *reinterpret_cast<const uint2*>(rp + k0 + 16 + 4 * j);
        return __builtin_bit_cast(bf16x8, uint4{a.x, a.y, b.x, b.y});
    } else {
        return *reinterpret_cast<const f32x4*>(rp + k0 + 4 * j);
    }
}

// B operand whose column n is the unit vector at k = n + 16 q. The product of a row fragment
// with it is exact and lands the 16 selected columns in an accumulator tile, where lane (j, n)
// holds rows 4 j .. 4 j + 3 of column n: a transpose done by the matrix core.
template <class E>
__device__ __forceinline__ typename MM<E>::frag unit_cols(int j, int n, int q) {
    using M = MM<E>;
    float x[M::EPF];
#pragma unroll
    for (int e = 0; e < M::EPF; ++e) x[e] = M::kofs(j, e) == n + 16 * q ? 1.f : 0.f;
    return M::pack(x);
}

// Operand fragment whose k index runs over the rows of KB / 16 consecutive accumulator tiles
// t[0], t[1], ... (16 rows each), row s scaled by sk[s] (sk indexed from the first tile's row 0).
template <class E>
__device__ __forceinline__ typename MM<E>::frag cols_frag(const f32x4* t, const float* sk, int j) {
    using M = MM<E>;
    float x[M::EPF];
#pragma unroll
    for (int i = 0; i < M::EPF / 4; ++i) {
        const float4 s = *reinterpret_cast<const float4*>(sk + 16 * i + 4 * j);
        x[4 * i + 0] = t[i][0] * s.x; x[4 * i + 1] = t[i][1] * s.y;
        x[4 * i + 2] = t[i][2] * s.z; x[4 * i + 3] = t[i][3] * s.w;
    }
    return M::pack(x);
}
template <class E>
__device__ __forceinline__ typename MM<E>::frag cols_frag(const f32x4* t) {
    using M = MM<E>;
    float x[M::EPF];
#pragma unroll
    for (int i = 0; i < M::EPF / 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * i + e] = t[i][e];
    return M::pack(x);
}

// Operand fragment (k = token, in the fragment k-order) of columns n0 .. n0 + 15 and tokens
// k0 .. k0 + 31 of a token-major bf16 array in LDS (row stride kp elements), by two transposing
// reads: within each 16-lane group, lane s supplies row k0 + 4 j + s / 4 (+ 16) at column
// n0 + 4 (s % 4), and lane m receives column n0 + m of the group's four rows.
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* base, int kp, int k0, int n0, int j, int m) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const int row = k0 + 4 * j + (m >> 2), col = n0 + 4 * (m & 3);
    const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + row * kp + col));
    const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + (row + 16) * kp + col));
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// bf16 fragment with element e (k = k0 + kofs(j, e)) multiplied by sk[k] in fp32, rounded once
__device__ __forceinline__ bf16x8 scale_frag(const bf16x8& f, const float* sk, int j) {
    const float4 s0 = *reinterpret_cast<const float4*>(sk + 4 * j);
    const float4 s1 = *reinterpret_cast<const float4*>(sk + 16 + 4 * j);
    const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = bf2f((uint16_t)f[e]) * s[e];
    return MM<BF16>::pack(x);
}

}  // namespace gdn
