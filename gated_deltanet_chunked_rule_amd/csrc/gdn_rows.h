// Row staging and small wave / workgroup helpers shared by the linear-attention kernels
// (causal and bidirectional). gfx950 only; 64-lane wavefronts, 256-thread workgroups unless stated.
#pragma once
#include <type_traits>
#include "gdn_mfma.h"

namespace gdn {

// Log gates below this bound are taken as the bound. Any product of gates that contains one is
// then exp(x) with x <= -110 (log a <= 0 otherwise), which is exactly zero in fp32 (below half the
// smallest subnormal), so such a gate, a zero gate (log a = -inf) included, closes the state
// exactly while every cumulative sum stays finite: no -inf - (-inf) in their differences. NaN is
// kept (it propagates).
constexpr float LOG_GATE_FLOOR = -110.f;
__device__ __forceinline__ float floor_log_gate(float x) { return x < LOG_GATE_FLOOR ? LOG_GATE_FLOOR : x; }

// One step of a wave scan on DPP: the value `ctrl` moves into each lane (rows outside
// `row_mask`, and lanes with no source, receive `id`).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_move(int x, int id) {
    return __builtin_amdgcn_update_dpp(id, x, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive scan over the 64 lanes of a wave (op associative, id its identity): shifts right by
// 1, 2, 4 and 8 lanes within each row of 16, then the totals of rows 0 and 2 (lanes 15 and 47)
// into rows 1 and 3, then the total of rows 0-1 (lane 31) into rows 2 and 3.
template <class V, class Op>
__device__ __forceinline__ V wave_scan_dpp(V x, V id, Op op) {
    const int idb = __builtin_bit_cast(int, id);
    auto step = [&](auto y) { x = op(x, __builtin_bit_cast(V, y)); };
    step(dpp_move<0x111, 0xF>(__builtin_bit_cast(int, x), idb));   // row_shr:1
    step(dpp_move<0x112, 0xF>(__builtin_bit_cast(int, x), idb));   // row_shr:2
    step(dpp_move<0x114, 0xF>(__builtin_bit_cast(int, x), idb));   // row_shr:4
    step(dpp_move<0x118, 0xF>(__builtin_bit_cast(int, x), idb));   // row_shr:8
    step(dpp_move<0x142, 0xA>(__builtin_bit_cast(int, x), idb));   // row_bcast:15
    step(dpp_move<0x143, 0xC>(__builtin_bit_cast(int, x), idb));   // row_bcast:31
    return x;
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ float wave_scan(float x, int /*lane*/) {
    return wave_scan_dpp(x, 0.f, [](float a, float b) { return a + b; });
}

// Inclusive prefix sum over the 64 lanes of a wave carried as an unevaluated sum hi + lo (the
// return value and `lo`): every step adds exactly (the rounding error of each fp32 addition is
// recovered and carried in lo), so a difference of two prefix sums formed as
// (hi_r - hi_s) + (lo_r - lo_s) keeps fp32 precision relative to the difference even where the
// sums themselves are large (strong decay: a chunk's log gates summing to -10^3).
__device__ __forceinline__ float wave_scan2(float x, float& lo) {
    float hi = x;
    lo = 0.f;
    auto add = [&](float h2, float l2) {   // (hi, lo) += (h2, l2), hi + h2 exactly
        const float s = hi + h2, bb = s - hi, e = (hi - (s - bb)) + (h2 - bb);
        lo = lo + l2 + e;
        hi = s;
    };
#define GDN_SCAN2_STEP(CTRL, MASK)                                                                     \
    add(__builtin_bit_cast(float, dpp_move<CTRL, MASK>(__builtin_bit_cast(int, hi), 0)),              \
        __builtin_bit_cast(float, dpp_move<CTRL, MASK>(__builtin_bit_cast(int, lo), 0)));
    GDN_SCAN2_STEP(0x111, 0xF)   // row_shr:1
    GDN_SCAN2_STEP(0x112, 0xF)   // row_shr:2
    GDN_SCAN2_STEP(0x114, 0xF)   // row_shr:4
    GDN_SCAN2_STEP(0x118, 0xF)   // row_shr:8
    GDN_SCAN2_STEP(0x142, 0xA)   // row_bcast:15
    GDN_SCAN2_STEP(0x143, 0xC)   // row_bcast:31
#undef GDN_SCAN2_STEP
    return hi;
}

// value of lane 63 (the inclusive total), in every lane
__device__ __forceinline__ float wave_last(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// LDS-only workgroup barrier: waits for this wave's LDS operations (lgkmcnt) and nothing else,
// for waves that exchange nothing through global memory (__syncthreads would also drain every
// outstanding global load and store first)
__device__ __forceinline__ void lds_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Row stride (elements) of a chunk's rows staged in LDS. The fragment reads take 8 bytes (bf16)
// or 16 bytes (fp32) per lane from 16 consecutive rows at the same column; with a stride of
// D + 4 elements (66 or 132 dwords, 2 or 4 mod 32) those rows fall on distinct banks of the
// 32-bank LDS, where D + 8 (4 or 8 mod 32) put two rows on each bank.
template <int D, class E>
constexpr int row_stride() { return D + 4; }

// 16 bytes of storage elements, unchanged
struct AsIs {
    __device__ __forceinline__ uint4 operator()(uint4 x) const { return x; }
};

// A 64-row chunk (row stride D in global memory) in flight in registers: NT threads (256 unless
// stated), 16 bytes each per step. Loading the next chunk while the current one is processed keeps more of HBM's
// latency covered than the workgroups of one CU do alone. Loads go through a buffer resource
// over the chunk's valid rows, so the rows past the end of the sequence read as zero and no
// load sits behind a branch.
template <int D, class E, int NT = 256>
struct RowRegs {
    static constexpr int ES = sizeof(typename E::T), EPU = 16 / ES, UPR = D / EPU, N = CH * UPR / NT;
    uint4 x[N];
    // rows [0, n) of src; the others are zero
    __device__ __forceinline__ void load(const typename E::T* src, int n, int tid) {
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src, n * D * ES);
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = buffer_load16(rs, (tid + NT * i) * 16);
    }
    // into LDS with row stride row_stride<D, E>() (rows 8-byte aligned: two 8-byte stores per
    // 16 bytes), f applied to rows [0, n), the others zero. Unit u = tid + NT i is row u / UPR,
    // column unit u % UPR; NT is a multiple of UPR, so step i moves NT / UPR rows down from one
    // base address. Rows past n already hold zeros (their loads were out of range); only a
    // transform f, which need not map zero to zero, needs the mask (masked, not branched, so that
    // the loads still in flight are not drained here).
    template <class F = AsIs>
    __device__ __forceinline__ void store(typename E::T* dst, int n, int tid, F f = F()) const {
        constexpr int KP = row_stride<D, E>();
        static_assert(NT % UPR == 0, "whole rows per step");
        constexpr bool MASK = !std::is_same<F, AsIs>::value;
        const unsigned ut = (unsigned)tid, r0 = ut / UPR;
        typename E::T* base = dst + r0 * KP + (ut % UPR) * EPU;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            uint4 y = f(x[i]);
            if constexpr (MASK) {
                const unsigned keep = 0u - (unsigned)((int)(r0 + (NT / UPR) * i) < n);
                y = uint4{y.x & keep, y.y & keep, y.z & keep, y.w & keep};
            }
            uint2* d = reinterpret_cast<uint2*>(base + (NT / UPR) * i * KP);
            d[0] = uint2{y.x, y.y};
            d[1] = uint2{y.z, y.w};
        }
    }
};

}  // namespace gdn
