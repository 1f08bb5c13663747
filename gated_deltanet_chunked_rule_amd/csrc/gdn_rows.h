// Row staging and small wave / workgroup helpers shared by the linear-attention kernels
// (causal and bidirectional). gfx950 only; 64-lane wavefronts, 256-thread workgroups unless stated.
#pragma once
#include "gdn_mfma.h"

namespace gdn {

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ float wave_scan(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
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
    // 16 bytes), f applied to rows [0, n), the others zero (masked, not branched, so that the
    // loads still in flight are not drained here)
    template <class F = AsIs>
    __device__ __forceinline__ void store(typename E::T* dst, int n, int tid, F f = F()) const {
        constexpr int KP = row_stride<D, E>();
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int u = tid + NT * i, r = u / UPR, cu = u % UPR;
            const unsigned keep = 0u - (unsigned)(r < n);
            const uint4 y = f(x[i]);
            uint2* d = reinterpret_cast<uint2*>(dst + r * KP + cu * EPU);
            d[0] = uint2{y.x & keep, y.y & keep};
            d[1] = uint2{y.z & keep, y.w & keep};
        }
    }
};

}  // namespace gdn
