// Bidirectional (non-causal) linear attention on gfx950.
//
// The datadaily.news overview (section "Linear attention") gives the kernel-feature-map form:
// with a feature map phi (elu(x) + 1 there; the identity when the caller has applied one),
//     KV = sum_n phi(k_n) v_n^T   (Dk x Dv, one per head, over the whole sequence)
//     o_n = KV^T phi(q_n),  divided by Z_n = phi(q_n) . sum_m phi(k_m) when normalising.
// Associativity makes the cost linear in L: the sequence is read once to build KV and once to
// produce the outputs.
//
// Three kernels, all on the matrix cores:
//   1. bidir_kv_kernel: one workgroup per (block of chunks, head) sums phi(K)^T V over its
//      chunks. The products contract over tokens, so both operands need fragments whose k index
//      is the token: K and V rows are staged in LDS and read as columns by gfx950's transposing
//      LDS reads (bf16), or turned into columns by one MFMA per 16 x 16 tile against a
//      unit-column fragment (fp32, an exact transpose). Each wave transposes a quarter of the key dimensions and publishes them in LDS, and
//      transposes its own value tiles, which it keeps; it owns the KV tiles of its value columns.
//      The per-block sums (and key sums) go to the workspace in accumulator-tile layout.
//   2. bidir_reduce_kernel: one wave per KV operand fragment sums the blocks' tiles in a fixed
//      order (deterministic), writes the fragment for stage 3 and, if asked, KV in fp32.
//   3. bidir_out_kernel: one workgroup per (group of chunks, head). Each wave keeps the KV
//      fragments of its value columns in registers for all its chunks; the chunk's phi(Q) rows
//      are staged in LDS; O^T tiles = KV^T phi(Q)^T come out with four consecutive value columns
//      per lane for the store, and Z from the same Q fragments and the fp32 key sums.
// phi is applied in fp32 when a row is staged and then rounded to the storage type, so KV, the
// key sums and Z all use the same rounded feature values. Rows past the end of the sequence
// stay zero (they are not passed through phi).
#include <stdint.h>

#include "gdn_launch.h"
#include "gdn_rows.h"

namespace gdn {

namespace {

// phi: elu(x) + 1 = x + 1 for x > 0, exp(x) otherwise; or the identity (both sides evaluated,
// so no branch)
template <bool ELU1>
__device__ __forceinline__ float phi(float x) {
    if constexpr (ELU1) {
        const float e = __expf(fminf(x, 0.f)), p = x + 1.f;
        return x > 0.f ? p : e;
    } else {
        return x;
    }
}

// 16-byte group of storage elements -> phi applied -> back to storage
template <class E, bool ELU1>
__device__ __forceinline__ uint4 phi16(uint4 x) {
    if constexpr (!ELU1) {
        return x;
    } else if constexpr (sizeof(typename E::T) == 2) {
        uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = f2bf2(phi<true>(__uint_as_float(w[i] << 16)), phi<true>(__uint_as_float(w[i] & 0xffff0000u)));
        return uint4{w[0], w[1], w[2], w[3]};
    } else {
        return uint4{__float_as_uint(phi<true>(__uint_as_float(x.x))), __float_as_uint(phi<true>(__uint_as_float(x.y))),
                     __float_as_uint(phi<true>(__uint_as_float(x.z))), __float_as_uint(phi<true>(__uint_as_float(x.w)))};
    }
}

// phi on 16 bytes of storage elements, as a row-staging transform
template <class E, bool ELU1>
struct Phi16 {
    __device__ __forceinline__ uint4 operator()(uint4 x) const { return phi16<E, ELU1>(x); }
};

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

}  // namespace

// Workspace layout per head (bytes): partial tiles [NB][NDT * NDT][64 lanes][4] fp32, partial
// key sums [NB][D] fp32, KV operand fragments [NDT][NKD] x 1 KB, key sums [D] fp32; the head's
// block is rounded up to 256 bytes.
template <int D, class E>
struct BidirLayout {
    static constexpr int NDT = D / 16;
    static constexpr int NKD = D / MM<E>::KB;
    static __host__ __device__ size_t part(int nb) { return (size_t)nb * NDT * NDT * 1024; }
    static __host__ __device__ size_t pks(int nb) { return part(nb); }
    static __host__ __device__ size_t kvf(int nb) { return pks(nb) + (size_t)nb * D * 4; }
    static __host__ __device__ size_t ks(int nb) { return kvf(nb) + (size_t)NDT * NKD * 1024; }
    static __host__ __device__ size_t head(int nb) { return (ks(nb) + D * 4 + 255) / 256 * 256; }
};

// Blocks of chunks per head for stage 1: enough workgroups to fill the chip (about 768), at
// least one chunk each.
static int bidir_blocks(long BH, long nch) {
    long nb = (768 + BH - 1) / BH;
    if (nb > nch) nb = nch;
    if (nb < 1) nb = 1;
    const long cpb = (nch + nb - 1) / nb;
    return (int)((nch + cpb - 1) / cpb);
}

size_t bidir_workspace_bytes(long BH, long L, int D, int dtype) {
    if (L <= 0) return 0;
    const long nch = (L + CH - 1) / CH;
    const int nb = bidir_blocks(BH, nch);
    const size_t head = D == 128 ? (dtype == 0 ? BidirLayout<128, BF16>::head(nb) : BidirLayout<128, F32>::head(nb))
                                 : (dtype == 0 ? BidirLayout<64, BF16>::head(nb) : BidirLayout<64, F32>::head(nb));
    return head * (size_t)BH;
}

// ---------------------------------------------------------------------------------------------
// stage 1: per-block sums of phi(K)^T V and of phi(K)
// ---------------------------------------------------------------------------------------------
template <int D, class E, bool ELU1>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(typename E::T) == 2 ? 3 : 1))) void bidir_kv_kernel(const typename E::T* __restrict__ k,
                                                       const typename E::T* __restrict__ v, unsigned char* ws,
                                                       long L, int cpb, int nb) {
    using T = typename E::T;
    using M = MM<E>;
    using Ly = BidirLayout<D, E>;
    using frag = typename M::frag;
    constexpr int KB = M::KB, NDT = Ly::NDT, NKT = CH / KB, FPD = KB / 16, KP = row_stride<D, E>();
    constexpr int DW = NDT / 4;   // key tiles a wave transposes = value tiles it owns
    extern __shared__ __align__(16) unsigned char smem[];
    T* Kr = reinterpret_cast<T*>(smem);                                   // [CH][KP]
    T* Vr = Kr + CH * KP;                                                 // [CH][KP]
    unsigned char* sKf = reinterpret_cast<unsigned char*>(Vr + CH * KP);  // K^T fragments [dt][kt]

    const int blk = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, j = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: no MFMA under a lane mask
    const long nch = (L + CH - 1) / CH;
    const long c_begin = (long)blk * cpb;
    const long c_end = c_begin + cpb < nch ? c_begin + cpb : nch;

    f32x4 acc[NDT][DW];   // KV tiles (dt, value tile DW w + i)
    float ksp[DW];        // per-lane partial key sums of key tiles DW w + i, column n = m
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < DW; ++i) acc[dt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < DW; ++i) ksp[i] = 0.f;

    // transposed tiles of d-tile dt of rows R: lane (j, n) holds R[16 st + 4 j + e][16 dt + n]
    auto tiles = [&](const T* R, int dt, f32x4 (&t)[4]) {
        const frag sel = unit_cols<E>(j, m, dt % FPD);
#pragma unroll
        for (int st = 0; st < 4; ++st)
            t[st] = M::mma(row_frag_raw<E>(R + (16 * st + m) * KP, KB * (dt / FPD), j), sel, f32x4{0.f, 0.f, 0.f, 0.f});
    };

    auto rows_of = [&](long c) { return (int)(L - c * CH < CH ? L - c * CH : CH); };
    RowRegs<D, E> rk, rv;
    rk.load(k + ((size_t)bh * L + c_begin * CH) * D, rows_of(c_begin), tid);
    rv.load(v + ((size_t)bh * L + c_begin * CH) * D, rows_of(c_begin), tid);
    for (long c = c_begin; c < c_end; ++c) {
        const int n = rows_of(c);
        rk.store(Kr, n, tid, Phi16<E, ELU1>());
        rv.store(Vr, n, tid);
        if (c + 1 < c_end) {   // the next chunk's rows, in flight during this one
            const size_t tok1 = (size_t)bh * L + (c + 1) * CH;
            rk.load(k + tok1 * D, rows_of(c + 1), tid);
            rv.load(v + tok1 * D, rows_of(c + 1), tid);
        }
        lds_sync();
        // this wave's key tiles -> K^T fragments in LDS (and key sums); its value tiles -> V
        // fragments kept in registers
        frag vf[DW][NKT];
#pragma unroll
        for (int i = 0; i < DW; ++i) {
            const int dt = DW * w + i;
            if constexpr (sizeof(T) == 2) {
                // bf16: gfx950's transposing LDS reads; fragment kt's elements 0-3 and 4-7 are the
                // lane's tokens of 16-token tiles 2 kt and 2 kt + 1, summed in that tile order
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    const frag kr = tr_frag(Kr, KP, KB * kt, 16 * dt, j, m);
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = bf2f((uint16_t)kr[e]);
                    ksp[i] += (x[0] + x[1]) + (x[2] + x[3]);
                    ksp[i] += (x[4] + x[5]) + (x[6] + x[7]);
                    st_frag(sKf + (size_t)(dt * NKT + kt) * 1024, lane, kr);
                    vf[i][kt] = tr_frag(Vr, KP, KB * kt, 16 * dt, j, m);
                }
            } else {   // fp32: transposed on the matrix core
                f32x4 t[4];
                tiles(Kr, dt, t);
#pragma unroll
                for (int st = 0; st < 4; ++st) ksp[i] += (t[st][0] + t[st][1]) + (t[st][2] + t[st][3]);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) st_frag(sKf + (size_t)(dt * NKT + kt) * 1024, lane, cols_frag<E>(&t[FPD * kt]));
                tiles(Vr, dt, t);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) vf[i][kt] = cols_frag<E>(&t[FPD * kt]);
            }
        }
        lds_sync();
        // KV tiles (dt, value tile) += phi(K)^T[dt rows][tokens] V[tokens][value columns]
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                const frag kf = ld_frag<frag>(sKf + (size_t)(dt * NKT + kt) * 1024, lane);
#pragma unroll
                for (int i = 0; i < DW; ++i) acc[dt][i] = M::mma(kf, vf[i][kt], acc[dt][i]);
            }
    }
    // the block's tiles and key sums
    unsigned char* hb = ws + (size_t)bh * Ly::head(nb);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < DW; ++i) {
            const int vt = DW * w + i;
            st_frag(hb + ((size_t)blk * NDT * NDT + dt * NDT + vt) * 1024, lane, acc[dt][i]);
        }
#pragma unroll
    for (int i = 0; i < DW; ++i) {
        float s = ksp[i];
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        if (j == 0) reinterpret_cast<float*>(hb + Ly::pks(nb))[(size_t)blk * D + 16 * (DW * w + i) + m] = s;
    }
}

// ---------------------------------------------------------------------------------------------
// stage 2: sum the blocks; KV operand fragments (and KV in fp32 if asked), key sums
// ---------------------------------------------------------------------------------------------
// One wave per fragment (value tile vt, key block kd): the fragment packs the FPD key tiles
// FPD kd .. of column tile vt (lane (j, n): KV[key KB kd + kofs(j, e)][value 16 vt + n]), which
// is both the A operand of KV^T (row = value) and the accumulator layout of stage 1.
template <int D, class E>
__global__ __launch_bounds__(256) void bidir_reduce_kernel(unsigned char* ws, float* kv_out, int nb) {
    using M = MM<E>;
    using Ly = BidirLayout<D, E>;
    constexpr int NDT = Ly::NDT, NKD = Ly::NKD, FPD = M::KB / 16;
    const int bh = blockIdx.y, lane = threadIdx.x & 63, j = lane >> 4, n = lane & 15;
    const int f = blockIdx.x * 4 + (threadIdx.x >> 6);   // fragment index vt * NKD + kd
    unsigned char* hb = ws + (size_t)bh * Ly::head(nb);
    if (f < NDT * NKD) {
        const int vt = f / NKD, kd = f % NKD;
        // the FPD tiles of the fragment summed over the blocks in block order, eight blocks'
        // loads in flight per step
        f32x4 t[FPD];
#pragma unroll
        for (int u = 0; u < FPD; ++u) t[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto tile_at = [&](int b, int u) {
            return ld_frag<f32x4>(hb + ((size_t)b * NDT * NDT + (FPD * kd + u) * NDT + vt) * 1024, lane);
        };
        int b = 0;
        for (; b + 8 <= nb; b += 8) {
            f32x4 x[8][FPD];
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int u = 0; u < FPD; ++u) x[i][u] = tile_at(b + i, u);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int u = 0; u < FPD; ++u)
                    t[u] = f32x4{t[u][0] + x[i][u][0], t[u][1] + x[i][u][1], t[u][2] + x[i][u][2], t[u][3] + x[i][u][3]};
        }
        for (; b < nb; ++b)
#pragma unroll
            for (int u = 0; u < FPD; ++u) {
                const f32x4 x = tile_at(b, u);
                t[u] = f32x4{t[u][0] + x[0], t[u][1] + x[1], t[u][2] + x[2], t[u][3] + x[3]};
            }
        if (kv_out) {
            float* dst = kv_out + (size_t)bh * D * D;
#pragma unroll
            for (int u = 0; u < FPD; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(size_t)(16 * (FPD * kd + u) + 4 * j + e) * D + 16 * vt + n] = t[u][e];
        }
        st_frag(hb + Ly::kvf(nb) + (size_t)f * 1024, lane, M::from_acc(t, 0));
    }
    if (blockIdx.x == 0 && threadIdx.x < D) {
        const float* pks = reinterpret_cast<const float*>(hb + Ly::pks(nb));
        float s = 0.f;
        for (int b = 0; b < nb; ++b) s += pks[(size_t)b * D + threadIdx.x];
        reinterpret_cast<float*>(hb + Ly::ks(nb))[threadIdx.x] = s;
    }
}

// ---------------------------------------------------------------------------------------------
// stage 3: o = KV^T phi(q) [/ Z]
// ---------------------------------------------------------------------------------------------
template <int D, class E, bool ELU1, bool NORM>
__global__ __launch_bounds__(256) void bidir_out_kernel(const typename E::T* __restrict__ q,
                                                        const unsigned char* __restrict__ ws,
                                                        typename E::T* __restrict__ o, long L, int cpw, int nb) {
    using T = typename E::T;
    using M = MM<E>;
    using Ly = BidirLayout<D, E>;
    using frag = typename M::frag;
    constexpr int KB = M::KB, NDT = Ly::NDT, NKD = Ly::NKD, KP = row_stride<D, E>(), EPF = M::EPF;
    constexpr int DW = NDT / 4;   // value tiles per wave
    extern __shared__ __align__(16) unsigned char smem[];
    T* Qr = reinterpret_cast<T*>(smem);                       // [CH][KP] phi(Q) rows
    float* sks = reinterpret_cast<float*>(Qr + CH * KP);      // key sums [D]

    const int bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, j = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const long nch = (L + CH - 1) / CH;
    const long c_begin = (long)blockIdx.x * cpw;
    const long c_end = c_begin + cpw < nch ? c_begin + cpw : nch;
    const unsigned char* hb = ws + (size_t)bh * Ly::head(nb);

    frag kvf[DW][NKD];   // A operands: rows = value columns of tile DW w + i, k = key
#pragma unroll
    for (int i = 0; i < DW; ++i)
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd)
            kvf[i][kd] = ld_frag<frag>(hb + Ly::kvf(nb) + (size_t)((DW * w + i) * NKD + kd) * 1024, lane);
    if (NORM && tid < D) sks[tid] = reinterpret_cast<const float*>(hb + Ly::ks(nb))[tid];

    auto rows_of = [&](long c) { return (int)(L - c * CH < CH ? L - c * CH : CH); };
    auto chunk_q = [&](long c) { return q + ((size_t)bh * L + c * CH) * D; };
    // two register sets: chunk c + 2 is loaded while chunk c + 1 is in flight and c is computed
    RowRegs<D, E> ra, rb;
    ra.load(chunk_q(c_begin), rows_of(c_begin), tid);
    if (c_begin + 1 < c_end) rb.load(chunk_q(c_begin + 1), rows_of(c_begin + 1), tid);
    auto step = [&](long c, RowRegs<D, E>& rq) {
        const long t0 = c * CH;
        const int n = rows_of(c);
        const size_t tok0 = (size_t)bh * L + t0;
        const __amdgpu_buffer_rsrc_t ors = buffer_rsrc(o + tok0 * D, n * D * (int)sizeof(T));
        if (c > c_begin) lds_sync();   // every wave is done with the previous chunk's rows
        rq.store(Qr, n, tid, Phi16<E, ELU1>());
        if (c + 2 < c_end) rq.load(chunk_q(c + 2), rows_of(c + 2), tid);
        lds_sync();
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            frag qf[NKD];   // B operands: column = token 16 rt + m, k = key
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) qf[kd] = row_frag_raw<E>(Qr + (16 * rt + m) * KP, kd * KB, j);
            float z = 1.f;
            if constexpr (NORM) {
                z = 0.f;
#pragma unroll
                for (int kd = 0; kd < NKD; ++kd)
#pragma unroll
                    for (int e = 0; e < EPF; ++e) {
                        float x;
                        if constexpr (EPF == 8) x = bf2f((uint16_t)qf[kd][e]);
                        else x = qf[kd][e];
                        z += x * sks[kd * KB + M::kofs(j, e)];
                    }
                z += __shfl_xor(z, 16);
                z += __shfl_xor(z, 32);
            }
            const int r = 16 * rt + m;   // this lane's token
            const float s = NORM ? 1.f / z : 1.f;
#pragma unroll
            for (int i = 0; i < DW; ++i) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kd = 0; kd < NKD; ++kd) acc = M::mma(kvf[i][kd], qf[kd], acc);
                // lane (j, m): o[token r][16 vt + 4 j .. + 3]; tokens past the end are dropped
                const int off = (r * D + 16 * (DW * w + i) + 4 * j) * (int)sizeof(T);
                if constexpr (sizeof(T) == 2) {
                    const i32x2 x = {(int)f2bf2(acc[0] * s, acc[1] * s), (int)f2bf2(acc[2] * s, acc[3] * s)};
                    __builtin_amdgcn_raw_buffer_store_b64(x, ors, off, 0, 0);
                } else {
                    const i32x4 x = {__float_as_int(acc[0] * s), __float_as_int(acc[1] * s),
                                     __float_as_int(acc[2] * s), __float_as_int(acc[3] * s)};
                    __builtin_amdgcn_raw_buffer_store_b128(x, ors, off, 0, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (long c = c_begin; c < c_end; c += 2) {
        step(c, ra);
        if (c + 1 < c_end) step(c + 1, rb);
    }
}

// kv_out [BH][D][D] fp32 or NULL; flags bit 0: normalise, bit 1: phi = elu + 1
template <int D, class E>
static int launch_bidir_t(const void* q, const void* k, const void* v, void* o, float* kv_out, long BH, long L,
                          int flags, unsigned char* ws, hipStream_t stream) {
    using T = typename E::T;
    constexpr int KP = row_stride<D, E>();
    const long nch = (L + CH - 1) / CH;
    const int nb = bidir_blocks(BH, nch);
    const int cpb = (int)((nch + nb - 1) / nb);
    const size_t lds_kv = (size_t)2 * CH * KP * sizeof(T) + (size_t)(D / 16) * (CH / MM<E>::KB) * 1024;
    const size_t lds_out = (size_t)CH * KP * sizeof(T) + D * 4;
    static const bool attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&bidir_kv_kernel<D, E, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_kv) == hipSuccess &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(&bidir_kv_kernel<D, E, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_kv) == hipSuccess;
    if (!attr) return -1;
    const dim3 g1((unsigned)nb, (unsigned)BH);
    if (flags & 2)
        hipLaunchKernelGGL((bidir_kv_kernel<D, E, true>), g1, dim3(256), lds_kv, stream, (const T*)k, (const T*)v, ws, L,
                           cpb, nb);
    else
        hipLaunchKernelGGL((bidir_kv_kernel<D, E, false>), g1, dim3(256), lds_kv, stream, (const T*)k, (const T*)v, ws,
                           L, cpb, nb);
    constexpr int NFR = (D / 16) * (D / MM<E>::KB);
    hipLaunchKernelGGL((bidir_reduce_kernel<D, E>), dim3((NFR + 3) / 4, (unsigned)BH), dim3(256), 0, stream, ws, kv_out,
                       nb);
    // stage 3: about 1024 workgroups, a whole number of chunks each
    long groups = (1024 + BH - 1) / BH;
    if (groups > nch) groups = nch;
    const int cpw = (int)((nch + groups - 1) / groups);
    const dim3 g3((unsigned)((nch + cpw - 1) / cpw), (unsigned)BH);
#define GDN_BIDIR_OUT(EL, NO)                                                                                       \
    hipLaunchKernelGGL((bidir_out_kernel<D, E, EL, NO>), g3, dim3(256), lds_out, stream, (const T*)q, ws, (T*)o, L, \
                       cpw, nb)
    switch (flags & 3) {
        case 0: GDN_BIDIR_OUT(false, false); break;
        case 1: GDN_BIDIR_OUT(false, true); break;
        case 2: GDN_BIDIR_OUT(true, false); break;
        default: GDN_BIDIR_OUT(true, true); break;
    }
#undef GDN_BIDIR_OUT
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

__global__ void zero_kernel(float* __restrict__ p, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

int launch_bidir(const void* q, const void* k, const void* v, void* o, float* kv_out, int BH, long L, int D,
                 int dtype, int flags, void* ws, hipStream_t stream) {
    if (L == 0) {   // no tokens: no output; KV is zero
        if (!kv_out) return 0;
        const size_t n = (size_t)BH * D * D;
        hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, kv_out, n);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    unsigned char* w = static_cast<unsigned char*>(ws);
    if (D == 128 && dtype == 0) return launch_bidir_t<128, BF16>(q, k, v, o, kv_out, BH, L, flags, w, stream);
    if (D == 128) return launch_bidir_t<128, F32>(q, k, v, o, kv_out, BH, L, flags, w, stream);
    if (dtype == 0) return launch_bidir_t<64, BF16>(q, k, v, o, kv_out, BH, L, flags, w, stream);
    return launch_bidir_t<64, F32>(q, k, v, o, kv_out, BH, L, flags, w, stream);
}

}  // namespace gdn
