// Block-parallel chunked prefill of causal linear attention, plain or with a per-token decay,
// on gfx950.
//
// The recurrence S_t = a_t S_{t-1} + v_t k_t^T, o_t = S_t q_t (the forpes.ru article on linear
// attention: its recurrent form and the decay modifications listed after it; a = 1 is the plain
// form of the AI RnD Day channel post, tgstat.ru, section "Linear attention") has a scalar
// transition, so the state at any token is a decayed sum of the chunks before it: the chunks'
// contributions can be formed in parallel and only their sums need a sequential pass. With the
// key-major state H = S^T, per chunk of C = 64 tokens and g the in-chunk inclusive prefix sum of
// log a:
//     O  = diag(e^g) Q H + (Q K^T .* Gamma) V,   Gamma[r][s] = e^{g_r - g_s} for s <= r, else 0
//     H' = e^{g_C} H + Khat^T V,                 Khat[s] = e^{g_C - g_s} k_s
// (only exponentials of non-positive differences are formed). Three kernels:
//   1. la_kv_kernel: one workgroup per (block of chunks, slice), all blocks but the last, runs H'
//      over its block from zero: S_b, the block's contribution to the state after it, and
//      Lambda_b, its summed log a.
//   2. la_scan_kernel: per slice and state element, H_0 = h0, H_{b+1} = e^{Lambda_b} H_b + S_b;
//      H_b replaces S_b in the workspace.
//   3. la_out_kernel: one workgroup per (block, slice) runs the block's chunks again from H_b and
//      forms their outputs; the last block's workgroups end with the final state and write
//      h_final. Each wave keeps the fp32 state of a quarter of the value columns in accumulator
//      registers, computes the gated causal P^T for one token tile and shares it and its quarter
//      of the Khat^T fragments through LDS.
// The products that contract over tokens (Khat^T V, V^T P^T) need fragments whose k index is the
// token: K and V rows are staged in LDS and turned into columns by one MFMA per 16 x 16 tile
// against a unit-column fragment, an exact transpose on the matrix core.
#include <stdint.h>

#include "gdn_launch.h"
#include "gdn_rows.h"

namespace gdn {

namespace {

// One block's state (or contribution) in the workspace: NDT x NDT fp32 accumulator tiles
// (d_k tile dt, value tile vt) of 64 lanes x 4, lane (j, n) holding rows 16 dt + 4 j .. + 3 of
// column 16 vt + n. The workspace holds [slices][blocks] of them, then [slices][blocks] fp32
// Lambda.
template <int D>
struct LaLayout {
    static constexpr int NDT = D / 16;
    static constexpr size_t TILES = (size_t)NDT * NDT * 1024;
};

typedef int i32x2v __attribute__((ext_vector_type(2)));
typedef int i32x4v __attribute__((ext_vector_type(4)));

template <int D, class E>
struct LaCfg {
    using T = typename E::T;
    static constexpr int KB = MM<E>::KB, NDT = D / 16, NKD = D / KB, NKT = CH / KB, FPD = KB / 16,
                         KP = row_stride<D, E>();
    static constexpr int DW = NDT / 4;                                  // value (and key) tiles per wave
    static constexpr size_t ROWS = (size_t)CH * KP * sizeof(T);         // one chunk's rows in LDS
    static constexpr size_t KF = (size_t)NDT * NKT * 1024;              // Khat^T fragments
    static constexpr size_t PF = (size_t)4 * NKT * 1024;                // P^T fragments
    static constexpr size_t LDS_KV = 2 * ROWS + KF + CH * 4;
    static constexpr size_t LDS_OUT = 3 * ROWS + KF + PF + 4 * CH * 4;
    // register prefetch of the next chunk's rows only where it fits beside the fp32 fragments
    static constexpr bool PREF = sizeof(T) == 2;
};

// transposed 16 x 16 tiles of d-tile dt of the rows R (row stride KP): lane (j, n) of t[st]
// holds R[16 st + 4 j + e][16 dt + n]
template <int D, class E>
__device__ __forceinline__ void col_tiles(const typename E::T* R, int dt, int j, int m, f32x4 (&t)[4]) {
    using C = LaCfg<D, E>;
    using M = MM<E>;
    const typename M::frag sel = unit_cols<E>(j, m, dt % C::FPD);
#pragma unroll
    for (int st = 0; st < 4; ++st)
        t[st] = M::mma(row_frag_raw<E>(R + (16 * st + m) * C::KP, C::KB * (dt / C::FPD), j), sel, f32x4{0.f, 0.f, 0.f, 0.f});
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// 1. each block's contribution to the state after it
// ---------------------------------------------------------------------------------------------
template <int D, class E, bool GATED>
__global__ __launch_bounds__(256) void la_kv_kernel(const typename E::T* __restrict__ k,
                                                    const typename E::T* __restrict__ v,
                                                    const float* __restrict__ log_alpha, unsigned char* ws, long L,
                                                    int cpb, int nb) {
    using T = typename E::T;
    using M = MM<E>;
    using C = LaCfg<D, E>;
    using frag = typename M::frag;
    constexpr int KB = C::KB, NDT = C::NDT, NKT = C::NKT, FPD = C::FPD, DW = C::DW;
    extern __shared__ __align__(16) unsigned char smem[];
    T* Kr = reinterpret_cast<T*>(smem);                                   // [CH][KP]
    T* Vr = reinterpret_cast<T*>(smem + C::ROWS);                         // [CH][KP]
    unsigned char* sKf = smem + 2 * C::ROWS;                              // Khat^T fragments [dt][kt]
    float* skh = reinterpret_cast<float*>(smem + 2 * C::ROWS + C::KF);    // e^{g_C - g}

    const int blk = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, j = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: no MFMA under a lane mask
    const long nch = (L + CH - 1) / CH;
    const long c_begin = (long)blk * cpb;
    const long c_end = c_begin + cpb < nch ? c_begin + cpb : nch;

    f32x4 acc[NDT][DW];   // contribution tiles (dt, value tile DW w + i)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < DW; ++i) acc[dt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lam = 0.f;   // the block's summed log a (the same in every lane)

    auto rows_of = [&](long c) { return (int)(L - c * CH < CH ? L - c * CH : CH); };
    RowRegs<D, E> rk, rv;
    rk.load(k + ((size_t)bh * L + c_begin * CH) * D, rows_of(c_begin), tid);
    rv.load(v + ((size_t)bh * L + c_begin * CH) * D, rows_of(c_begin), tid);
    for (long c = c_begin; c < c_end; ++c) {
        const int n = rows_of(c);
        float la = 0.f;
        if constexpr (GATED)   // through a buffer resource: no branch, so no wait for older loads
            la = floor_log_gate(__uint_as_float(buffer_load4(buffer_rsrc(log_alpha + (size_t)bh * L + c * CH, n * 4), lane * 4)));
        rk.store(Kr, n, tid);
        rv.store(Vr, n, tid);
        if (c + 1 < c_end) {   // the next chunk's rows, in flight during this one
            const size_t tok1 = (size_t)bh * L + (c + 1) * CH;
            rk.load(k + tok1 * D, rows_of(c + 1), tid);
            rv.load(v + tok1 * D, rows_of(c + 1), tid);
        }
        float gC = 0.f;
        if constexpr (GATED) {   // fp32 inputs: sums as exact hi + lo pairs (see wave_scan2)
            float glo = 0.f;
            const float g = sizeof(T) == 4 ? wave_scan2(la, glo) : wave_scan(la, lane);
            gC = wave_last(g);
            if (w == 0) skh[lane] = __expf(sizeof(T) == 4 ? (gC - g) + (wave_last(glo) - glo) : gC - g);
        }
        lds_sync();
        // this wave's key tiles -> Khat^T fragments in LDS; its value tiles -> V fragments
        frag vf[DW][NKT];
#pragma unroll
        for (int i = 0; i < DW; ++i) {
            const int dt = DW * w + i;
            if constexpr (sizeof(T) == 2) {   // bf16: gfx950's transposing LDS reads
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    const frag kr = tr_frag(Kr, C::KP, KB * kt, 16 * dt, j, m);
                    st_frag(sKf + (size_t)(dt * NKT + kt) * 1024, lane, GATED ? scale_frag(kr, skh + KB * kt, j) : kr);
                    vf[i][kt] = tr_frag(Vr, C::KP, KB * kt, 16 * dt, j, m);
                }
            } else {   // fp32: transposed on the matrix core
                f32x4 t[4];
                col_tiles<D, E>(Kr, dt, j, m, t);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
                    st_frag(sKf + (size_t)(dt * NKT + kt) * 1024, lane,
                            GATED ? cols_frag<E>(&t[FPD * kt], skh + 16 * FPD * kt, j) : cols_frag<E>(&t[FPD * kt]));
                col_tiles<D, E>(Vr, dt, j, m, t);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) vf[i][kt] = cols_frag<E>(&t[FPD * kt]);
            }
        }
        lds_sync();
        if constexpr (GATED) {
            const float dc = __expf(gC);
            lam += gC;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < DW; ++i)
                    acc[dt][i] = f32x4{acc[dt][i][0] * dc, acc[dt][i][1] * dc, acc[dt][i][2] * dc, acc[dt][i][3] * dc};
        }
        // S = e^{g_C} S + Khat^T V over this wave's value tiles
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                const frag kf = ld_frag<frag>(sKf + (size_t)(dt * NKT + kt) * 1024, lane);
#pragma unroll
                for (int i = 0; i < DW; ++i) acc[dt][i] = M::mma(kf, vf[i][kt], acc[dt][i]);
            }
    }
    unsigned char* sb = ws + ((size_t)bh * nb + blk) * LaLayout<D>::TILES;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < DW; ++i) st_frag(sb + (size_t)(dt * NDT + DW * w + i) * 1024, lane, acc[dt][i]);
    if (GATED && tid == 0) {
        float* lamb = reinterpret_cast<float*>(ws + (size_t)gridDim.y * nb * LaLayout<D>::TILES);
        lamb[(size_t)bh * nb + blk] = lam;
    }
}

// ---------------------------------------------------------------------------------------------
// 2. block-start states: a sequential pass over the blocks, one thread per state element
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void la_scan_kernel(unsigned char* ws, const float* __restrict__ h0, int nb,
                                                      int gated) {
    constexpr int NDT = D / 16;
    constexpr size_t TF = LaLayout<D>::TILES / 4;   // floats per block
    const int bh = blockIdx.y;
    const int u = blockIdx.x * 256 + threadIdx.x;   // element in tile order, < D * D
    const int e = u & 3, lane = (u >> 2) & 63, tile = u >> 8;
    const int row = 16 * (tile / NDT) + 4 * (lane >> 4) + e, col = 16 * (tile % NDT) + (lane & 15);
    float* S = reinterpret_cast<float*>(ws + (size_t)bh * nb * LaLayout<D>::TILES) + u;
    const float* lamb = reinterpret_cast<const float*>(ws + (size_t)gridDim.y * nb * LaLayout<D>::TILES) + (size_t)bh * nb;
    // h0 is read here, before stage 3 writes h_final: the two may be the same array
    float H = h0 ? h0[((size_t)bh * D + row) * D + col] : 0.f;
    for (int b = 0; b + 1 < nb; ++b) {
        const float s = S[b * TF];
        S[b * TF] = H;
        H = (gated ? __expf(lamb[b]) * H : H) + s;
    }
    S[(nb - 1) * TF] = H;   // the last block's start state (its own contribution is never formed)
}

// ---------------------------------------------------------------------------------------------
// 3. outputs from each block's start state
// ---------------------------------------------------------------------------------------------
template <int D, class E, bool GATED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void la_out_kernel(const typename E::T* __restrict__ q,
                                                     const typename E::T* __restrict__ k,
                                                     const typename E::T* __restrict__ v,
                                                     const float* __restrict__ log_alpha,
                                                     const unsigned char* __restrict__ ws, typename E::T* __restrict__ o,
                                                     float* __restrict__ h_final, long L, int cpb, int nb) {
    using T = typename E::T;
    using M = MM<E>;
    using C = LaCfg<D, E>;
    using frag = typename M::frag;
    constexpr int KB = C::KB, NDT = C::NDT, NKD = C::NKD, NKT = C::NKT, FPD = C::FPD, KP = C::KP, DW = C::DW;
    extern __shared__ __align__(16) unsigned char smem[];
    T* Qr = reinterpret_cast<T*>(smem);                                           // [CH][KP]
    T* Kr = reinterpret_cast<T*>(smem + C::ROWS);                                 // [CH][KP]
    T* Vr = reinterpret_cast<T*>(smem + 2 * C::ROWS);                             // [CH][KP]
    unsigned char* sKf = smem + 3 * C::ROWS;                                      // Khat^T fragments [dt][kt]
    unsigned char* sPf = sKf + C::KF;                                             // P^T fragments [rt][kt]
    float* sg = reinterpret_cast<float*>(sPf + C::PF);                            // g
    float* seg = sg + CH;                                                         // e^g
    float* skh = seg + CH;                                                        // e^{g_C - g}
    float* slo = skh + CH;                                                        // g's low part

    const int blk = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, j = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const long nch = (L + CH - 1) / CH;
    const long c_begin = (long)blk * cpb;
    const long c_end = c_begin + cpb < nch ? c_begin + cpb : nch;

    // the block-start state of this wave's value tiles vt = DW w + i
    f32x4 H[DW][NDT];
    const unsigned char* hb = ws + ((size_t)bh * nb + blk) * LaLayout<D>::TILES;
#pragma unroll
    for (int i = 0; i < DW; ++i)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) H[i][dt] = ld_frag<f32x4>(hb + (size_t)(dt * NDT + DW * w + i) * 1024, lane);

    auto rows_of = [&](long c) { return (int)(L - c * CH < CH ? L - c * CH : CH); };
    auto src = [&](const T* p, long c) { return p + ((size_t)bh * L + c * CH) * D; };
    RowRegs<D, E> rq, rk, rv;
    auto load_rows = [&](long c) {
        const int n = rows_of(c);
        rq.load(src(q, c), n, tid);
        rk.load(src(k, c), n, tid);
        rv.load(src(v, c), n, tid);
    };
    load_rows(c_begin);
    for (long c = c_begin; c < c_end; ++c) {
        const int n = rows_of(c);
        const size_t tok0 = (size_t)bh * L + c * CH;
        float la = 0.f;
        if constexpr (GATED)   // through a buffer resource: no branch, so no wait for older loads
            la = floor_log_gate(__uint_as_float(buffer_load4(buffer_rsrc(log_alpha + tok0, n * 4), lane * 4)));
        if (c > c_begin) lds_sync();   // every wave is done with the previous chunk's LDS data
        rq.store(Qr, n, tid);
        rk.store(Kr, n, tid);
        rv.store(Vr, n, tid);
        float gC = 0.f;
        if (C::PREF && c + 1 < c_end) load_rows(c + 1);
        if constexpr (GATED) {
            // fp32 inputs, whose bound is tight: the sums as exact hi + lo pairs, so that their
            // differences keep fp32 precision where the sums are large (see wave_scan2)
            constexpr bool PAIR = sizeof(T) == 4;
            float glo = 0.f;
            const float g = PAIR ? wave_scan2(la, glo) : wave_scan(la, lane);
            gC = wave_last(g);
            if (w == 0) {
                sg[lane] = g;
                if constexpr (PAIR) slo[lane] = glo;
                seg[lane] = __expf(PAIR ? g + glo : g);
                skh[lane] = __expf(PAIR ? (gC - g) + (wave_last(glo) - glo) : gC - g);
            }
        }
        lds_sync();
        // this wave's key tiles -> Khat^T fragments in LDS; its value tiles -> V fragments
        frag vf[DW][NKT];
#pragma unroll
        for (int i = 0; i < DW; ++i) {
            const int dt = DW * w + i;
            if constexpr (sizeof(T) == 2) {   // bf16: gfx950's transposing LDS reads
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    const frag kr = tr_frag(Kr, C::KP, KB * kt, 16 * dt, j, m);
                    st_frag(sKf + (size_t)(dt * NKT + kt) * 1024, lane, GATED ? scale_frag(kr, skh + KB * kt, j) : kr);
                    vf[i][kt] = tr_frag(Vr, C::KP, KB * kt, 16 * dt, j, m);
                }
            } else {   // fp32: transposed on the matrix core
                f32x4 t[4];
                col_tiles<D, E>(Kr, dt, j, m, t);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
                    st_frag(sKf + (size_t)(dt * NKT + kt) * 1024, lane,
                            GATED ? cols_frag<E>(&t[FPD * kt], skh + 16 * FPD * kt, j) : cols_frag<E>(&t[FPD * kt]));
                col_tiles<D, E>(Vr, dt, j, m, t);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) vf[i][kt] = cols_frag<E>(&t[FPD * kt]);
            }
        }
        // P^T for token tile rt = w: lane (j, n) of t[st] holds k_s . q_r, s = 16 st + 4 j + e,
        // r = 16 w + n, kept for s <= r and gated by e^{g_r - g_s}
        {
            f32x4 t[4];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                t[st] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (st <= w) {
#pragma unroll
                    for (int kd = 0; kd < NKD; ++kd)
                        t[st] = M::mma(row_frag_raw<E>(Kr + (16 * st + m) * KP, kd * KB, j),
                                       row_frag_raw<E>(Qr + (16 * w + m) * KP, kd * KB, j), t[st]);
                    const int r = 16 * w + m;
                    const float gr = GATED ? sg[r] : 0.f, grl = GATED && sizeof(T) == 4 ? slo[r] : 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = 16 * st + 4 * j + e;
                        const float d = sizeof(T) == 4 ? (gr - sg[s]) + (grl - slo[s]) : gr - sg[s];
                        const float x = GATED ? t[st][e] * __expf(s <= r ? d : 0.f) : t[st][e];
                        t[st][e] = s <= r ? x : 0.f;
                    }
                }
            }
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) st_frag(sPf + (size_t)(w * NKT + kt) * 1024, lane, cols_frag<E>(&t[FPD * kt]));
        }
        // the chunk-start state as A operands (rows = value columns, k = key)
        frag Hf[DW][NKD];
#pragma unroll
        for (int i = 0; i < DW; ++i)
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) Hf[i][kd] = M::from_acc(H[i], kd);
        lds_sync();
        // O^T tiles (value tile DW w + i, token tile rt) = e^g (H^T Q^T) + V^T P^T
        const __amdgpu_buffer_rsrc_t ors = buffer_rsrc(o + tok0 * D, n * D * (int)sizeof(T));
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            frag qf[NKD];
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) qf[kd] = row_frag_raw<E>(Qr + (16 * rt + m) * KP, kd * KB, j);
            frag pf[NKT];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) pf[kt] = ld_frag<frag>(sPf + (size_t)(rt * NKT + kt) * 1024, lane);
            const float egr = GATED ? seg[16 * rt + m] : 1.f;
#pragma unroll
            for (int i = 0; i < DW; ++i) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kd = 0; kd < NKD; ++kd) acc = M::mma(Hf[i][kd], qf[kd], acc);
                if constexpr (GATED) acc = f32x4{acc[0] * egr, acc[1] * egr, acc[2] * egr, acc[3] * egr};
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
                    if (kt * KB <= 16 * rt + 15) acc = M::mma(vf[i][kt], pf[kt], acc);
                // lane (j, m): o[token 16 rt + m][16 vt + 4 j .. + 3]; tokens past the end are dropped
                const int off = ((16 * rt + m) * D + 16 * (DW * w + i) + 4 * j) * (int)sizeof(T);
                if constexpr (sizeof(T) == 2) {
                    const i32x2v x = {(int)f2bf2(acc[0], acc[1]), (int)f2bf2(acc[2], acc[3])};
                    __builtin_amdgcn_raw_buffer_store_b64(x, ors, off, 0, 0);
                } else {
                    const i32x4v x = {__float_as_int(acc[0]), __float_as_int(acc[1]), __float_as_int(acc[2]),
                                      __float_as_int(acc[3])};
                    __builtin_amdgcn_raw_buffer_store_b128(x, ors, off, 0, 0);
                }
            }
        }
        // H = e^{g_C} H + Khat^T V
        if constexpr (GATED) {
            const float dc = __expf(gC);
#pragma unroll
            for (int i = 0; i < DW; ++i)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    H[i][dt] = f32x4{H[i][dt][0] * dc, H[i][dt][1] * dc, H[i][dt][2] * dc, H[i][dt][3] * dc};
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                const frag kf = ld_frag<frag>(sKf + (size_t)(dt * NKT + kt) * 1024, lane);
#pragma unroll
                for (int i = 0; i < DW; ++i) H[i][dt] = M::mma(kf, vf[i][kt], H[i][dt]);
            }
        if (!C::PREF && c + 1 < c_end) load_rows(c + 1);
    }
    if (blk == nb - 1) {   // the final state: lane (j, n) of tile (dt, vt) holds rows 16 dt + 4 j .. + 3, column 16 vt + n
        float* hf = h_final + (size_t)bh * D * D;
#pragma unroll
        for (int i = 0; i < DW; ++i)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int e = 0; e < 4; ++e) hf[(size_t)(16 * dt + 4 * j + e) * D + 16 * (DW * w + i) + m] = H[i][dt][e];
    }
}

// ---------------------------------------------------------------------------------------------
// Gated linear attention with a gate per key dimension (the forpes.ru article's survey of
// linearised models: GLA, gating over the key vectors): H_t = diag(a_t) H_{t-1} + k_t v_t^T with
// a_t in R^Dk. With G the in-chunk inclusive prefix sum of log a (a Dk-vector per token):
//     O[r]  = (q_r .* e^{G_r})^T H + sum_{s<=r} (sum_d q_r[d] k_s[d] e^{G_r[d] - G_s[d]}) v_s
//     H'    = diag(e^{G_C}) H + Khat^T V,   Khat[s][d] = k_s[d] e^{G_C[d] - G_s[d]}
// The same three stages as above, with the block decay a Dk-vector. The intra-chunk products
// take a reference token per pair of 16-token tiles: tile rt against any earlier tile uses the
// last token before rt (one scaled query operand serves all of them), so both factors
// e^{G_r - G_ref} and e^{G_ref - G_s} are at most 1. A tile against itself uses its middle token
// when the chunk's gates fall by at most GLA_WIDE across every tile (no factor above e^{GLA_WIDE});
// otherwise it is split by the highest bit in which the pair's positions differ, with a
// reference between the two tokens of every pair (gla_diag_tile), so any gates are exact.
// ---------------------------------------------------------------------------------------------
namespace {

template <int D, int NT = 256>
struct GlaCfg {
    static constexpr int GS = D + 4;                        // row stride of the cumulative gates (floats)
    static constexpr size_t GSZ = (size_t)CH * GS * 4;       // the chunk's cumulative gates
    static constexpr int NQ = NT / D, TPQ = CH / NQ;        // gate-scan threads per column, tokens each
    static constexpr size_t TOT = (size_t)NQ * D * 4;        // per-thread block totals
};

// Cumulative log gates of a chunk, sG[s][d] = sum_{s' <= s} la[s'][d] (rows past the end add
// zero). Thread t takes column d = t % D and tokens [qq TPQ, (qq + 1) TPQ), qq = t / D: load,
// local prefix and block total (then a workgroup barrier), then the earlier blocks' totals added.
template <int D, int NT = 256>
struct GateScan {
    using G = GlaCfg<D, NT>;
    float x[G::TPQ];
    __device__ __forceinline__ void load(const float* la_chunk, int n, int tid) {
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(la_chunk, n * D * 4);
        const int d = tid % D, s0 = (tid / D) * G::TPQ;
#pragma unroll
        for (int i = 0; i < G::TPQ; ++i) x[i] = __uint_as_float(buffer_load4(rs, ((s0 + i) * D + d) * 4));
    }
    __device__ __forceinline__ void prefix(float* tot, int tid) {
        x[0] = floor_log_gate(x[0]);
#pragma unroll
        for (int i = 1; i < G::TPQ; ++i) x[i] = floor_log_gate(x[i]) + x[i - 1];
        tot[tid] = x[G::TPQ - 1];   // tot[qq][d]
    }
    // whether the cumulative gate falls by more than `lim` across one of this thread's 16-token
    // tiles (after prefix; differences within the thread's tokens need no carry)
    __device__ __forceinline__ bool tile_span_over(float lim) const {
        static_assert(G::TPQ % 16 == 0, "whole tiles per thread");
        bool over = false;
#pragma unroll
        for (int i = 0; i + 15 < G::TPQ; i += 16) over = over || x[i] - x[i + 15] > lim;
        return over;
    }
    // after the barrier; returns this thread's last cumulative value (G_C[d] for the last block)
    __device__ __forceinline__ float store(float* sG, const float* tot, int tid) {
        const int d = tid % D, qq = tid / D;
        float carry = 0.f;
        for (int q2 = 0; q2 < qq; ++q2) carry += tot[q2 * D + d];
#pragma unroll
        for (int i = 0; i < G::TPQ; ++i) sG[(qq * G::TPQ + i) * G::GS + d] = x[i] + carry;
        return x[G::TPQ - 1] + carry;
    }
};

// Khat^T fragment (k = token s = s0 + kofs(j, e), column d = 16 dt + m) of a per-key-dimension
// gated chunk from K's transposed bf16 fragment: k_s[d] e^{G_C[d] - G_s[d]} (gcd = G_C[d], sG the
// cumulative gates, row stride GS), multiplied in fp32 and rounded once.
template <int D, int GS>
__device__ __forceinline__ bf16x8 khat_frag(const bf16x8& kr, const float* sG, float gcd, int s0, int dt, int j, int m) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        x[e] = bf2f((uint16_t)kr[e]) * __expf(gcd - sG[(s0 + MM<BF16>::kofs(j, e)) * GS + 16 * dt + m]);
    return MM<BF16>::pack(x);
}

// Fragment of row rp (k = d, the row_frag_raw order) with element d scaled by exp(gp[d] - gq[d])
// (gq == nullptr: exp(gp[d])).
template <class E>
__device__ __forceinline__ typename MM<E>::frag row_frag_exp(const typename E::T* rp, const float* gp, const float* gq,
                                                            int k0, int j) {
    using M = MM<E>;
    float x[M::EPF];
#pragma unroll
    for (int h = 0; h < M::EPF / 4; ++h) {
        const int d0 = k0 + 16 * h + 4 * j;
        const float4 a = load4(rp + d0);
        const float4 p = *reinterpret_cast<const float4*>(gp + d0);
        float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
        if (gq) r = *reinterpret_cast<const float4*>(gq + d0);
        x[4 * h + 0] = a.x * __expf(p.x - r.x);
        x[4 * h + 1] = a.y * __expf(p.y - r.y);
        x[4 * h + 2] = a.z * __expf(p.z - r.z);
        x[4 * h + 3] = a.w * __expf(p.w - r.w);
    }
    return M::pack(x);
}

// Largest fall of the cumulative log gates across a 16-token tile for which a diagonal tile is
// formed in one product against its middle token (operand factors up to e^{64}).
constexpr float GLA_WIDE = 64.f;

// P^T tile of a 16-token tile against itself (lane (j, n): key s = 4 j + e, query r = n of the
// tile, s <= r), with no factor above 1 whatever the gates. A pair s < r is taken by the pass b
// (8, 4, 2, 1) of the highest bit in which s and r differ: s in the first and r in the second
// half of a group of 2b tokens. Pass b scales each key row in a first half by e^{G_ref - G_s} and
// each query row in a second half by e^{G_r - G_ref}, ref the last token of the group's first half
// (s <= ref < r); the other rows are zero (selected, not multiplied) and the product's entries
// outside the pass's pairs are dropped. The diagonal s = r is q_r . k_r.
template <class E, int D, int KP, int GS>
__device__ __forceinline__ f32x4 gla_diag_tile(const typename E::T* Kr, const typename E::T* Qr, const float* sG,
                                               int tile, int j, int m) {
    using M = MM<E>;
    using frag = typename M::frag;
    constexpr int KB = M::KB, NKD = D / KB;
    const int r0 = 16 * tile;
    const typename E::T* kr = Kr + (r0 + m) * KP;   // key row m (A operand row m)
    const typename E::T* qr = Qr + (r0 + m) * KP;   // query row m (B operand column m)
    const float* gm = sG + (r0 + m) * GS;
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    {
        f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) p = M::mma(row_frag_raw<E>(kr, kd * KB, j), row_frag_raw<E>(qr, kd * KB, j), p);
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = 4 * j + e == m ? p[e] : 0.f;
    }
#pragma unroll
    for (int b = 8; b >= 1; b >>= 1) {
        __builtin_amdgcn_sched_barrier(0);   // one pass's operands at a time
        const bool first = (m % (2 * b)) < b;                     // row m in the first half of its group
        const float* gref = sG + (r0 + m - m % (2 * b) + b - 1) * GS;
        f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) {
            const frag kf = row_frag_exp<E>(kr, gref, gm, kd * KB, j);   // e^{G_ref - G_s}, key rows in first halves
            const frag qf = row_frag_exp<E>(qr, gm, gref, kd * KB, j);   // e^{G_r - G_ref}, query rows in second halves
            p = M::mma(first ? kf : frag{}, first ? frag{} : qf, p);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = 4 * j + e;
            const bool pair = s / (2 * b) == m / (2 * b) && s % (2 * b) < b && m % (2 * b) >= b;
            t[e] += pair ? p[e] : 0.f;
        }
    }
    return t;
}

}  // namespace

// 1. block contributions (all blocks but the last) and their Dk-vector of summed log gates
template <int D, class E>
__global__ __launch_bounds__(256) void gla_kv_kernel(const typename E::T* __restrict__ k,
                                                     const typename E::T* __restrict__ v,
                                                     const float* __restrict__ log_alpha, unsigned char* ws, long L,
                                                     int cpb, int nb) {
    using T = typename E::T;
    using M = MM<E>;
    using C = LaCfg<D, E>;
    using G = GlaCfg<D>;
    using frag = typename M::frag;
    constexpr int NDT = C::NDT, NKT = C::NKT, FPD = C::FPD, DW = C::DW, GS = G::GS;
    extern __shared__ __align__(16) unsigned char smem[];
    T* Kr = reinterpret_cast<T*>(smem);                                        // [CH][KP]
    T* Vr = reinterpret_cast<T*>(smem + C::ROWS);                              // [CH][KP]
    unsigned char* sKf = smem + 2 * C::ROWS;                                   // Khat^T fragments [dt][kt]
    float* sG = reinterpret_cast<float*>(smem + 2 * C::ROWS + C::KF);          // [CH][GS] cumulative gates
    float* sTot = reinterpret_cast<float*>(smem + 2 * C::ROWS + C::KF + G::GSZ);

    const int blk = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, j = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const long nch = (L + CH - 1) / CH;
    const long c_begin = (long)blk * cpb;
    const long c_end = c_begin + cpb < nch ? c_begin + cpb : nch;

    f32x4 acc[NDT][DW];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < DW; ++i) acc[dt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lamv = 0.f;   // summed log gate of column tid % D (kept by the last token block's threads)

    auto rows_of = [&](long c) { return (int)(L - c * CH < CH ? L - c * CH : CH); };
    RowRegs<D, E> rk, rv;
    rk.load(k + ((size_t)bh * L + c_begin * CH) * D, rows_of(c_begin), tid);
    rv.load(v + ((size_t)bh * L + c_begin * CH) * D, rows_of(c_begin), tid);
    GateScan<D> gsc;
    gsc.load(log_alpha + ((size_t)bh * L + c_begin * CH) * D, rows_of(c_begin), tid);
    for (long c = c_begin; c < c_end; ++c) {
        const int n = rows_of(c);
        const size_t tok0 = (size_t)bh * L + c * CH;
        rk.store(Kr, n, tid);
        rv.store(Vr, n, tid);
        if (c + 1 < c_end) {
            rk.load(k + (tok0 + CH) * D, rows_of(c + 1), tid);
            rv.load(v + (tok0 + CH) * D, rows_of(c + 1), tid);
        }
        gsc.prefix(sTot, tid);
        lds_sync();
        lamv += gsc.store(sG, sTot, tid);
        if (c + 1 < c_end) gsc.load(log_alpha + (tok0 + CH) * D, rows_of(c + 1), tid);
        lds_sync();
        const float* gC = sG + (CH - 1) * GS;
        frag vf[DW][NKT];
#pragma unroll
        for (int i = 0; i < DW; ++i) {
            const int dt = DW * w + i;
            const float gcd = gC[16 * dt + m];
            if constexpr (sizeof(T) == 2) {   // bf16: gfx950's transposing LDS reads
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    st_frag(sKf + (size_t)(dt * NKT + kt) * 1024, lane,
                            khat_frag<D, GS>(tr_frag(Kr, C::KP, C::KB * kt, 16 * dt, j, m), sG, gcd, C::KB * kt, dt, j, m));
                    vf[i][kt] = tr_frag(Vr, C::KP, C::KB * kt, 16 * dt, j, m);
                }
            } else {
                f32x4 t[4];
                col_tiles<D, E>(Kr, dt, j, m, t);
#pragma unroll
                for (int st = 0; st < 4; ++st)
#pragma unroll
                    for (int e = 0; e < 4; ++e) t[st][e] *= __expf(gcd - sG[(16 * st + 4 * j + e) * GS + 16 * dt + m]);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) st_frag(sKf + (size_t)(dt * NKT + kt) * 1024, lane, cols_frag<E>(&t[FPD * kt]));
                col_tiles<D, E>(Vr, dt, j, m, t);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) vf[i][kt] = cols_frag<E>(&t[FPD * kt]);
            }
        }
        lds_sync();
        // S = diag(e^{G_C}) S + Khat^T V; tile (dt, .) rows 16 dt + 4 j + e
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const float4 gc = *reinterpret_cast<const float4*>(gC + 16 * dt + 4 * j);
            const float f[4] = {__expf(gc.x), __expf(gc.y), __expf(gc.z), __expf(gc.w)};
#pragma unroll
            for (int i = 0; i < DW; ++i)
                acc[dt][i] = f32x4{acc[dt][i][0] * f[0], acc[dt][i][1] * f[1], acc[dt][i][2] * f[2], acc[dt][i][3] * f[3]};
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                const frag kf = ld_frag<frag>(sKf + (size_t)(dt * NKT + kt) * 1024, lane);
#pragma unroll
                for (int i = 0; i < DW; ++i) acc[dt][i] = M::mma(kf, vf[i][kt], acc[dt][i]);
            }
    }
    unsigned char* sb = ws + ((size_t)bh * nb + blk) * LaLayout<D>::TILES;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < DW; ++i) st_frag(sb + (size_t)(dt * NDT + DW * w + i) * 1024, lane, acc[dt][i]);
    if (tid / D == G::NQ - 1) {   // the threads that hold the chunks' last cumulative gates
        float* lamb = reinterpret_cast<float*>(ws + (size_t)gridDim.y * nb * LaLayout<D>::TILES);
        lamb[((size_t)bh * nb + blk) * D + tid % D] = lamv;
    }
}

// 2. block-start states with Dk-vector block decays
template <int D>
__global__ __launch_bounds__(256) void gla_scan_kernel(unsigned char* ws, const float* __restrict__ h0, int nb) {
    constexpr int NDT = D / 16;
    constexpr size_t TF = LaLayout<D>::TILES / 4;
    const int bh = blockIdx.y;
    const int u = blockIdx.x * 256 + threadIdx.x;
    const int e = u & 3, lane = (u >> 2) & 63, tile = u >> 8;
    const int row = 16 * (tile / NDT) + 4 * (lane >> 4) + e, col = 16 * (tile % NDT) + (lane & 15);
    float* S = reinterpret_cast<float*>(ws + (size_t)bh * nb * LaLayout<D>::TILES) + u;
    const float* lamb = reinterpret_cast<const float*>(ws + (size_t)gridDim.y * nb * LaLayout<D>::TILES) + (size_t)bh * nb * D;
    float H = h0 ? h0[((size_t)bh * D + row) * D + col] : 0.f;   // before stage 3 writes h_final
    for (int b = 0; b + 1 < nb; ++b) {
        const float s = S[b * TF];
        S[b * TF] = H;
        H = __expf(lamb[(size_t)b * D + row]) * H + s;
    }
    S[(nb - 1) * TF] = H;
}

// 3. outputs from each block's start state; the last block writes h_final. At d = 128 its LDS
// (the cumulative gates beside the rows) allows one workgroup per CU, which therefore has eight
// waves (NW = 8: one value tile each, two per SIMD) rather than four.
template <int D, class E, int NW>
__global__ __launch_bounds__(64 * NW) void gla_out_kernel(
    const typename E::T* __restrict__ q, const typename E::T* __restrict__ k, const typename E::T* __restrict__ v,
    const float* __restrict__ log_alpha, const unsigned char* __restrict__ ws, typename E::T* __restrict__ o,
    float* __restrict__ h_final, long L, int cpb, int nb) {
    using T = typename E::T;
    using M = MM<E>;
    using C = LaCfg<D, E>;
    constexpr int NT = 64 * NW;
    using G = GlaCfg<D, NT>;
    using frag = typename M::frag;
    constexpr int KB = C::KB, NDT = C::NDT, NKD = C::NKD, NKT = C::NKT, FPD = C::FPD, KP = C::KP, GS = G::GS;
    constexpr int DW = NDT / NW;        // value and key tiles per wave
    constexpr int SPW = 16 / NW;        // key tiles of P per wave (all four with four waves, two with eight)
    static_assert(DW >= 1 && NDT % NW == 0 && (NW == 4 || NW == 8), "waves");
    extern __shared__ __align__(16) unsigned char smem[];
    T* Qr = reinterpret_cast<T*>(smem);
    T* Kr = reinterpret_cast<T*>(smem + C::ROWS);
    T* Vr = reinterpret_cast<T*>(smem + 2 * C::ROWS);
    unsigned char* sKf = smem + 3 * C::ROWS;
    unsigned char* sPf = sKf + C::KF;
    float* sTot = reinterpret_cast<float*>(sPf + C::PF);
    // the cumulative gates take the V rows' space once V is in registers (fp32), else their own
    float* sG = sizeof(T) == 4 ? reinterpret_cast<float*>(Vr) : reinterpret_cast<float*>(sPf + C::PF + G::TOT);

    const int blk = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, j = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // per chunk parity: set when a 16-token tile's cumulative gates span more than WIDE in some
    // key dimension; the diagonal tiles then take the exact pass-by-pass form
    __shared__ unsigned s_wide[2];
    if (tid == 0) s_wide[0] = s_wide[1] = 0u;
    const long nch = (L + CH - 1) / CH;
    const long c_begin = (long)blk * cpb;
    const long c_end = c_begin + cpb < nch ? c_begin + cpb : nch;

    f32x4 H[DW][NDT];
    const unsigned char* hb = ws + ((size_t)bh * nb + blk) * LaLayout<D>::TILES;
#pragma unroll
    for (int i = 0; i < DW; ++i)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) H[i][dt] = ld_frag<f32x4>(hb + (size_t)(dt * NDT + DW * w + i) * 1024, lane);

    auto rows_of = [&](long c) { return (int)(L - c * CH < CH ? L - c * CH : CH); };
    auto src = [&](const T* p, long c) { return p + ((size_t)bh * L + c * CH) * D; };
    RowRegs<D, E, NT> rq, rk, rv;
    auto load_rows = [&](long c) {
        const int n = rows_of(c);
        rq.load(src(q, c), n, tid);
        rk.load(src(k, c), n, tid);
        rv.load(src(v, c), n, tid);
    };
    load_rows(c_begin);
    GateScan<D, NT> gsc;
    gsc.load(log_alpha + ((size_t)bh * L + c_begin * CH) * D, rows_of(c_begin), tid);
    for (long c = c_begin; c < c_end; ++c) {
        const int n = rows_of(c);
        const size_t tok0 = (size_t)bh * L + c * CH;
        if (c > c_begin) lds_sync();   // every wave is done with the previous chunk's LDS data
        rq.store(Qr, n, tid);
        rk.store(Kr, n, tid);
        rv.store(Vr, n, tid);
        gsc.prefix(sTot, tid);
        lds_sync();
        // V fragments (k = token) into registers; V rows are not read after this
        frag vf[DW][NKT];
#pragma unroll
        for (int i = 0; i < DW; ++i) {
            if constexpr (sizeof(T) == 2) {   // bf16: gfx950's transposing LDS reads
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) vf[i][kt] = tr_frag(Vr, KP, KB * kt, 16 * (DW * w + i), j, m);
            } else {
                f32x4 t[4];
                col_tiles<D, E>(Vr, DW * w + i, j, m, t);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) vf[i][kt] = cols_frag<E>(&t[FPD * kt]);
            }
        }
        lds_sync();
        if (gsc.tile_span_over(GLA_WIDE)) s_wide[c & 1] = 1u;
        gsc.store(sG, sTot, tid);
        if (c + 1 < c_end) gsc.load(log_alpha + (tok0 + CH) * D, rows_of(c + 1), tid);
        lds_sync();
        const bool wide = __builtin_amdgcn_readfirstlane(s_wide[c & 1]) != 0u;   // scalar
        if (tid == 0) s_wide[(c + 1) & 1] = 0u;   // every wave read it in the previous chunk
        const float* gC = sG + (CH - 1) * GS;
        // Khat^T fragments of this wave's key tiles
#pragma unroll
        for (int i = 0; i < DW; ++i) {
            const int dt = DW * w + i;
            const float gcd = gC[16 * dt + m];
            if constexpr (sizeof(T) == 2) {   // bf16: gfx950's transposing LDS reads
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
                    st_frag(sKf + (size_t)(dt * NKT + kt) * 1024, lane,
                            khat_frag<D, GS>(tr_frag(Kr, KP, KB * kt, 16 * dt, j, m), sG, gcd, KB * kt, dt, j, m));
            } else {
                f32x4 t[4];
                col_tiles<D, E>(Kr, dt, j, m, t);
#pragma unroll
                for (int st = 0; st < 4; ++st)
#pragma unroll
                    for (int e = 0; e < 4; ++e) t[st][e] *= __expf(gcd - sG[(16 * st + 4 * j + e) * GS + 16 * dt + m]);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) st_frag(sKf + (size_t)(dt * NKT + kt) * 1024, lane, cols_frag<E>(&t[FPD * kt]));
            }
        }
        // P^T of token tile rt = w % 4, key tiles [SPW h, SPW h + SPW) (h = w / 4): lane (j, n) of
        // t[st] holds sum_d k_s[d] q_r[d] e^{G_r[d] - G_s[d]}, s = 16 st + 4 j + e, r = 16 rt + n,
        // kept for s <= r. Both operands are scaled against a reference token between s and r: for
        // the tiles before the diagonal the last token before tile rt (so the query operand is
        // shared by them), on the diagonal per pass of gla_diag_tile.
        {
            const int rt_w = w & 3, st0 = SPW * (w >> 2);
            const float* gq = sG + (16 * rt_w + m) * GS;    // this lane's query row (B operand column m)
            f32x4 t[4];
            frag qo[NKD];
            if (st0 < rt_w) {
                const float* gb = sG + (16 * rt_w - 1) * GS;
#pragma unroll
                for (int kd = 0; kd < NKD; ++kd) qo[kd] = row_frag_exp<E>(Qr + (16 * rt_w + m) * KP, gq, gb, kd * KB, j);
            }
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                t[st] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (st < st0 || st >= st0 + SPW) continue;
                const float* gk = sG + (16 * st + m) * GS;   // this lane's key row (A operand row m)
                if (st < rt_w) {
                    const float* gb = sG + (16 * rt_w - 1) * GS;
#pragma unroll
                    for (int kd = 0; kd < NKD; ++kd)
                        t[st] = M::mma(row_frag_exp<E>(Kr + (16 * st + m) * KP, gb, gk, kd * KB, j), qo[kd], t[st]);
                } else if (st == rt_w) {
                    if (wide) {
                        t[st] = gla_diag_tile<E, D, KP, GS>(Kr, Qr, sG, st, j, m);
                    } else {
                        // one product against the tile's middle token: no factor exceeds
                        // e^{GLA_WIDE} (finite, and the pair's two factors multiply to at most 1)
                        const float* gref = sG + (16 * st + 7) * GS;
#pragma unroll
                        for (int kd = 0; kd < NKD; ++kd)
                            t[st] = M::mma(row_frag_exp<E>(Kr + (16 * st + m) * KP, gref, gk, kd * KB, j),
                                           row_frag_exp<E>(Qr + (16 * rt_w + m) * KP, gq, gref, kd * KB, j), t[st]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) t[st][e] = 16 * st + 4 * j + e <= 16 * rt_w + m ? t[st][e] : 0.f;
                    }
                }
            }
            // the fragments whose key tiles this wave owns (FPD tiles each)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
                if (FPD * kt >= st0 && FPD * kt < st0 + SPW)
                    st_frag(sPf + (size_t)(rt_w * NKT + kt) * 1024, lane, cols_frag<E>(&t[FPD * kt]));
        }
        // Q rows scaled by e^{G_r}, in place, 64 / NW rows per wave. With four waves a wave's rows
        // are those of its own P tile, which no other wave reads; with eight, two waves read each
        // tile's query rows, so all of P is formed first.
        if constexpr (NW == 8) lds_sync();
        {
            constexpr int RPW = 64 / NW, LPR = 64 / RPW;
            const int r = RPW * w + lane / LPR;
            T* qp = Qr + r * KP;
            const float* gp = sG + r * GS;
#pragma unroll
            for (int i = 0; i < D / (4 * LPR); ++i) {
                const int d0 = 4 * (lane % LPR + LPR * i);
                const float4 a = load4(qp + d0);
                const float4 g = *reinterpret_cast<const float4*>(gp + d0);
                store4(qp + d0, make_float4(a.x * __expf(g.x), a.y * __expf(g.y), a.z * __expf(g.z), a.w * __expf(g.w)));
            }
        }
        frag Hf[DW][NKD];
#pragma unroll
        for (int i = 0; i < DW; ++i)
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) Hf[i][kd] = M::from_acc(H[i], kd);
        lds_sync();
        // O^T = H^T (Q .* e^G)^T + V^T P^T
        const __amdgpu_buffer_rsrc_t ors = buffer_rsrc(o + tok0 * D, n * D * (int)sizeof(T));
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            frag qf[NKD];
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) qf[kd] = row_frag_raw<E>(Qr + (16 * rt + m) * KP, kd * KB, j);
            frag pf[NKT];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) pf[kt] = ld_frag<frag>(sPf + (size_t)(rt * NKT + kt) * 1024, lane);
#pragma unroll
            for (int i = 0; i < DW; ++i) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kd = 0; kd < NKD; ++kd) acc = M::mma(Hf[i][kd], qf[kd], acc);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
                    if (kt * KB <= 16 * rt + 15) acc = M::mma(vf[i][kt], pf[kt], acc);
                const int off = ((16 * rt + m) * D + 16 * (DW * w + i) + 4 * j) * (int)sizeof(T);
                if constexpr (sizeof(T) == 2) {
                    const i32x2v x = {(int)f2bf2(acc[0], acc[1]), (int)f2bf2(acc[2], acc[3])};
                    __builtin_amdgcn_raw_buffer_store_b64(x, ors, off, 0, 0);
                } else {
                    const i32x4v x = {__float_as_int(acc[0]), __float_as_int(acc[1]), __float_as_int(acc[2]),
                                      __float_as_int(acc[3])};
                    __builtin_amdgcn_raw_buffer_store_b128(x, ors, off, 0, 0);
                }
            }
        }
        // H = diag(e^{G_C}) H + Khat^T V
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const float4 gc = *reinterpret_cast<const float4*>(gC + 16 * dt + 4 * j);
            const float f[4] = {__expf(gc.x), __expf(gc.y), __expf(gc.z), __expf(gc.w)};
#pragma unroll
            for (int i = 0; i < DW; ++i)
                H[i][dt] = f32x4{H[i][dt][0] * f[0], H[i][dt][1] * f[1], H[i][dt][2] * f[2], H[i][dt][3] * f[3]};
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                const frag kf = ld_frag<frag>(sKf + (size_t)(dt * NKT + kt) * 1024, lane);
#pragma unroll
                for (int i = 0; i < DW; ++i) H[i][dt] = M::mma(kf, vf[i][kt], H[i][dt]);
            }
        if (c + 1 < c_end) load_rows(c + 1);
    }
    if (blk == nb - 1) {
        float* hf = h_final + (size_t)bh * D * D;
#pragma unroll
        for (int i = 0; i < DW; ++i)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int e = 0; e < 4; ++e) hf[(size_t)(16 * dt + 4 * j + e) * D + 16 * (DW * w + i) + m] = H[i][dt][e];
    }
}

// ---------------------------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------------------------
namespace {

// blocks of chunks per slice: about 512 workgroups for stages 1 and 3 (two per CU), no more than the
// workspace holds at `per_block` bytes per block and slice (at least one: the smallest workspace
// accepted holds one block's state tiles and summed log gates per slice)
int la_blocks(long BH, long nch, size_t per_block, size_t ws_bytes) {
    long nb = (512 + BH - 1) / BH;
    if (nb > nch) nb = nch;
    const long fit = (long)(ws_bytes / ((size_t)BH * per_block));
    if (nb > fit) nb = fit;
    if (nb < 1) nb = 1;
    const long cpb = (nch + nb - 1) / nb;
    return (int)((nch + cpb - 1) / cpb);
}

}  // namespace

static size_t la_tiles(int D) { return D == 128 ? LaLayout<128>::TILES : LaLayout<64>::TILES; }

size_t linattn_workspace_bytes(long BH, long L, int D) {
    if (L <= 0) return 0;
    const long nch = (L + CH - 1) / CH;
    return (size_t)BH * la_blocks(BH, nch, la_tiles(D) + 4, ~(size_t)0) * (la_tiles(D) + 4);
}

size_t linattn_workspace_min_bytes(long BH, long L, int D) {
    return L <= 0 ? 0 : (size_t)BH * (la_tiles(D) + 4);
}

template <int D, class E, bool GATED>
static int launch_linattn_t(const void* q, const void* k, const void* v, const float* log_alpha, const float* h0,
                            void* o, float* h_final, long BH, long L, unsigned char* ws, size_t ws_bytes,
                            hipStream_t stream) {
    using T = typename E::T;
    using C = LaCfg<D, E>;
    const long nch = (L + CH - 1) / CH;
    const int nb = la_blocks(BH, nch, LaLayout<D>::TILES + 4, ws_bytes);
    if ((size_t)BH * nb * (LaLayout<D>::TILES + 4) > ws_bytes) return -1;
    const int cpb = (int)((nch + nb - 1) / nb);
    static const bool attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&la_kv_kernel<D, E, GATED>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_KV) == hipSuccess &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(&la_out_kernel<D, E, GATED>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_OUT) == hipSuccess;
    if (!attr) return -1;
    const dim3 grid((unsigned)nb, (unsigned)BH);
    if (nb > 1)   // every block's contribution but the last one's
        hipLaunchKernelGGL((la_kv_kernel<D, E, GATED>), dim3((unsigned)(nb - 1), (unsigned)BH), dim3(256), C::LDS_KV,
                           stream, (const T*)k, (const T*)v, log_alpha, ws, L, cpb, nb);
    hipLaunchKernelGGL((la_scan_kernel<D>), dim3(D * D / 256, (unsigned)BH), dim3(256), 0, stream, ws, h0, nb,
                       GATED ? 1 : 0);
    hipLaunchKernelGGL((la_out_kernel<D, E, GATED>), grid, dim3(256), C::LDS_OUT, stream, (const T*)q, (const T*)k,
                       (const T*)v, log_alpha, (const unsigned char*)ws, (T*)o, h_final, L, cpb, nb);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// per-key-dimension gated linear attention: state tiles and a Dk-vector of summed log gates per block
size_t gla_workspace_bytes(long BH, long L, int D) {
    if (L <= 0) return 0;
    const long nch = (L + CH - 1) / CH;
    const size_t per = la_tiles(D) + (size_t)4 * D;
    return (size_t)BH * la_blocks(BH, nch, per, ~(size_t)0) * per;
}

size_t gla_workspace_min_bytes(long BH, long L, int D) {
    return L <= 0 ? 0 : (size_t)BH * (la_tiles(D) + (size_t)4 * D);
}

template <int D, class E>
static int launch_gla_t(const void* q, const void* k, const void* v, const float* log_alpha, const float* h0,
                        void* o, float* h_final, long BH, long L, unsigned char* ws, size_t ws_bytes,
                        hipStream_t stream) {
    using T = typename E::T;
    using C = LaCfg<D, E>;
    using G = GlaCfg<D>;
    constexpr int NWO = D == 128 ? 8 : 4;   // waves of the output stage
    using GO = GlaCfg<D, 64 * NWO>;
    constexpr size_t LDS_KV = 2 * C::ROWS + C::KF + G::GSZ + G::TOT;
    constexpr size_t LDS_OUT = 3 * C::ROWS + C::KF + C::PF + GO::TOT + (sizeof(T) == 2 ? G::GSZ : 0);
    static_assert(sizeof(T) == 2 || C::ROWS >= G::GSZ, "the cumulative gates fit in the V rows' space");
    static_assert(LDS_KV <= 160 * 1024 && LDS_OUT <= 160 * 1024, "LDS");
    const long nch = (L + CH - 1) / CH;
    const size_t per = LaLayout<D>::TILES + (size_t)4 * D;
    const int nb = la_blocks(BH, nch, per, ws_bytes);
    if ((size_t)BH * nb * per > ws_bytes) return -1;
    const int cpb = (int)((nch + nb - 1) / nb);
    static const bool attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&gla_kv_kernel<D, E>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_KV) == hipSuccess &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(&gla_out_kernel<D, E, NWO>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_OUT) == hipSuccess;
    if (!attr) return -1;
    if (nb > 1)
        hipLaunchKernelGGL((gla_kv_kernel<D, E>), dim3((unsigned)(nb - 1), (unsigned)BH), dim3(256), LDS_KV, stream,
                           (const T*)k, (const T*)v, log_alpha, ws, L, cpb, nb);
    hipLaunchKernelGGL((gla_scan_kernel<D>), dim3(D * D / 256, (unsigned)BH), dim3(256), 0, stream, ws, h0, nb);
    hipLaunchKernelGGL((gla_out_kernel<D, E, NWO>), dim3((unsigned)nb, (unsigned)BH), dim3(64 * NWO), LDS_OUT, stream,
                       (const T*)q, (const T*)k, (const T*)v, log_alpha, (const unsigned char*)ws, (T*)o, h_final, L,
                       cpb, nb);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gla(const void* q, const void* k, const void* v, const float* log_alpha, const float* h0, void* o,
               float* h_final, int BH, long L, int D, int dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
    unsigned char* w = static_cast<unsigned char*>(ws);
    if (D == 128 && dtype == 0) return launch_gla_t<128, BF16>(q, k, v, log_alpha, h0, o, h_final, BH, L, w, ws_bytes, stream);
    if (D == 128) return launch_gla_t<128, F32>(q, k, v, log_alpha, h0, o, h_final, BH, L, w, ws_bytes, stream);
    if (dtype == 0) return launch_gla_t<64, BF16>(q, k, v, log_alpha, h0, o, h_final, BH, L, w, ws_bytes, stream);
    return launch_gla_t<64, F32>(q, k, v, log_alpha, h0, o, h_final, BH, L, w, ws_bytes, stream);
}

int launch_linattn(const void* q, const void* k, const void* v, const float* log_alpha, const float* h0, void* o,
                   float* h_final, int BH, long L, int D, int dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
    unsigned char* w = static_cast<unsigned char*>(ws);
#define GDN_LA(DD, EE)                                                                                          \
    return log_alpha ? launch_linattn_t<DD, EE, true>(q, k, v, log_alpha, h0, o, h_final, BH, L, w, ws_bytes, stream) \
                     : launch_linattn_t<DD, EE, false>(q, k, v, nullptr, h0, o, h_final, BH, L, w, ws_bytes, stream)
    if (D == 128 && dtype == 0) GDN_LA(128, BF16);
    if (D == 128) GDN_LA(128, F32);
    if (dtype == 0) GDN_LA(64, BF16);
    GDN_LA(64, F32);
#undef GDN_LA
}

}  // namespace gdn
