// Chunked prefill of the gated delta rule (and of plain causal linear attention) on gfx950.
//
// The SparseGDN article (fileenergy.com, section "Why GDN prefill is expensive") splits chunked
// GDN prefill into three sources of work: the intra-chunk delta-system solve, the sequential
// chunk-to-chunk state pass for each head, and the outputs computed from every chunk's start
// state. The three kernels below are those three stages.
//
// Per chunk of C = 64 tokens, with g the inclusive cumulative log-gate (restarting at each
// chunk) and the key-major state H (Dk x Dv) at chunk start, the token recurrence
//     H_r = a_r (I - beta_r k_r k_r^T) H_{r-1} + beta_r k_r v_r^T
// unrolls to (exactly, up to rounding):
//     A[r][s] = beta_r exp(g_r - g_s) k_r.k_s  (s < r),     T = (I + A)^-1
//     W = T diag(beta e^g) K,   Ut = T diag(beta) V,        U = Ut - W H
//     O = diag(e^g) Q H + P U,  P[r][s] = exp(g_r - g_s) q_r.k_s  (s <= r)
//     H' = e^{g_C} H + Khat^T U,  Khat[s] = exp(g_C - g_s) k_s
// i.e. the affine chunk map H' = A_c H + B_c of the article's skip-scan illustration
// (section on embedding the selector into FLA) with A_c = e^{g_C} I - Khat^T W, B_c = Khat^T Ut.
// Only exponentials of non-positive differences are ever formed, so strong gates underflow to
// exact zeros instead of overflowing.
//
//   prep_kernel   (one workgroup per chunk and head, fully parallel): g, A, T by forward
//                 substitution in LDS, -W, Khat^T and Ut, written as MFMA-ready fragments.
//   chain_kernel  (one wave per head and 16 value columns): the sequential pass. The fp32
//                 state slice stays in accumulator registers for the whole sequence; per chunk
//                 it emits the chunk-start state and U as fragments for the output stage.
//   output_kernel (one workgroup per chunk and head): P = (Q K^T) gated and masked, then
//                 O^T = H^T (e^g Q)^T + U^T P^T, stored four value columns per lane.
// Plain linear attention uses the same kernels with T = I, W = 0, Ut = V, g = 0.
#include "gdn_mfma.h"
#include "gdn_launch.h"

namespace gdn {

// ---------------------------------------------------------------------------------------------
// workspace records
// ---------------------------------------------------------------------------------------------
template <int D, class E>
struct Layout {
    using M = MM<E>;
    static constexpr int KB = M::KB;
    static constexpr int NKD = D / KB;   // fragments along d
    static constexpr int NKT = CH / KB;  // fragments along the chunk's tokens
    static constexpr int NDT = D / 16;   // 16-wide tiles along d
    static constexpr int FR = 1024;      // bytes per fragment
    // prep record: -W [rt 4][NKD], Khat^T [dt NDT][NKT], Ut accumulators [vt NDT][rt 4][lane] (4 x T), decay
    static constexpr size_t A_W = 0;
    static constexpr size_t A_KH = A_W + (size_t)4 * NKD * FR;
    static constexpr size_t A_UT = A_KH + (size_t)NDT * NKT * FR;
    static constexpr size_t A_DEC = A_UT + (size_t)NDT * 4 * 64 * 4 * sizeof(typename E::T);
    static constexpr size_t REC_A = (A_DEC + 4 + 255) / 256 * 256;
    // chain record: chunk-start state [cg NDT][NKD], U [cg NDT][NKT]
    static constexpr size_t B_H = 0;
    static constexpr size_t B_U = (size_t)NDT * NKD * FR;
    static constexpr size_t REC_B = B_U + (size_t)NDT * NKT * FR;
    static constexpr size_t REC = REC_A + REC_B;
};

size_t prefill_workspace_bytes(long BH, long L, int D, int dtype) {
    const long nchunks = (L + CH - 1) / CH;
    size_t rec = 0;
    if (D == 128 && dtype == 0) rec = Layout<128, BF16>::REC;
    else if (D == 128) rec = Layout<128, F32>::REC;
    else if (D == 64 && dtype == 0) rec = Layout<64, BF16>::REC;
    else rec = Layout<64, F32>::REC;
    return (size_t)BH * nchunks * rec;
}

struct PrefArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* beta;
    const float* log_alpha;
    const float* h0;
    void* o;
    float* h_final;
    unsigned char* ws;
    long L;
    int BH;
    int nchunks;
};

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ float wave_scan(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// ---------------------------------------------------------------------------------------------
// stage 1: intra-chunk delta-system solve and WY/UT transform
// ---------------------------------------------------------------------------------------------
template <int D, class E, bool DELTA>
__global__ __launch_bounds__(256) void prep_kernel(PrefArgs a) {
    using T = typename E::T;
    using M = MM<E>;
    using Ly = Layout<D, E>;
    using frag = typename M::frag;
    constexpr int KB = M::KB, NKD = Ly::NKD, NKT = Ly::NKT, NDT = Ly::NDT;
    constexpr int TP = CH + 8;   // token stride of the transposed tiles (elements)
    constexpr int AS = CH + 4;   // row stride of the A / T matrix (floats)

    extern __shared__ __align__(16) unsigned char smem[];
    T* Kt = reinterpret_cast<T*>(smem);            // [D][TP]  K^T
    T* Vt = Kt + D * TP;                           // [D][TP]  V^T
    float* Am = reinterpret_cast<float*>(Vt + D * TP);  // [CH][AS] A, then T
    float* sg = Am + CH * AS;                      // g
    float* sbe = sg + CH;                          // beta e^g
    float* sb = sbe + CH;                          // beta
    float* skh = sb + CH;                          // e^{g_C - g}

    const int c = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, j = lane >> 4, m = lane & 15;
    const long t0 = (long)c * CH;
    const int n = (int)min((long)CH, a.L - t0);
    const size_t tok0 = (size_t)bh * a.L + t0;
    const T* kp = static_cast<const T*>(a.k) + tok0 * D;
    const T* vp = static_cast<const T*>(a.v) + tok0 * D;
    unsigned char* rec = a.ws + ((size_t)bh * a.nchunks + c) * Ly::REC;

    if (w == 0) {
        float la = 0.f, bt = 0.f;
        if (DELTA && lane < n) {
            la = a.log_alpha[tok0 + lane];
            bt = a.beta[tok0 + lane];
        }
        const float g = wave_scan(la, lane);
        const float gC = __shfl(g, 63);
        sg[lane] = g;
        sb[lane] = bt;
        sbe[lane] = bt * __expf(g);
        skh[lane] = __expf(gC - g);
        if (lane == 0) *reinterpret_cast<float*>(rec + Ly::A_DEC) = DELTA ? __expf(gC) : 1.f;
    }
    {   // K^T and V^T into LDS; padded tokens are zero (identity steps)
        const int r = tid >> 2, qd = tid & 3;
        constexpr int DQ = D / 4;
#pragma unroll
        for (int d0 = 0; d0 < DQ; d0 += 4) {
            const int d = qd * DQ + d0;
            float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
            if (r < n) {
                kk = load4(kp + (size_t)r * D + d);
                vv = load4(vp + (size_t)r * D + d);
            }
            Kt[(d + 0) * TP + r] = E::from(kk.x); Kt[(d + 1) * TP + r] = E::from(kk.y);
            Kt[(d + 2) * TP + r] = E::from(kk.z); Kt[(d + 3) * TP + r] = E::from(kk.w);
            Vt[(d + 0) * TP + r] = E::from(vv.x); Vt[(d + 1) * TP + r] = E::from(vv.y);
            Vt[(d + 2) * TP + r] = E::from(vv.z); Vt[(d + 3) * TP + r] = E::from(vv.w);
        }
    }
    __syncthreads();

    if constexpr (DELTA) {
        // Gram tiles (rt, st), st <= rt, of A[r][s] = beta_r exp(g_r - g_s) k_r.k_s, s < r
        for (int ti = w; ti < 10; ti += 4) {
            int rt = 0, st = ti;
            while (st > rt) { st -= rt + 1; ++rt; }
            const T* ra = (16 * rt + m < n) ? kp + (size_t)(16 * rt + m) * D : nullptr;
            const T* rb = (16 * st + m < n) ? kp + (size_t)(16 * st + m) * D : nullptr;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKD; ++kb)
                acc = M::mma(row_frag<E>(ra, kb * KB, j, 1.f), row_frag<E>(rb, kb * KB, j, 1.f), acc);
            const int s = 16 * st + m;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + 4 * j + e;
                Am[r * AS + s] = (s < r) ? sb[r] * __expf(sg[r] - sg[s]) * acc[e] : 0.f;
            }
        }
        __syncthreads();
        if (w == 0) {
            // T = (I + A)^-1 by forward substitution, lane c owns column c of T
            float tc[CH];
#pragma unroll
            for (int r = 0; r < CH; ++r) tc[r] = 0.f;
#pragma unroll
            for (int r = 0; r < CH; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int s = 0; s < r; s += 4) {
                    const float4 a4 = *reinterpret_cast<const float4*>(Am + r * AS + s);
                    acc += a4.x * tc[s] + a4.y * tc[s + 1] + a4.z * tc[s + 2] + a4.w * tc[s + 3];
                }
                tc[r] = (r == lane) ? 1.f : ((r < lane) ? 0.f : -acc);
            }
#pragma unroll
            for (int r = 0; r < CH; ++r) Am[r * AS + lane] = tc[r];
        } else {
            // Khat^T fragments (d-tile dt, token block kb), waves 1..3 while wave 0 solves
            for (int f = w - 1; f < NDT * NKT; f += 3) {
                const int dt = f / NKT, kb = f % NKT;
                st_frag(rec + Ly::A_KH + (size_t)f * Ly::FR, lane,
                        row_frag_ks<E>(Kt + (16 * dt + m) * TP, kb * KB, j, skh));
            }
        }
        __syncthreads();
        // wave w: token tile rt = w. T rows 16 rt .. 16 rt + 15 are zero beyond column 16 rt + 15.
        const int rt = w;
        const int kbmax = (16 * rt + 15) / KB;
        frag Tf[NKT];
#pragma unroll
        for (int kb = 0; kb < NKT; ++kb) Tf[kb] = row_frag_f32<E>(Am + (16 * rt + m) * AS, kb * KB, j);
        // -W fragments: W^T tile (dt, rt) = sum_s (beta e^g K)^T[d][s] T^T[s][r]
        f32x4 wt[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            wt[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKT; ++kb)
                if (kb <= kbmax)
                    wt[dt] = M::mma(row_frag_ks<E>(Kt + (16 * dt + m) * TP, kb * KB, j, sbe), Tf[kb], wt[dt]);
        }
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd)
            st_frag(rec + Ly::A_W + (size_t)(rt * NKD + kd) * Ly::FR, lane, M::from_acc(wt, kd, -1.f));
        // Ut tile (rt, vt) = sum_s T[r][s] (beta V)[s][v], stored as accumulators
#pragma unroll
        for (int vt = 0; vt < NDT; ++vt) {
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKT; ++kb)
                if (kb <= kbmax) u = M::mma(Tf[kb], row_frag_ks<E>(Vt + (16 * vt + m) * TP, kb * KB, j, sb), u);
            T* dst = reinterpret_cast<T*>(rec + Ly::A_UT) + ((size_t)(vt * 4 + rt) * 64 + lane) * 4;
            store4(dst, make_float4(u[0], u[1], u[2], u[3]));
        }
    } else {
        // plain linear attention: Khat = K, Ut = V
        for (int f = w; f < NDT * NKT; f += 4) {
            const int dt = f / NKT, kb = f % NKT;
            st_frag(rec + Ly::A_KH + (size_t)f * Ly::FR, lane, row_frag<E>(Kt + (16 * dt + m) * TP, kb * KB, j, 1.f));
        }
        const int rt = w;
#pragma unroll
        for (int vt = 0; vt < NDT; ++vt) {
            const float4 x = load4(Vt + (16 * vt + m) * TP + 16 * rt + 4 * j);
            T* dst = reinterpret_cast<T*>(rec + Ly::A_UT) + ((size_t)(vt * 4 + rt) * 64 + lane) * 4;
            store4(dst, x);
        }
    }
}

// ---------------------------------------------------------------------------------------------
// stage 2: the sequential chunk-to-chunk pass, state resident in registers
// ---------------------------------------------------------------------------------------------
template <int D, class E, bool DELTA>
__global__ __launch_bounds__(64) void chain_kernel(PrefArgs a) {
    using T = typename E::T;
    using M = MM<E>;
    using Ly = Layout<D, E>;
    using frag = typename M::frag;
    constexpr int NKD = Ly::NKD, NKT = Ly::NKT, NDT = Ly::NDT;
    // blockIdx -> (slice, column group) so that all column groups of one slice run on the same
    // XCD (workgroups are dealt to the 8 XCDs round-robin) and share its L2.
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int cg = slot % NDT, bh = (slot / NDT) * 8 + xcd;
    if (bh >= a.BH) return;
    const int lane = threadIdx.x, j = lane >> 4, m = lane & 15;
    const int col = 16 * cg + m;

    f32x4 H[NDT];  // lane (j, m): H[16 dt + 4 j + e][col]
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            H[dt][e] = a.h0 ? a.h0[((size_t)bh * D + 16 * dt + 4 * j + e) * D + col] : 0.f;

    const unsigned char* recA = a.ws + (size_t)bh * a.nchunks * Ly::REC;
    for (int c = 0; c < a.nchunks; ++c, recA += Ly::REC) {
        unsigned char* recB = const_cast<unsigned char*>(recA) + Ly::REC_A;
        frag Hf[NKD];
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) {
            Hf[kd] = M::from_acc(H, kd);
            st_frag(recB + Ly::B_H + (size_t)(cg * NKD + kd) * Ly::FR, lane, Hf[kd]);
        }
        f32x4 U[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const float4 x = load4(reinterpret_cast<const T*>(recA + Ly::A_UT) + ((size_t)(cg * 4 + rt) * 64 + lane) * 4);
            U[rt] = f32x4{x.x, x.y, x.z, x.w};
        }
        if constexpr (DELTA) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int kd = 0; kd < NKD; ++kd)
                    U[rt] = M::mma(ld_frag<frag>(recA + Ly::A_W + (size_t)(rt * NKD + kd) * Ly::FR, lane), Hf[kd], U[rt]);
        }
        frag Uf[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            Uf[kt] = M::from_acc(U, kt);
            st_frag(recB + Ly::B_U + (size_t)(cg * NKT + kt) * Ly::FR, lane, Uf[kt]);
        }
        const float dec = *reinterpret_cast<const float*>(recA + Ly::A_DEC);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            f32x4 h = H[dt];
            if constexpr (DELTA) h = f32x4{h[0] * dec, h[1] * dec, h[2] * dec, h[3] * dec};
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
                h = M::mma(ld_frag<frag>(recA + Ly::A_KH + (size_t)(dt * NKT + kt) * Ly::FR, lane), Uf[kt], h);
            H[dt] = h;
        }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) a.h_final[((size_t)bh * D + 16 * dt + 4 * j + e) * D + col] = H[dt][e];
}

// ---------------------------------------------------------------------------------------------
// stage 3: outputs from the chunk-start state
// ---------------------------------------------------------------------------------------------
template <int D, class E, bool DELTA>
__global__ __launch_bounds__(256) void output_kernel(PrefArgs a) {
    using T = typename E::T;
    using M = MM<E>;
    using Ly = Layout<D, E>;
    using frag = typename M::frag;
    constexpr int KB = M::KB, NKD = Ly::NKD, NKT = Ly::NKT, NDT = Ly::NDT;
    __shared__ float sg[CH];
    __shared__ __align__(16) unsigned char sP[4 * NKT * 1024];   // P fragments [rt][kt]
    __shared__ __align__(16) unsigned char sQ[4 * NKD * 1024];   // e^g Q fragments [rt][kd]

    const int c = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, j = lane >> 4, m = lane & 15;
    const long t0 = (long)c * CH;
    const int n = (int)min((long)CH, a.L - t0);
    const size_t tok0 = (size_t)bh * a.L + t0;
    const T* qp = static_cast<const T*>(a.q) + tok0 * D;
    const T* kp = static_cast<const T*>(a.k) + tok0 * D;
    T* op = static_cast<T*>(a.o) + tok0 * D;
    const unsigned char* recB = a.ws + ((size_t)bh * a.nchunks + c) * Ly::REC + Ly::REC_A;

    if (w == 0) {
        float la = 0.f;
        if (DELTA && lane < n) la = a.log_alpha[tok0 + lane];
        sg[lane] = wave_scan(la, lane);
    }
    __syncthreads();
    {
        // wave w: token tile rt = w. P^T tiles (st, rt) for st <= rt, then P fragments.
        const int rt = w;
        const int r = 16 * rt + m;   // this lane's token as the B-operand column
        const T* rq = (r < n) ? qp + (size_t)r * D : nullptr;
        f32x4 pt[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            pt[st] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (st <= rt) {
                const T* rk = (16 * st + m < n) ? kp + (size_t)(16 * st + m) * D : nullptr;
#pragma unroll
                for (int kd = 0; kd < NKD; ++kd)
                    pt[st] = M::mma(row_frag<E>(rk, kd * KB, j, 1.f), row_frag<E>(rq, kd * KB, j, 1.f), pt[st]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 16 * st + 4 * j + e;
                    pt[st][e] = (s <= r) ? pt[st][e] * __expf(sg[r] - sg[s]) : 0.f;
                }
            }
        }
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) st_frag(sP + (rt * NKT + kt) * 1024, lane, M::from_acc(pt, kt));
        const float eg = __expf(sg[r]);
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) st_frag(sQ + (rt * NKD + kd) * 1024, lane, row_frag<E>(rq, kd * KB, j, eg));
    }
    __syncthreads();
    // wave w: value tiles vt = w, w + 4, ...; all four token tiles
    for (int vt = w; vt < NDT; vt += 4) {
        frag Hc[NKD], Uf[NKT];
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) Hc[kd] = ld_frag<frag>(recB + Ly::B_H + (size_t)(vt * NKD + kd) * Ly::FR, lane);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) Uf[kt] = ld_frag<frag>(recB + Ly::B_U + (size_t)(vt * NKT + kt) * Ly::FR, lane);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) acc = M::mma(Hc[kd], ld_frag<frag>(sQ + (rt * NKD + kd) * 1024, lane), acc);
            const int kbmax = (16 * rt + 15) / KB;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
                if (kt <= kbmax) acc = M::mma(Uf[kt], ld_frag<frag>(sP + (rt * NKT + kt) * 1024, lane), acc);
            // lane (j, m): O[token 16 rt + m][16 vt + 4 j .. + 3]
            const int r = 16 * rt + m;
            if (r < n) store4(op + (size_t)r * D + 16 * vt + 4 * j, make_float4(acc[0], acc[1], acc[2], acc[3]));
        }
    }
}

// h_final = h0 (or zeros) for L = 0
__global__ void copy_state_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

template <int D, class E, bool DELTA>
static int launch_prefill_t(const PrefArgs& a, hipStream_t stream) {
    using Ly = Layout<D, E>;
    using T = typename E::T;
    constexpr int TP = CH + 8, AS = CH + 4;
    const size_t lds = (size_t)2 * D * TP * sizeof(T) + (size_t)CH * AS * 4 + 4 * CH * 4;
    static bool attr_done = false;  // benign race: every caller sets the same value
    if (!attr_done) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&prep_kernel<D, E, DELTA>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return -1;
        attr_done = true;
    }
    hipLaunchKernelGGL((prep_kernel<D, E, DELTA>), dim3(a.nchunks, a.BH), dim3(256), lds, stream, a);
    const int nslot = (a.BH + 7) / 8;
    hipLaunchKernelGGL((chain_kernel<D, E, DELTA>), dim3(8 * nslot * Ly::NDT), dim3(64), 0, stream, a);
    hipLaunchKernelGGL((output_kernel<D, E, DELTA>), dim3(a.nchunks, a.BH), dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_prefill(const void* q, const void* k, const void* v, const float* beta, const float* log_alpha,
                   const float* h0, void* o, float* h_final, int BH, long L, int D, int dtype, bool delta,
                   void* ws, hipStream_t stream) {
    if (L == 0) {
        const size_t n = (size_t)BH * D * D;
        if (h0 == h_final) return 0;
        hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, h0, h_final, n);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    PrefArgs a{q, k, v, beta, log_alpha, h0, o, h_final, static_cast<unsigned char*>(ws), L, BH,
               (int)((L + CH - 1) / CH)};
#define GDN_PF(DD, EE)                                                                             \
    return delta ? launch_prefill_t<DD, EE, true>(a, stream) : launch_prefill_t<DD, EE, false>(a, stream)
    if (D == 128 && dtype == 0) GDN_PF(128, BF16);
    if (D == 128) GDN_PF(128, F32);
    if (dtype == 0) GDN_PF(64, BF16);
    GDN_PF(64, F32);
#undef GDN_PF
}

}  // namespace gdn
