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
//   prep_kernel   (one workgroup per chunk and head, fully parallel): g, A, T = (I + A)^-1 by
//                 a blocked inverse in LDS, -W, Khat^T and Ut, written as MFMA-ready fragments.
//   chain_kernel  (one workgroup per head and 32 value columns): the sequential pass. The fp32
//                 state stays in accumulator registers for the whole sequence while loader
//                 waves stream the next chunks' operands into an LDS ring; per chunk it emits
//                 the chunk-start state and U as fragments for the output stage.
//   output_kernel (one workgroup per chunk and head): P = (Q K^T) gated and masked, then
//                 O^T = H^T (e^g Q)^T + U^T P^T, stored four value columns per lane.
// Plain linear attention uses the same kernels with T = I, W = 0, Ut = V, g = 0.
#include <mutex>
#include <type_traits>

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
    static constexpr size_t A_KEEP = A_DEC + 4;   // chunk keep flag (u32, 0 = skipped state update)
    static constexpr size_t REC_A = (A_KEEP + 4 + 255) / 256 * 256;
    // chain record: chunk-start state [cg NDT][NKD], U [cg NDT][NKT]
    static constexpr size_t B_H = 0;
    static constexpr size_t B_U = (size_t)NDT * NKD * FR;
    static constexpr size_t REC_B = B_U + (size_t)NDT * NKT * FR;
    static constexpr size_t REC = REC_A + REC_B;
};

size_t prefill_record_bytes(int D, int dtype) {
    if (D == 128 && dtype == 0) return Layout<128, BF16>::REC;
    if (D == 128) return Layout<128, F32>::REC;
    if (D == 64 && dtype == 0) return Layout<64, BF16>::REC;
    return Layout<64, F32>::REC;
}

// Preferred workspace: the whole sequence if it is short, else NBUF segment buffers of about
// SEG_TARGET bytes each, so that the three stages of consecutive segments overlap and the
// buffers can stay resident in the 256 MB Infinity Cache between the stage that writes them
// and the stage that reads them.
static constexpr size_t SEG_TARGET = (size_t)72 << 20;
static constexpr int NBUF = 2;
// A segmented call keeps three 32-bit progress counters (prep, chain, output: segments done)
// after its buffers; the streams wait on them (hipStreamWaitValue32) rather than on events,
// which measured about 5 us less per cross-stream hand-off (128K: 2.75 -> 2.63 ms).
static constexpr size_t FLAG_BYTES = 256;

size_t prefill_workspace_bytes(long BH, long L, int D, int dtype) {
    const long nch = (L + CH - 1) / CH;
    const size_t rec = prefill_record_bytes(D, dtype) * (size_t)BH;   // one chunk of every slice
    long seg = (long)(SEG_TARGET / rec);
    seg = seg < 4 ? 4 : seg;
    if (nch <= NBUF * seg) return (size_t)nch * rec;                   // one segment
    return NBUF * (size_t)seg * rec + FLAG_BYTES;
}

// Smallest workspace a call accepts: NBUF segment buffers of one chunk each and the progress
// counters (or the whole sequence when it is that short).
size_t prefill_workspace_min_bytes(long BH, long L, int D, int dtype) {
    const long nch = (L + CH - 1) / CH;
    const size_t rec = prefill_record_bytes(D, dtype) * (size_t)BH;
    return nch <= NBUF ? (size_t)nch * rec : NBUF * rec + FLAG_BYTES;
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
    unsigned char* ws;   // this segment's buffer: segcap records per slice
    long L;
    int BH;
    int c0;              // first chunk of the segment
    int nseg;            // chunks in the segment
    int segcap;          // records per slice in the buffer
    const unsigned char* keep;   // [BH][nchk] chunk keep mask, or NULL (keep all)
    int nchk;                    // chunks per slice of the whole sequence
    int band;                    // 16 x 16 blocks of T kept below the diagonal (3: all, exact)
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


// Off-diagonal block (bi, bj), bi > bj, of T = (I + A)^-1 (16 x 16 blocks, fp32, row stride AS):
//     T_ij = -T_ii * sum_{k=j}^{i-1} A_ik T_kj
// on fp32 MFMA. Every T_kj with k < i must be final. Called by one whole wave.
template <int AS>
__device__ __forceinline__ void inverse_block_t(const float* Am, float* Tm, int bi, int bj, int j, int m) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    for (int bk = bj; bk < bi; ++bk) {
        // A_ik rows (lane (j, m): A[m][4 j + e]) times T_kj as B (lane (j, n): T[4 j + e][n])
        const float4 a = *reinterpret_cast<const float4*>(Am + (16 * bi + m) * AS + 16 * bk + 4 * j);
        f32x4 b;
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = Tm[(16 * bk + 4 * j + e) * AS + 16 * bj + m];
        x = MM<F32>::mma(f32x4{a.x, a.y, a.z, a.w}, b, x);
    }
    const float4 t = *reinterpret_cast<const float4*>(Tm + (16 * bi + m) * AS + 16 * bi + 4 * j);
    const f32x4 y = MM<F32>::mma(f32x4{t.x, t.y, t.z, t.w}, x, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int e = 0; e < 4; ++e) Tm[(16 * bi + 4 * j + e) * AS + 16 * bj + m] = -y[e];
}

// Workgroup barrier for kernels whose waves share only LDS: it waits for this wave's LDS
// operations (lgkmcnt) and nothing else. __syncthreads also fences global memory, which makes
// every wave first wait for all of its outstanding global stores and loads (vmcnt(0)); none of
// the prefill kernels reads back through global memory what another wave of its workgroup
// wrote, so that wait is pure latency.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------------------------
// stage 1: intra-chunk delta-system solve and WY/UT transform
// ---------------------------------------------------------------------------------------------
// Work split of the prep workgroup's four waves. The d extent is cut into fragment groups of
// KB / 16 d-tiles (one operand fragment wide); a wave owns GPW groups, or shares one group with
// WPG - 1 other waves and then takes RPW of the four token tiles.
template <int D, class E>
struct PrepCfg {
    using Ly = Layout<D, E>;
    static constexpr int FPD = MM<E>::KB / 16;                   // d tiles per fragment
    static constexpr int WPG = Ly::NKD >= 4 ? 1 : 4 / Ly::NKD;   // waves per fragment group
    static constexpr int GPW = Ly::NKD >= 4 ? Ly::NKD / 4 : 1;   // fragment groups per wave
    static constexpr int RPW = 4 / WPG;                          // token tiles per wave
    static constexpr int DPW = GPW * FPD;                        // d tiles per wave
    static constexpr int KP = D + 8;                             // K / V row stride (elements)
    static constexpr int AS = CH + 4;                            // A / T row stride (floats)
    static constexpr size_t ROWS = (size_t)CH * KP * sizeof(typename E::T);
    static constexpr size_t MAT = (size_t)CH * AS * 4;
    // region 0: K rows, then T; region 1: V rows, then A
    static constexpr size_t REGION = ((ROWS > MAT ? ROWS : MAT) + 15) / 16 * 16;
    static constexpr size_t LDS = 2 * REGION + 4 * CH * 4;
};

template <int D, class E, bool DELTA>
__global__ __launch_bounds__(256) void prep_kernel(PrefArgs a) {
    using T = typename E::T;
    using M = MM<E>;
    using Ly = Layout<D, E>;
    using P = PrepCfg<D, E>;
    using frag = typename M::frag;
    constexpr int KB = M::KB, NKD = Ly::NKD, NKT = Ly::NKT;
    constexpr int FPD = P::FPD, WPG = P::WPG, GPW = P::GPW, RPW = P::RPW, DPW = P::DPW, KP = P::KP, AS = P::AS;

    extern __shared__ __align__(16) unsigned char smem[];
    T* Kr = reinterpret_cast<T*>(smem);                               // [CH][KP] K rows
    float* Tm = reinterpret_cast<float*>(smem);                       // [CH][AS] T = (I + A)^-1, after K
    T* Vr = reinterpret_cast<T*>(smem + P::REGION);                   // [CH][KP] V rows
    float* Am = reinterpret_cast<float*>(smem + P::REGION);           // [CH][AS] A (strictly lower), after V
    float* sg = reinterpret_cast<float*>(smem + 2 * P::REGION);       // g
    float* sbe = sg + CH;                                             // -beta e^g
    float* sb = sbe + CH;                                             // beta
    float* skh = sb + CH;                                             // e^{g_C - g}

    const int cl = blockIdx.x, bh = blockIdx.y;     // chunk within the segment, slice
    // The wave index lives in a scalar register so that every branch on it (token tiles,
    // fragment groups, tile bounds) is a scalar branch. Matrix-core instructions write their
    // result whatever the lane mask, so none may sit in a block that is skipped by masking lanes.
    const int tid = threadIdx.x, lane = tid & 63, j = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = GPW * (w / WPG);                // this wave's first d-fragment group
    const int rt0 = RPW * (w % WPG);                // this wave's first token tile
    const long t0 = (long)(a.c0 + cl) * CH;
    const int n = (int)min((long)CH, a.L - t0);
    const size_t tok0 = (size_t)bh * a.L + t0;
    const T* kp = static_cast<const T*>(a.k) + tok0 * D;
    const T* vp = static_cast<const T*>(a.v) + tok0 * D;
    unsigned char* rec = a.ws + ((size_t)bh * a.segcap + cl) * Ly::REC;

    if (w == 0) {
        float la = 0.f, bt = 0.f;
        if (lane < n) {
            if (a.log_alpha) la = a.log_alpha[tok0 + lane];   // optional without the delta term
            if (DELTA) bt = a.beta[tok0 + lane];
        }
        const float g = wave_scan(la, lane);
        const float gC = __shfl(g, 63);
        sg[lane] = g;
        sb[lane] = bt;
        sbe[lane] = -bt * __expf(g);
        skh[lane] = __expf(gC - g);
        if (lane == 0) {
            *reinterpret_cast<float*>(rec + Ly::A_DEC) = a.log_alpha ? __expf(gC) : 1.f;
            *reinterpret_cast<unsigned*>(rec + Ly::A_KEEP) =
                a.keep ? (a.keep[(size_t)bh * a.nchk + a.c0 + cl] != 0 ? 1u : 0u) : 1u;
        }
    }
    {   // K and V rows, 16 bytes per lane, all loads in flight at once; rows past the chunk's
        // end read as zero (identity steps)
        constexpr int EPU = 16 / sizeof(T), UPR = D / EPU, NU = CH * UPR / 256;
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kp, n * D * (int)sizeof(T));
        const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vp, n * D * (int)sizeof(T));
        uint4 xk[NU], xv[NU];
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            xk[i] = buffer_load16(rk, (tid + 256 * i) * 16);
            xv[i] = buffer_load16(rv, (tid + 256 * i) * 16);
        }
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = tid + 256 * i, r = u / UPR, cu = u % UPR;
            *reinterpret_cast<uint4*>(Kr + r * KP + cu * EPU) = xk[i];
            *reinterpret_cast<uint4*>(Vr + r * KP + cu * EPU) = xv[i];
        }
    }
    lds_barrier();

    // Rows to columns on the matrix core: kc[i][st] is the accumulator tile of tokens 16 st ..
    // 16 st + 15 and d-tile dt = FPD grp + i of K (lane (j, n): K[16 st + 4 j + e][16 dt + n]);
    // vc likewise for V. Fragments built from them have k = token, which the products over a
    // chunk's tokens need.
    // tiles(R, i, t): the four token tiles of d-tile FPD grp + i of the rows R
    auto tiles = [&](const T* R, int i, f32x4 (&t)[4]) {
        const int dt = FPD * grp + i;
        const frag sel = unit_cols<E>(j, m, dt % FPD);
#pragma unroll
        for (int st = 0; st < 4; ++st)
            t[st] = M::mma(row_frag_raw<E>(R + (16 * st + m) * KP, KB * (dt / FPD), j), sel, f32x4{0.f, 0.f, 0.f, 0.f});
    };

    if constexpr (!DELTA) {
        // linear attention without the delta term: Khat = e^{g_C - g} K (K without gates), Ut = V
#pragma unroll
        for (int i = 0; i < DPW; ++i) {
            const int dt = FPD * grp + i;
            f32x4 kc[4], vc[4];
            tiles(Kr, i, kc);
            tiles(Vr, i, vc);
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
                if (kt % WPG == w % WPG)
                    st_frag(rec + Ly::A_KH + (size_t)(dt * NKT + kt) * Ly::FR, lane,
                            a.log_alpha ? cols_frag<E>(&kc[FPD * kt], skh + KB * kt, j) : cols_frag<E>(&kc[FPD * kt]));
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const int rt = rt0 + r;
                T* dst = reinterpret_cast<T*>(rec + Ly::A_UT) + ((size_t)(dt * 4 + rt) * 64 + lane) * 4;
                store4(dst, make_float4(vc[rt][0], vc[rt][1], vc[rt][2], vc[rt][3]));
            }
        }
        return;
    } else {
        // Gram tiles (rt, st), st <= rt, of K K^T: ten tiles over the four waves
        f32x4 gacc[3];
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            const int ti = w + 4 * x;
            gacc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (ti < 10) {
                int rt = 0, st = ti;
                while (st > rt) { st -= rt + 1; ++rt; }
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb)
                    gacc[x] = M::mma(row_frag_raw<E>(Kr + (16 * rt + m) * KP, kb * KB, j),
                                     row_frag_raw<E>(Kr + (16 * st + m) * KP, kb * KB, j), gacc[x]);
            }
        }
        // Register pressure sets how many prep workgroups share a CU (four need at most 128
        // VGPRs). The scheduling barriers keep the compiler from hoisting the LDS reads of one
        // phase (Gram, K transposes, V transposes) into the previous one, and the kept fragments
        // are pinned packed in registers: left alone, the compiler sinks their scaling and
        // packing to the end of the kernel and keeps the fp32 tiles alive across the solve.
        __builtin_amdgcn_sched_barrier(0);
        // Khat^T fragments (stored), -beta e^g K^T and beta V^T fragments (kept), one d-tile's
        // transposed tiles live at a time
        frag kbe[DPW][NKT], vb[DPW][NKT];
#pragma unroll
        for (int i = 0; i < DPW; ++i) {
            const int dt = FPD * grp + i;
            f32x4 kc[4];
            tiles(Kr, i, kc);
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                if (kt % WPG == w % WPG)
                    st_frag(rec + Ly::A_KH + (size_t)(dt * NKT + kt) * Ly::FR, lane,
                            cols_frag<E>(&kc[FPD * kt], skh + KB * kt, j));
                kbe[i][kt] = cols_frag<E>(&kc[FPD * kt], sbe + KB * kt, j);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < DPW; ++i) {
            f32x4 vc[4];
            tiles(Vr, i, vc);
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) vb[i][kt] = cols_frag<E>(&vc[FPD * kt], sb + KB * kt, j);
        }
#pragma unroll
        for (int i = 0; i < DPW; ++i)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                asm volatile("" : "+v"(kbe[i][kt]));
                asm volatile("" : "+v"(vb[i][kt]));
            }
        lds_barrier();   // K and V rows are no longer read: their space takes T and A
        // A[r][s] = beta_r exp(g_r - g_s) k_r.k_s for s < r
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            const int ti = w + 4 * x;
            if (ti < 10) {
                int rt = 0, st = ti;
                while (st > rt) { st -= rt + 1; ++rt; }
                const int s = 16 * st + m;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rt + 4 * j + e;
                    Am[r * AS + s] = (s < r) ? sb[r] * __expf(sg[r] - sg[s]) * gacc[x][e] : 0.f;
                }
            }
        }
        // zero the above-diagonal 16 x 16 blocks of T (fragments of 32 tokens read some of them)
        // and, for the block-adjacent approximation, the blocks more than `band` below it
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const int bi = b >> 2, bj = b & 3;
            if (bj > bi || bi - bj > a.band) Tm[(16 * bi + (tid >> 4)) * AS + 16 * bj + (tid & 15)] = 0.f;
        }
        lds_barrier();
        // T = (I + A)^-1, blocked by 16: diagonal blocks by forward substitution (wave i inverts
        // block i, lane c < 16 owns column c), then T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj level
        // by level on fp32 MFMA.
        {
            const int i0 = 16 * w, c = lane & 15;
            float tc[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < r; ++s2) acc += Am[(i0 + r) * AS + i0 + s2] * tc[s2];
                tc[r] = (r == c) ? 1.f : ((r < c) ? 0.f : -acc);
            }
            if (lane < 16) {
#pragma unroll
                for (int r = 0; r < 16; ++r) Tm[(i0 + r) * AS + i0 + c] = tc[r];
            }
        }
#pragma unroll
        for (int lvl = 1; lvl < 4; ++lvl) {
            lds_barrier();
            if (w + lvl < 4 && lvl <= a.band) inverse_block_t<AS>(Am, Tm, w + lvl, w, j, m);
        }
        lds_barrier();
        // this wave's token tiles: T rows as fragments (rows 16 rt .. 16 rt + 15 of T are zero
        // beyond column 16 rt + 15, so token blocks past kbmax are skipped)
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int rt = rt0 + r;
            const int kbmax = (16 * rt + 15) / KB;
            frag Tf[NKT];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
                if (kt <= kbmax) Tf[kt] = row_frag_f32<E>(Tm + (16 * rt + m) * AS, kt * KB, j);
            // -W^T tiles (dt, rt) = sum_s (-beta e^g K)^T[d][s] T[r][s], then -W fragments [rt][kd]
            f32x4 wt[DPW];
#pragma unroll
            for (int i = 0; i < DPW; ++i) {
                wt[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
                    if (kt <= kbmax) wt[i] = M::mma(kbe[i][kt], Tf[kt], wt[i]);
            }
#pragma unroll
            for (int g2 = 0; g2 < GPW; ++g2)
                st_frag(rec + Ly::A_W + (size_t)(rt * NKD + grp + g2) * Ly::FR, lane, M::from_acc(&wt[FPD * g2], 0));
            // Ut tiles (rt, vt) = sum_s T[r][s] (beta V)[s][v], stored as accumulators
#pragma unroll
            for (int i = 0; i < DPW; ++i) {
                const int vt = FPD * grp + i;
                f32x4 ut = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
                    if (kt <= kbmax) ut = M::mma(Tf[kt], vb[i][kt], ut);
                T* dst = reinterpret_cast<T*>(rec + Ly::A_UT) + ((size_t)(vt * 4 + rt) * 64 + lane) * 4;
                store4(dst, make_float4(ut[0], ut[1], ut[2], ut[3]));
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// stage 2: the sequential chunk-to-chunk pass, state resident in registers
// ---------------------------------------------------------------------------------------------
// Chain workgroup: one slice (batch, head) and 16 value columns (a column group), four waves.
// The fp32 state of the column group (Dk x 16) is split by rows between the two compute waves,
// each holding its half in accumulator registers for the whole sequence; per chunk they exchange
// their fp32 partial products W H through LDS (4 KB each), so each wave's chain step is half the
// MFMA work. The compute waves touch no global memory in their loop: the two loader waves
//   - stream each chunk's -W and Khat^T fragments (contiguous at the start of its prep record,
//     shared by all column groups of the slice), the group's Ut tiles and the decay into a ring
//     of NS LDS slots, NS - 1 chunks ahead, and
//   - store the chunk-start state and U fragments the compute waves leave in an LDS staging
//     area (three steps deep) to the workspace for the output stage.
// A CU's vector-memory path serves all its waves in order, so stores issued by the compute
// waves would queue behind the loaders' streaming loads and stall the sequential chain; issued
// by the loaders, they only delay loads that are steps ahead of their use.
template <int D, class E, bool DELTA>
struct ChainCfg {
    using Ly = Layout<D, E>;
    static constexpr int NCW = D / 16;                                   // workgroups per slice
    static constexpr int THREADS = 256;                                  // 2 compute waves, then 2 loaders
    static constexpr size_t SLOT = Ly::A_UT;                             // -W and Khat^T fragments
    static constexpr int NBLK = (int)(SLOT / 1024);                      // 1 KB wave blocks per slot
    static constexpr int BPW = NBLK / 2;                                 // blocks per loader wave
    static_assert(SLOT % 2048 == 0, "slot splits into whole blocks per loader wave");
    static constexpr size_t UTSUB = (size_t)4 * 64 * 4 * sizeof(typename E::T);  // Ut bytes of 16 columns
    static constexpr int UTL = (int)(UTSUB / 2048);                      // Ut 1 KB loads per loader wave
    static_assert(UTSUB % 2048 == 0, "Ut splits into whole blocks per loader wave");
    static constexpr size_t USLOT = UTSUB + 256;                         // Ut, then the decay (a dword per lane)
    static constexpr int DMA_OPS = BPW + UTL + 1;                        // loads per loader wave and chunk
    static constexpr size_t XHALF = (size_t)4 * 64 * 16;                 // one wave's partial W H
    static constexpr size_t XBYTES = DELTA ? (size_t)2 * 2 * XHALF : 0; // [step parity][half]
    // per compute wave and step: its Dk/2 rows of the state (Ly::NKD / 2 fragments) and half of
    // the U fragments
    static constexpr int STG = Ly::NKD / 2 + Ly::NKT / 2;
    static constexpr size_t STB = (size_t)STG * 1024;
    // the loaders store them when the staging area fits beside two or more slots (not for fp32 at
    // Dk = 128, whose compute waves store their own fragments)
    static constexpr bool SL = (SLOT + USLOT) * 2 + XBYTES + 3 * 2 * STB <= 156 * 1024;
    static constexpr size_t STAGE = SL ? 3 * 2 * STB : 0;                // [step % 3][wave][fragment]
    static constexpr size_t FIXED = XBYTES + STAGE;
    static constexpr int NS = (SLOT + USLOT) * 4 + FIXED <= 156 * 1024 ? 4 : ((SLOT + USLOT) * 3 + FIXED <= 156 * 1024 ? 3 : 2);
    static constexpr size_t O_X = NS * SLOT;                             // LDS offsets of the areas
    static constexpr size_t O_UT = O_X + XBYTES;
    static constexpr size_t O_ST = O_UT + NS * USLOT;
    static constexpr size_t LDS = O_ST + STAGE;
    static_assert(LDS <= 156 * 1024, "chain LDS");
    static constexpr int INFLIGHT = NS - 2;                              // chunks still loading at a barrier
    // a loader's vector-memory operations after chunk c + 1's loads when it waits for them:
    // that chunk's iteration's stores, then INFLIGHT whole iterations
    static constexpr int LST = SL ? STG : 0;                             // stores per loader iteration
    static constexpr int WAITN = LST + INFLIGHT * (DMA_OPS + LST);
    static_assert(WAITN < 64, "vmcnt is 6 bits");
};

// Barrier of the chain workgroup: see lds_barrier. Its loader waves fill the LDS ring with
// direct-to-LDS loads whose completion they establish themselves (wait_vmcnt) before arriving,
// and the compute waves exchange partial products through ordinary LDS writes, so the barrier
// must not wait for the global stores and the loads still in flight for later chunks.
// Wait until at most N vector-memory operations of this wave are outstanding (gfx9 encoding:
// vmcnt split over bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Direct-to-LDS load of 16 bytes per lane: lane l's bytes land at LDS address lds_base + 16 l.
// Issued as inline assembly so that the compiler does not track it: the loader waves account
// for these loads themselves (wait_vmcnt), and the compute waves, which only read LDS, must not
// be made to wait on them or on their own global stores.
// M0 is a reserved register, so clang warns about the clobber; the kernels that call dma16 use
// M0 for nothing else, and the asm sets it before each load.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, unsigned lds_base) {
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);   // wave-uniform by construction
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base)
                 : "memory", "m0");
}
// Same with 4 bytes per lane: lane l's dword lands at lds_base + 4 l.
__device__ __forceinline__ void dma4(const void* src, unsigned lds_base) {
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds_base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// Loader wave lw's share of chunk c's loads into slot s: BPW 1 KB blocks of the -W / Khat^T
// fragments (interleaved with the other loader's), its half of the Ut tiles, and the decay
// (both loaders load it; same bytes, same place).
template <int D, class E, bool DELTA>
__device__ __forceinline__ void chain_issue(unsigned char* smem, const unsigned char* rec, int s, int cg, int lw,
                                            int lane) {
    using C = ChainCfg<D, E, DELTA>;
    using Ly = Layout<D, E>;
    const unsigned base = lds_addr(smem + (size_t)s * C::SLOT);
#pragma unroll
    for (int i = 0; i < C::BPW; ++i) {
        const unsigned blk = (unsigned)(lw + 2 * i) * 1024u;
        dma16(rec + blk + lane * 16, base + blk);
    }
    const unsigned ubase = lds_addr(smem + C::O_UT + (size_t)s * C::USLOT);
    const unsigned char* ut = rec + Ly::A_UT + (size_t)cg * C::UTSUB;
#pragma unroll
    for (int i = 0; i < C::UTL; ++i) {
        const unsigned blk = (unsigned)(lw * C::UTL + i) * 1024u;
        dma16(ut + blk + lane * 16, ubase + blk);
    }
    dma4(rec + Ly::A_DEC + 4 * (lane & 1), ubase + (unsigned)C::UTSUB);   // decay, keep flag, decay, ...
}

// Loader wave lw's stores of step c's staged fragments (those of compute wave lw): its rows of
// the chunk-start state, then its U fragments (kt = lw, lw + 2, ...).
template <int D, class E, bool DELTA>
__device__ __forceinline__ void chain_store(const unsigned char* smem, unsigned char* recB, int c, int cg, int lw,
                                            int lane) {
    using C = ChainCfg<D, E, DELTA>;
    using Ly = Layout<D, E>;
    constexpr int HKD = Ly::NKD / 2;
    const unsigned char* st = smem + C::O_ST + ((size_t)(c % 3) * 2 + lw) * C::STB;
#pragma unroll
    for (int i = 0; i < C::STG; ++i) {
        const uint4 x = *reinterpret_cast<const uint4*>(st + (size_t)i * 1024 + lane * 16);
        const size_t off = i < HKD ? Ly::B_H + (size_t)(cg * Ly::NKD + lw * HKD + i) * Ly::FR
                                   : Ly::B_U + (size_t)(cg * Ly::NKT + lw + 2 * (i - HKD)) * Ly::FR;
        *reinterpret_cast<uint4*>(recB + off + lane * 16) = x;
    }
}

// Loader wave lw (0 or 1) of a chain workgroup. Iteration c (after barrier c - 1): issue chunk
// c + NS - 1 into the slot of chunk c - 1 (whose fragments the compute waves read before
// barrier c - 1), store step c - 2's staged fragments (complete since barrier c - 1), wait for
// chunk c + 1 (read by the compute waves after barrier c), barrier c. Every iteration issues the
// same operations, so the wait is a fixed count once the first NS iterations are past (those
// drain fully). After the last step, one more barrier and the last two steps' stores.
template <int D, class E, bool DELTA>
__device__ __forceinline__ void chain_loader(unsigned char* smem, const unsigned char* rec0, int nch, int cg, int lw,
                                             int lane) {
    using Ly = Layout<D, E>;
    using C = ChainCfg<D, E, DELTA>;
    constexpr int NS = C::NS;
    auto recb = [&](int c) { return const_cast<unsigned char*>(rec0) + (size_t)c * Ly::REC + Ly::REC_A; };
    for (int c = 0; c < NS - 1; ++c)
        chain_issue<D, E, DELTA>(smem, rec0 + (size_t)min(c, nch - 1) * Ly::REC, c, cg, lw, lane);
    wait_vmcnt<0>();
    lds_barrier();
    for (int c = 0; c < nch; ++c) {
        const int cn = c + NS - 1;   // always issued (clamped to the last chunk): fixed counts
        chain_issue<D, E, DELTA>(smem, rec0 + (size_t)min(cn, nch - 1) * Ly::REC, cn % NS, cg, lw, lane);
        // step c - 2's fragments (before step 0: step 0's record, rewritten with the real ones
        // two iterations later by this same wave, in order)
        if constexpr (C::SL) chain_store<D, E, DELTA>(smem, recb(max(c - 2, 0)), max(c - 2, 0), cg, lw, lane);
        if (c < NS)
            wait_vmcnt<0>();
        else
            wait_vmcnt<C::WAITN>();
        lds_barrier();
    }
    lds_barrier();   // the compute waves' last step is staged
    if constexpr (C::SL)
        for (int c = max(nch - 2, 0); c < nch; ++c) chain_store<D, E, DELTA>(smem, recb(c), c, cg, lw, lane);
    wait_vmcnt<0>();   // no LDS write may land after the workgroup ends
}

// Compute wave HH of a chain workgroup: it owns state rows [HH Dk/2, (HH + 1) Dk/2) of column
// group cg. Per chunk c:
//   A  Hf = bf16(H), staged for the output stage; partial product P_HH = (-W)[:, half] Hf, with
//      Ut folded into the accumulators of token tiles 2 HH and 2 HH + 1; P_HH -> LDS;
//      H *= chunk decay.
//   B  U = P_HH + P_other (fp32 addition is commutative, so both waves hold the same U), its
//      fragments half staged; H += Khat^T[half, :] bf16(U); then chunk c + 1's -W and Khat^T
//      fragments are read from its slot (complete since barrier c), so neither product of the
//      next step waits on LDS.
// One barrier per step, between A and B: the partial products alternate between two LDS areas
// by step parity, so an area is rewritten only after the partner has passed the next barrier.
// Ut and the decay are read in A, before the barrier after which their slot may be refilled.
template <int D, class E, bool DELTA, int HH>
__device__ __forceinline__ void chain_compute(const PrefArgs& a, unsigned char* smem, const unsigned char* rec0,
                                              int nch, int bh, int cg, int lane) {
    using T = typename E::T;
    using M = MM<E>;
    using Ly = Layout<D, E>;
    using C = ChainCfg<D, E, DELTA>;
    using frag = typename M::frag;
    constexpr int NKD = Ly::NKD, NKT = Ly::NKT, NDT = Ly::NDT, NS = C::NS;
    constexpr int HKD = NKD / 2, HDT = NDT / 2;   // fragments / tiles of one row half
    f32x4* X0 = reinterpret_cast<f32x4*>(smem + C::O_X);                   // [parity][half][rt][lane]
    constexpr size_t XPAR = 2 * C::XHALF / sizeof(f32x4);
    const int j = lane >> 4, m = lane & 15;
    const int col = 16 * cg + m;
    f32x4 H[HDT];   // lane (j, m): H[16 (HH HDT + t) + 4 j + e][col]
#pragma unroll
    for (int t = 0; t < HDT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            H[t][e] = a.h0 ? a.h0[((size_t)bh * D + 16 * (HH * HDT + t) + 4 * j + e) * D + col] : 0.f;
    // -W and Khat^T fragments of the chunk in slot s
    frag wf[4 * HKD], kf[HDT * NKT];
    auto read_slot = [&](int s) {
        const unsigned char* slot = smem + (size_t)s * C::SLOT;
        if constexpr (DELTA) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int kk = 0; kk < HKD; ++kk)
                    wf[rt * HKD + kk] = ld_frag<frag>(slot + Ly::A_W + (size_t)(rt * NKD + HH * HKD + kk) * Ly::FR, lane);
        }
#pragma unroll
        for (int t = 0; t < HDT; ++t)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
                kf[t * NKT + kt] = ld_frag<frag>(slot + Ly::A_KH + (size_t)((HH * HDT + t) * NKT + kt) * Ly::FR, lane);
    };
    lds_barrier();
    read_slot(0);
    for (int c = 0; c < nch; ++c) {
        f32x4* X = X0 + (c & 1) * XPAR;
        const unsigned char* us = smem + C::O_UT + (size_t)(c % NS) * C::USLOT;
        const T* ut = reinterpret_cast<const T*>(us);   // [rt][lane][4]
        unsigned char* st = smem + C::O_ST + ((size_t)(c % 3) * 2 + HH) * C::STB;
        unsigned char* recB = const_cast<unsigned char*>(rec0) + (size_t)c * Ly::REC + Ly::REC_A;
        frag Hf[HKD];
#pragma unroll
        for (int kk = 0; kk < HKD; ++kk) {
            Hf[kk] = M::from_acc(H, kk);
            if constexpr (C::SL)
                st_frag(st + (size_t)kk * 1024, lane, Hf[kk]);
            else
                st_frag(recB + Ly::B_H + (size_t)(cg * NKD + HH * HKD + kk) * Ly::FR, lane, Hf[kk]);
        }
        f32x4 P[4];
        const float dec = *reinterpret_cast<const float*>(us + C::UTSUB);
        const unsigned keep = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const unsigned*>(us + C::UTSUB + 4));
        if constexpr (DELTA) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                if ((rt >> 1) == HH) {
                    const float4 x = load4(ut + ((size_t)rt * 64 + lane) * 4);
                    P[rt] = f32x4{x.x, x.y, x.z, x.w};
                } else {
                    P[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
#pragma unroll
            for (int kk = 0; kk < HKD; ++kk)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) P[rt] = M::mma(wf[rt * HKD + kk], Hf[kk], P[rt]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) X[(HH * 4 + rt) * 64 + lane] = P[rt];
#pragma unroll
            for (int t = 0; t < HDT; ++t) H[t] = f32x4{H[t][0] * dec, H[t][1] * dec, H[t][2] * dec, H[t][3] * dec};
        } else {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const float4 x = load4(ut + ((size_t)rt * 64 + lane) * 4);
                P[rt] = f32x4{x.x, x.y, x.z, x.w};
            }
#pragma unroll
            for (int t = 0; t < HDT; ++t) H[t] = f32x4{H[t][0] * dec, H[t][1] * dec, H[t][2] * dec, H[t][3] * dec};
        }
        lds_barrier();   // partial products exchanged; chunk c + 1's slot is complete
        f32x4 U[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            if constexpr (DELTA) {
                const f32x4 po = X[((1 - HH) * 4 + rt) * 64 + lane];
                U[rt] = f32x4{P[rt][0] + po[0], P[rt][1] + po[1], P[rt][2] + po[2], P[rt][3] + po[3]};
            } else {
                U[rt] = P[rt];
            }
        }
        frag Uf[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            Uf[kt] = M::from_acc(U, kt);
            if (kt % 2 == HH) {
                if constexpr (C::SL)
                    st_frag(st + (size_t)(HKD + kt / 2) * 1024, lane, Uf[kt]);
                else
                    st_frag(recB + Ly::B_U + (size_t)(cg * NKT + kt) * Ly::FR, lane, Uf[kt]);
            }
        }
        if (keep) {   // a skipped chunk's update leaves the decayed state (its U still feeds its outputs)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int t = 0; t < HDT; ++t) H[t] = M::mma(kf[t * NKT + kt], Uf[kt], H[t]);
        }
        read_slot((c + 1) % NS);
    }
    lds_barrier();   // the last step's fragments are staged for the loaders
#pragma unroll
    for (int t = 0; t < HDT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            a.h_final[((size_t)bh * D + 16 * (HH * HDT + t) + 4 * j + e) * D + col] = H[t][e];
}

// One workgroup per CU (its LDS ring). Waves 0 and 1 compute (row half w), waves 2 and 3 load
// and store; the roles run separate loops with the same barrier sequence.
template <int D, class E, bool DELTA>
__global__ __launch_bounds__(256) void chain_kernel(PrefArgs a) {
    using Ly = Layout<D, E>;
    using C = ChainCfg<D, E, DELTA>;
    extern __shared__ __align__(16) unsigned char smem[];
    // blockIdx -> (slice, column group) so that all column groups of one slice run on the same
    // XCD (workgroups are dealt to the 8 XCDs round-robin) and share its L2.
    const int xcd = blockIdx.x & 7, sl = blockIdx.x >> 3;
    const int cg = sl % C::NCW, bh = (sl / C::NCW) * 8 + xcd;
    if (bh >= a.BH) return;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const unsigned char* rec0 = a.ws + (size_t)bh * a.segcap * Ly::REC;
    if (w >= 2)
        chain_loader<D, E, DELTA>(smem, rec0, a.nseg, cg, w - 2, lane);
    else if (w == 1)
        chain_compute<D, E, DELTA, 1>(a, smem, rec0, a.nseg, bh, cg, lane);
    else
        chain_compute<D, E, DELTA, 0>(a, smem, rec0, a.nseg, bh, cg, lane);
}

// ---------------------------------------------------------------------------------------------
// stage 3: outputs from the chunk-start state
// ---------------------------------------------------------------------------------------------
// P^T tiles (st, rt) the output stage needs: every tile inside a token block that some P
// fragment of token tile rt reads (tiles above the diagonal come out as zeros)
template <class E>
struct OutTiles {
    static constexpr int FPD = MM<E>::KB / 16;
    static constexpr int kbmax(int rt) { return (16 * rt + 15) / MM<E>::KB; }
    static constexpr int count() {
        int c = 0;
        for (int rt = 0; rt < 4; ++rt) c += FPD * (kbmax(rt) + 1);
        return c;
    }
    static constexpr int N = count();
    static constexpr int PER_WAVE = (N + 3) / 4;
    // tile i -> (rt, st), in order of rt then st
    static __device__ __forceinline__ void tile(int i, int& rt, int& st) {
        rt = 0;
        while (i >= FPD * (kbmax(rt) + 1)) { i -= FPD * (kbmax(rt) + 1); ++rt; }
        st = i;
    }
};

template <int D, class E, bool DELTA>
__global__ __launch_bounds__(256) void output_kernel(PrefArgs a) {
    using T = typename E::T;
    using M = MM<E>;
    using Ly = Layout<D, E>;
    using OT = OutTiles<E>;
    using frag = typename M::frag;
    constexpr int KB = M::KB, NKD = Ly::NKD, NKT = Ly::NKT, NDT = Ly::NDT, FPD = OT::FPD;
    constexpr int KP = D + 8;   // row stride of the staged Q and K tiles (elements)
    extern __shared__ __align__(16) unsigned char smem[];
    T* Qr = reinterpret_cast<T*>(smem);                          // [CH][KP] Q rows
    T* Kr = Qr + CH * KP;                                        // [CH][KP] K rows, then
    unsigned char* sP = reinterpret_cast<unsigned char*>(Kr);    //   the P fragments [rt][kt]
    float* sg = reinterpret_cast<float*>(Kr + CH * KP);          // g
    static_assert((size_t)4 * NKT * 1024 <= (size_t)CH * KP * sizeof(T), "P fragments fit in the K rows");

    const int cl = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, j = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar, as in prep_kernel
    const long t0 = (long)(a.c0 + cl) * CH;
    const int n = (int)min((long)CH, a.L - t0);
    const size_t tok0 = (size_t)bh * a.L + t0;
    const T* qp = static_cast<const T*>(a.q) + tok0 * D;
    const T* kp = static_cast<const T*>(a.k) + tok0 * D;
    T* op = static_cast<T*>(a.o) + tok0 * D;
    const unsigned char* recB = a.ws + ((size_t)bh * a.segcap + cl) * Ly::REC + Ly::REC_A;

    // Q and K rows (16 bytes per lane, rows past the chunk's end read as zero) are requested
    // first, then the chunk-start state and U fragments of this wave's value tiles vt = w, w + 4,
    // ...: the rows are waited for before the staging, the fragments stay in flight through the
    // P computation
    constexpr int EPU = 16 / sizeof(T), UPR = D / EPU, NU = CH * UPR / 256;
    uint4 xq[NU], xk[NU];
    {
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(qp, n * D * (int)sizeof(T));
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kp, n * D * (int)sizeof(T));
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            xq[i] = buffer_load16(rq, (tid + 256 * i) * 16);
            xk[i] = buffer_load16(rk, (tid + 256 * i) * 16);
        }
    }
    static_assert(NDT % 4 == 0, "every wave owns the same number of value tiles");
    constexpr int NVW = NDT / 4;
    frag Hc[NVW][NKD], Uf[NVW][NKT];
#pragma unroll
    for (int iv = 0; iv < NVW; ++iv) {   // no branch here: the loads above must stay in flight
        const int vt = w + 4 * iv;
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd)
            Hc[iv][kd] = ld_frag<frag>(recB + Ly::B_H + (size_t)(vt * NKD + kd) * Ly::FR, lane);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
            Uf[iv][kt] = ld_frag<frag>(recB + Ly::B_U + (size_t)(vt * NKT + kt) * Ly::FR, lane);
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        const int u = tid + 256 * i, r = u / UPR, cu = u % UPR;
        *reinterpret_cast<uint4*>(Qr + r * KP + cu * EPU) = xq[i];
        *reinterpret_cast<uint4*>(Kr + r * KP + cu * EPU) = xk[i];
    }
    if (w == 0) {
        float la = 0.f;
        if (a.log_alpha && lane < n) la = a.log_alpha[tok0 + lane];
        sg[lane] = wave_scan(la, lane);
    }
    lds_barrier();
    // P^T tile (st, rt), lane (j, n): P[r = 16 rt + n][s = 16 st + 4 j + e] = exp(g_r - g_s) q_r.k_s
    // for s <= r, else 0. Written straight into its half (bf16) or whole (fp32) of the P fragment
    // [rt][st / FPD], whose lane (j, n) holds column r and k = s; the fragments take the place of
    // the K rows once every wave has read those (35 KB of LDS: four workgroups per CU, not three).
    f32x4 pts[OT::PER_WAVE];
#pragma unroll
    for (int x = 0; x < OT::PER_WAVE; ++x) {
        const int ti = w + 4 * x;
        if (ti < OT::N) {
            int rt, st;
            OT::tile(ti, rt, st);
            f32x4& pt = pts[x];
            pt = f32x4{0.f, 0.f, 0.f, 0.f};
            if (st <= rt) {
#pragma unroll
                for (int kd = 0; kd < NKD; ++kd)
                    pt = M::mma(row_frag_raw<E>(Kr + (16 * st + m) * KP, kd * KB, j),
                                row_frag_raw<E>(Qr + (16 * rt + m) * KP, kd * KB, j), pt);
                const int r = 16 * rt + m;
                const float gr = sg[r];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s2 = 16 * st + 4 * j + e;
                    pt[e] = (s2 <= r) ? pt[e] * __expf(gr - sg[s2]) : 0.f;
                }
            }
        }
    }
    lds_barrier();   // the K rows are read
#pragma unroll
    for (int x = 0; x < OT::PER_WAVE; ++x) {
        const int ti = w + 4 * x;
        if (ti < OT::N) {
            int rt, st;
            OT::tile(ti, rt, st);
            const f32x4 pt = pts[x];
            unsigned char* dst = sP + (size_t)(rt * NKT + st / FPD) * 1024 + lane * 16;
            if constexpr (FPD == 2) {
                *reinterpret_cast<uint2*>(dst + 8 * (st % 2)) = uint2{f2bf2(pt[0], pt[1]), f2bf2(pt[2], pt[3])};
            } else {
                *reinterpret_cast<f32x4*>(dst) = pt;
            }
        }
    }
    lds_barrier();
    // O^T tiles (vt, rt) = H^T e^g Q^T + U^T P^T: the state product with raw Q fragments, scaled
    // by e^{g_r} per token column, then the intra-chunk part accumulated on top. The Q fragments
    // are read one token tile at a time (the scheduling barrier keeps the compiler from reading
    // all sixteen ahead), which keeps the kernel within 128 VGPRs.
    float eg[4];
    f32x4 acc[NVW][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        eg[rt] = __expf(sg[16 * rt + m]);
        frag qf[NKD];
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) qf[kd] = row_frag_raw<E>(Qr + (16 * rt + m) * KP, kd * KB, j);
#pragma unroll
        for (int iv = 0; iv < NVW; ++iv) {
            acc[iv][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (w + 4 * iv < NDT) {
#pragma unroll
                for (int kd = 0; kd < NKD; ++kd) acc[iv][rt] = M::mma(Hc[iv][kd], qf[kd], acc[iv][rt]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int iv = 0; iv < NVW; ++iv) {
        const int vt = w + 4 * iv;
        if (vt >= NDT) break;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
            acc[iv][rt] = f32x4{acc[iv][rt][0] * eg[rt], acc[iv][rt][1] * eg[rt], acc[iv][rt][2] * eg[rt],
                                acc[iv][rt][3] * eg[rt]};
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                if (kt <= OT::kbmax(rt))
                    acc[iv][rt] = M::mma(Uf[iv][kt], ld_frag<frag>(sP + (rt * NKT + kt) * 1024, lane), acc[iv][rt]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            // lane (j, m): O[token 16 rt + m][16 vt + 4 j .. + 3]
            const int r = 16 * rt + m;
            if (r < n)
                store4(op + (size_t)r * D + 16 * vt + 4 * j,
                       make_float4(acc[iv][rt][0], acc[iv][rt][1], acc[iv][rt][2], acc[iv][rt][3]));
        }
    }
}

// h_final = h0 (or zeros) for L = 0
__global__ void copy_state_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

template <int D, class E, bool DELTA>
struct Launch {
    using T = typename E::T;
    using Ly = Layout<D, E>;
    using CC = ChainCfg<D, E, DELTA>;
    static constexpr int KP = D + 8;
    static constexpr size_t LDS_PREP = PrepCfg<D, E>::LDS;
    static constexpr size_t LDS_CHAIN = CC::LDS;
    static constexpr size_t LDS_OUT = (size_t)2 * CH * KP * sizeof(T) + CH * 4;   // Q rows, K rows / P, g
    // While the chain runs on some of the CUs, the prep and output stages beside it are held to
    // three workgroups per CU by asking for more than a quarter of the CU's 160 KB of LDS: more
    // concurrent stage work slows the latency-bound chain by more than it gains (B=1, H=16,
    // L=128K: 2.82 ms at four per CU, 2.75 ms at three, 2.87 ms at two).
    static constexpr size_t LDS_BESIDE = 41 * 1024;
    static constexpr size_t lds_prep(bool beside) { return beside && LDS_PREP < LDS_BESIDE ? LDS_BESIDE : LDS_PREP; }
    static constexpr size_t lds_out(bool beside) { return beside && LDS_OUT < LDS_BESIDE ? LDS_BESIDE : LDS_OUT; }

    // raise the dynamic-LDS limits once per process (every caller sets the same values)
    static bool attributes() {
        static const bool ok =
            hipFuncSetAttribute(reinterpret_cast<const void*>(&prep_kernel<D, E, DELTA>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_prep(true)) == hipSuccess &&
            hipFuncSetAttribute(reinterpret_cast<const void*>(&chain_kernel<D, E, DELTA>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_CHAIN) == hipSuccess &&
            hipFuncSetAttribute(reinterpret_cast<const void*>(&output_kernel<D, E, DELTA>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_out(true)) == hipSuccess;
        return ok;
    }
    static int chain_blocks(int BH) { return 8 * ((BH + 7) / 8) * CC::NCW; }
    static void prep(const PrefArgs& a, hipStream_t s, bool beside = false) {
        hipLaunchKernelGGL((prep_kernel<D, E, DELTA>), dim3(a.nseg, a.BH), dim3(256), lds_prep(beside), s, a);
    }
    static void chain(const PrefArgs& a, hipStream_t s) {
        hipLaunchKernelGGL((chain_kernel<D, E, DELTA>), dim3(chain_blocks(a.BH)), dim3(CC::THREADS), LDS_CHAIN, s, a);
    }
    static void output(const PrefArgs& a, hipStream_t s, bool beside = false) {
        hipLaunchKernelGGL((output_kernel<D, E, DELTA>), dim3(a.nseg, a.BH), dim3(256), lds_out(beside), s, a);
    }
};

// Two streams and an event per device, created on first use and kept for the process: the
// intra-chunk stage of later segments and the output stage of earlier ones run on them while
// the chain works on the current segment on the caller's stream.
struct StreamCtx {
    std::mutex mu;
    bool ready = false;
    int ncu = 0;   // compute units of the device
    hipStream_t sp = nullptr, so = nullptr;
    hipEvent_t start = nullptr;
};

static StreamCtx g_ctx[64];

static bool init_ctx(StreamCtx& c, int dev) {
    if (c.ready) return true;
    if (hipDeviceGetAttribute(&c.ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
    if (hipStreamCreateWithFlags(&c.sp, hipStreamNonBlocking) != hipSuccess) return false;
    if (hipStreamCreateWithFlags(&c.so, hipStreamNonBlocking) != hipSuccess) return false;
    if (hipEventCreateWithFlags(&c.start, hipEventDisableTiming) != hipSuccess) return false;
    c.ready = true;
    return true;
}

template <int D, class E, bool DELTA>
static int launch_prefill_t(PrefArgs a, long nch, size_t ws_bytes, hipStream_t stream) {
    using LN = Launch<D, E, DELTA>;
    if (!LN::attributes()) return -1;
    const size_t rec = Layout<D, E>::REC * (size_t)a.BH;
    if (ws_bytes >= (size_t)nch * rec) {   // whole sequence in one segment, caller's stream only
        a.c0 = 0; a.nseg = (int)nch; a.segcap = (int)nch;
        LN::prep(a, stream);
        LN::chain(a, stream);
        LN::output(a, stream);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    const int seg = (int)((ws_bytes - FLAG_BYTES) / (NBUF * rec));   // >= 1 (validated)
    const size_t buf = (size_t)seg * rec;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
    StreamCtx& cx = g_ctx[dev];
    std::lock_guard<std::mutex> lk(cx.mu);
    if (!init_ctx(cx, dev)) return -1;
    const bool beside = LN::chain_blocks(a.BH) < cx.ncu;   // the chain leaves CUs to the other stages
    unsigned char* ws0 = a.ws;
    const float* h0 = a.h0;
    // progress counters after the buffers, cleared on the caller's stream; the internal streams
    // start after that (and after the work already queued on the caller's stream)
    unsigned* done = reinterpret_cast<unsigned*>(ws0 + NBUF * buf);   // [0] prep, [1] chain, [2] output
    bool ok = true;
    for (int i = 0; i < 3; ++i) ok = ok && hipStreamWriteValue32(stream, done + i, 0u, 0) == hipSuccess;
    ok = ok && hipEventRecord(cx.start, stream) == hipSuccess && hipStreamWaitEvent(cx.sp, cx.start, 0) == hipSuccess &&
         hipStreamWaitEvent(cx.so, cx.start, 0) == hipSuccess;
    auto wait = [&](hipStream_t s, int which, int count) {
        return hipStreamWaitValue32(s, done + which, (unsigned)count, hipStreamWaitValueGte, 0xffffffffu) == hipSuccess;
    };
    auto mark = [&](hipStream_t s, int which, int count) {
        return hipStreamWriteValue32(s, done + which, (unsigned)count, 0) == hipSuccess;
    };
    const int nsegs = (int)((nch + seg - 1) / seg);
    for (int sgi = 0; ok && sgi < nsegs; ++sgi) {
        PrefArgs b = a;
        b.c0 = sgi * seg;
        b.nseg = (int)(nch - b.c0 < seg ? nch - b.c0 : seg);
        b.segcap = seg;
        b.ws = ws0 + (size_t)(sgi % NBUF) * buf;
        b.h0 = sgi == 0 ? h0 : a.h_final;   // later segments continue from the running state
        // the buffer is free once the output stage of the segment NBUF back has read it. (Its
        // halves are used by different stages, but letting prep start once that segment's chain
        // is done puts three kernels on the memory system at once and slows the chain more than
        // it saves.) Each counter is written after its stage's kernel completes, so a stage
        // waiting for a count sees that kernel's results.
        if (sgi >= NBUF) ok = ok && wait(cx.sp, 2, sgi - NBUF + 1);
        LN::prep(b, cx.sp, beside);
        ok = ok && mark(cx.sp, 0, sgi + 1) && wait(stream, 0, sgi + 1);
        LN::chain(b, stream);
        ok = ok && mark(stream, 1, sgi + 1) && wait(cx.so, 1, sgi + 1);
        LN::output(b, cx.so, beside);
        ok = ok && mark(cx.so, 2, sgi + 1);
    }
    // the caller's stream continues only after the last output stage
    ok = ok && wait(stream, 2, nsegs);
    return ok && hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_prefill(const void* q, const void* k, const void* v, const float* beta, const float* log_alpha,
                   const unsigned char* keep, const float* h0, void* o, float* h_final, int BH, long L, int D,
                   int dtype, bool delta, int band, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (L == 0) {
        const size_t n = (size_t)BH * D * D;
        if (h0 == h_final) return 0;
        hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, h0, h_final, n);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    const long nch = (L + CH - 1) / CH;
    PrefArgs a{q, k, v, beta, log_alpha, h0, o, h_final, static_cast<unsigned char*>(ws), L, BH, 0, 0, 0, keep, (int)nch,
               band};
#define GDN_PF(DD, EE)                                                                 \
    return delta ? launch_prefill_t<DD, EE, true>(a, nch, ws_bytes, stream)            \
                 : launch_prefill_t<DD, EE, false>(a, nch, ws_bytes, stream)
    if (D == 128 && dtype == 0) GDN_PF(128, BF16);
    if (D == 128) GDN_PF(128, F32);
    if (dtype == 0) GDN_PF(64, BF16);
    GDN_PF(64, F32);
#undef GDN_PF
}

}  // namespace gdn
