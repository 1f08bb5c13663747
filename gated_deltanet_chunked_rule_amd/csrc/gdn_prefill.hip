// Chunked prefill of the gated delta rule on gfx950.
//
// The SparseGDN article (fileenergy.com, section "Why GDN prefill is expensive") splits chunked
// GDN prefill into three sources of work: the intra-chunk delta-system solve, the sequential
// chunk-to-chunk state pass for each head, and the outputs computed from every chunk's start
// state. Here the first is one kernel and the other two share the second.
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
//                 a blocked inverse in LDS, then -W, Khat^T, Ut, the gated causal P^T and Q,
//                 written as MFMA-ready fragments into the chunk's record.
//   chain_kernel  (one workgroup per head and 16 value columns): the sequential pass. The fp32
//                 state stays in accumulator registers for the whole sequence while loader
//                 waves stream the next chunks' records into an LDS ring; output waves form
//                 O^T = e^g H^T Q^T + U^T P^T from the state and U the compute waves hand them,
//                 and store waves write it.
// Long sequences run as segments through a pair of workspace buffers: prep of later segments
// on a side stream beside the chain of the current one on the caller's stream.
#include <mutex>
#include <type_traits>

#include "gdn_launch.h"
#include "gdn_rows.h"

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
    // chunk record, written by prep and read by the chain:
    //   -W [rt 4][NKD] and Khat^T [dt NDT][NKT] fragments (streamed whole into the chain's LDS),
    //   Ut accumulators [vt NDT][rt 4][lane] (4 x T), Q fragments [rt 4][NKD] (k = d, column =
    //   token), the gated causal P^T fragments [rt 4][NKT] (kt <= kbmax(rt) written), e^g per
    //   token, the chunk decay e^{g_C} and the keep flag
    static constexpr size_t A_W = 0;
    static constexpr size_t A_KH = A_W + (size_t)4 * NKD * FR;
    static constexpr size_t A_UT = A_KH + (size_t)NDT * NKT * FR;
    static constexpr size_t A_Q = A_UT + (size_t)NDT * 4 * 64 * 4 * sizeof(typename E::T);
    static constexpr size_t A_P = A_Q + (size_t)4 * NKD * FR;
    static constexpr size_t A_EG = A_P + (size_t)4 * NKT * FR;
    static constexpr size_t A_DEC = A_EG + (size_t)CH * 4;
    static constexpr size_t A_KEEP = A_DEC + 4;   // u32, 0 = skipped state update
    static constexpr size_t REC = (A_KEEP + 4 + 255) / 256 * 256;
    // last d-fragment of P^T's token-column tile rt that holds any s <= r
    static constexpr int kbmax(int rt) { return (16 * rt + 15) / KB; }
};

size_t prefill_record_bytes(int D, int dtype) {
    if (D == 128 && dtype == 0) return Layout<128, BF16>::REC;
    if (D == 128) return Layout<128, F32>::REC;
    if (D == 64 && dtype == 0) return Layout<64, BF16>::REC;
    return Layout<64, F32>::REC;
}

// Preferred workspace: the whole sequence if it is short, else NBUF segment buffers of about
// SEG_TARGET bytes each, so that the two stages of consecutive segments overlap and the buffers
// can stay resident in the 256 MB Infinity Cache between the stage that writes them and the
// stage that reads them.
static constexpr size_t SEG_TARGET = (size_t)72 << 20;
static constexpr int NBUF = 2;
// A segmented call keeps 32-bit progress counters after its buffers; the streams wait on them
// (hipStreamWaitValue32) rather than on events, which measured about 5 us less per cross-stream
// hand-off.
static constexpr size_t FLAG_BYTES = 256;

// Where the chain's workgroups fill every CU of the device, prep cannot run beside it and the two
// stages alternate segment by segment; the fewest hand-offs then win, so the preferred workspace
// holds the whole sequence's records if they take at most WHOLE_MAX bytes (B=1, H=32, L=32768:
// 1.31 ms in 72 MB segments, 1.06 ms in one).
static constexpr size_t WHOLE_MAX = (size_t)2 << 30;

static int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return n;
}

size_t prefill_workspace_bytes(long BH, long L, int D, int dtype) {
    const long nch = (L + CH - 1) / CH;
    const size_t rec = prefill_record_bytes(D, dtype) * (size_t)BH;   // one chunk of every slice
    const long chain_wgs = 8 * ((BH + 7) / 8) * (D / 16);             // the chain's grid
    const int ncu = device_cus();
    if (ncu > 0 && chain_wgs >= ncu && (size_t)nch * rec <= WHOLE_MAX) return (size_t)nch * rec;
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
    unsigned* flags;             // segment pipeline counters, or NULL (the call is one segment)
    int sgi;                     // this launch's segment
};


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
// segment pipeline counters
// ---------------------------------------------------------------------------------------------
// A segmented call keeps 32-bit words in the workspace after its segment buffers: for each stage
// the number of segments it has finished, the chain's arrival count and an error word. The side
// stream waits on the chain's count with hipStreamWaitValue32; the chain kernel polls the prep
// count itself and publishes its own, so that consecutive chain launches follow each other on
// their stream with nothing queued between them.
enum : int { FL_PREP = 0, FL_CHAIN = 1, FL_ERR = 3, FL_ARRIVE = 16, FL_WORDS = 64 };
// about 10 s of the 100 MHz constant clock (s_memrealtime)
static constexpr unsigned long long WAIT_TICKS = 1000000000ull;

// Wait (the whole wave, polling one word) until flags[which] >= target, then acquire, so that
// this wave's later loads see what the stage that published the count wrote. A wait longer than
// WAIT_TICKS gives up and sets the error word rather than spin for ever; the call's outputs and
// final state then come out NaN.
__device__ __forceinline__ void wait_count(unsigned* flags, int which, unsigned target) {
    auto rd = [&] { return __hip_atomic_load(flags + which, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM); };
    if (rd() < target) {
        const unsigned long long t0 = wall_clock64();
        while (rd() < target) {
            __builtin_amdgcn_s_sleep(1);
            if (wall_clock64() - t0 > WAIT_TICKS) {
                __hip_atomic_store(flags + FL_ERR, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                break;
            }
            // after one timeout the call's result is lost anyway: later waits end at once
            if (__hip_atomic_load(flags + FL_ERR, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)) break;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Count this wave in among the `waves` waves of a stage launch that only read the segment's
// buffer; the last to arrive resets the arrival count (launches of a stage run in order on one
// stream) and publishes `value`. The count licenses the next writer of the buffer, so it only has
// to follow the wave's reads: the caller has waited for all of them (vmcnt 0), and nothing this
// launch wrote is needed by that writer, so no cache write-back is needed either.
__device__ __forceinline__ void publish_read(unsigned* flags, int which, unsigned value, unsigned waves, int lane) {
    if (lane == 0) {
        unsigned* arrive = flags + FL_ARRIVE + which;
        const unsigned n = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (n + 1 == waves) {
            __hip_atomic_store(arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(flags + which, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
}

// nonzero once a wait of this call has timed out (scalar, for uniform branches)
__device__ __forceinline__ unsigned call_failed(const PrefArgs& a) {
    return a.flags ? __builtin_amdgcn_readfirstlane(
                         __hip_atomic_load(a.flags + FL_ERR, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM))
                   : 0u;
}

__global__ void flags_reset_kernel(unsigned* flags) { flags[threadIdx.x] = 0u; }

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
    // region 0: K rows, then T; region 1: V rows, then A; four per-token arrays; Q rows
    static constexpr size_t REGION = ((ROWS > MAT ? ROWS : MAT) + 15) / 16 * 16;
    static constexpr size_t O_Q = 2 * REGION + 4 * CH * 4;
    static constexpr size_t LDS = O_Q + (ROWS + 15) / 16 * 16;
};

template <int D, class E>
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
    T* Qr = reinterpret_cast<T*>(smem + P::O_Q);                      // [CH][KP] Q rows

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
    const T* qp = static_cast<const T*>(a.q) + tok0 * D;
    const T* kp = static_cast<const T*>(a.k) + tok0 * D;
    const T* vp = static_cast<const T*>(a.v) + tok0 * D;
    unsigned char* rec = a.ws + ((size_t)bh * a.segcap + cl) * Ly::REC;

    if (w == 0) {
        float la = 0.f, bt = 0.f;
        if (lane < n) {
            la = a.log_alpha[tok0 + lane];
            bt = a.beta[tok0 + lane];
        }
        const float g = wave_scan(la, lane);
        const float gC = __shfl(g, 63);
        const float eg = __expf(g);
        sg[lane] = g;
        sb[lane] = bt;
        sbe[lane] = -bt * eg;
        skh[lane] = __expf(gC - g);
        reinterpret_cast<float*>(rec + Ly::A_EG)[lane] = eg;
        if (lane == 0) {
            *reinterpret_cast<float*>(rec + Ly::A_DEC) = __expf(gC);
            *reinterpret_cast<unsigned*>(rec + Ly::A_KEEP) =
                a.keep ? (a.keep[(size_t)bh * a.nchk + a.c0 + cl] != 0 ? 1u : 0u) : 1u;
        }
    }
    {   // Q, K and V rows, 16 bytes per lane, all loads in flight at once; rows past the
        // chunk's end read as zero (identity steps)
        constexpr int EPU = 16 / sizeof(T), UPR = D / EPU, NU = CH * UPR / 256;
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(qp, n * D * (int)sizeof(T));
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kp, n * D * (int)sizeof(T));
        const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vp, n * D * (int)sizeof(T));
        uint4 xq[NU], xk[NU], xv[NU];
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            xk[i] = buffer_load16(rk, (tid + 256 * i) * 16);
            xv[i] = buffer_load16(rv, (tid + 256 * i) * 16);
            xq[i] = buffer_load16(rq, (tid + 256 * i) * 16);
        }
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = tid + 256 * i, r = u / UPR, cu = u % UPR;
            *reinterpret_cast<uint4*>(Kr + r * KP + cu * EPU) = xk[i];
            *reinterpret_cast<uint4*>(Vr + r * KP + cu * EPU) = xv[i];
            *reinterpret_cast<uint4*>(Qr + r * KP + cu * EPU) = xq[i];
        }
    }
    lds_barrier();

    // Q as MFMA fragments for the chain's H^T Q^T (one contiguous 1 KB load each there)
    for (int f = w; f < 4 * NKD; f += 4)
        st_frag(rec + Ly::A_Q + (size_t)f * Ly::FR, lane,
                row_frag_raw<E>(Qr + (16 * (f / NKD) + m) * KP, (f % NKD) * KB, j));
    // The chain computes the outputs; what it needs of the chunk beyond the state is the gated
    // causal P^T. Fragment (rt, kt) packs the tiles (st, rt), st = FPD kt .. FPD kt + FPD - 1,
    // whose lane (j, n) holds P[r = 16 rt + n][s = 16 st + 4 j + e] = exp(g_r - g_s) q_r.k_s for
    // s <= r, else 0: the B operand (k = s, column r) of O^T += U^T P^T. Only kt <= kbmax(rt)
    // is written (the rest is all zero and never read).
    {
        constexpr int NPFR = [] {
            int c = 0;
            for (int rt = 0; rt < 4; ++rt) c += Ly::kbmax(rt) + 1;
            return c;
        }();
        for (int f = w; f < NPFR; f += 4) {   // w is scalar: so is every branch below
            int rt = 0, kt = f;
            while (kt > Ly::kbmax(rt)) { kt -= Ly::kbmax(rt) + 1; ++rt; }
            f32x4 t[FPD];
#pragma unroll
            for (int i = 0; i < FPD; ++i) {
                const int st = FPD * kt + i;
                t[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (st <= rt) {
                    // gates first, read for every lane (selected below, no lane-masked branch)
                    const int r = 16 * rt + m;
                    const float4 gs = *reinterpret_cast<const float4*>(sg + 16 * st + 4 * j);
                    const float gr = sg[r];
                    const int s0 = 16 * st + 4 * j;   // s <= r: exp(g_r - g_s); else exp(0), masked below
                    const float ge[4] = {__expf(s0 <= r ? gr - gs.x : 0.f), __expf(s0 + 1 <= r ? gr - gs.y : 0.f),
                                         __expf(s0 + 2 <= r ? gr - gs.z : 0.f), __expf(s0 + 3 <= r ? gr - gs.w : 0.f)};
#pragma unroll
                    for (int kd = 0; kd < NKD; ++kd)
                        t[i] = M::mma(row_frag_raw<E>(Kr + (16 * st + m) * KP, kd * KB, j),
                                      row_frag_raw<E>(Qr + (16 * rt + m) * KP, kd * KB, j), t[i]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)   // t finite: the 0/1 factor masks exactly
                        t[i][e] *= ge[e] * (float)(s0 + e <= r);
                }
            }
            st_frag(rec + Ly::A_P + (size_t)(rt * NKT + kt) * Ly::FR, lane, M::from_acc(t, 0));
        }
    }

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

    {
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
// MFMA work. The two loader waves stream each chunk's -W and Khat^T fragments (contiguous at
// the start of its record, shared by all column groups of the slice) and the group's Ut tiles
// into a ring of NS LDS slots, NS - 1 chunks ahead; they issue nothing else, so their waits are
// fixed counts.
//
// The workgroup also produces the chunk's outputs for its 16 columns,
//     O^T = e^g (H^T Q^T) + U^T P^T,
// from the chunk-start state and U. Two further output waves do it: the compute waves stage
// their bf16 state half and U fragments in LDS (three steps deep), and each output wave
// finishes two token tiles ({0, 3} or {1, 2}: equal causal P work) one step later with the Q
// and P^T fragments and e^g of the record, read into registers NSET chunks ahead. The finished
// tiles go through LDS to two store waves, which write them to memory a step later: a wave's
// loads and stores share one in-order completion count, so loads issued after stores could not
// be waited for without also waiting for the stores. Waves are dealt to the four SIMDs in
// order: compute 0, 1 and output 2, 3 on their own SIMDs, the loaders 4, 5 and store waves
// 6, 7 beside them (they mostly wait). Where the staging does not fit beside the ring (fp32 at
// Dk = 128) the compute waves form and store the outputs themselves, handing each other their
// halves of H^T Q^T through LDS; that puts the output work on the chain's dependence path.
template <int D, class E>
struct ChainCfg {
    using Ly = Layout<D, E>;
    static constexpr int NCW = D / 16;                                   // workgroups per slice
    static constexpr size_t SLOT = Ly::A_UT;                             // -W and Khat^T fragments
    static constexpr int NBLK = (int)(SLOT / 1024);                      // 1 KB wave blocks per slot
    static constexpr int BPW = NBLK / 2;                                 // blocks per loader wave
    static_assert(SLOT % 2048 == 0, "slot splits into whole blocks per loader wave");
    static constexpr size_t UTSUB = (size_t)4 * 64 * 4 * sizeof(typename E::T);  // Ut bytes of 16 columns
    static constexpr int UTL = (int)(UTSUB / 2048);                      // Ut 1 KB loads per loader wave
    static_assert(UTSUB % 2048 == 0, "Ut splits into whole blocks per loader wave");
    static constexpr int DMA_OPS = BPW + UTL;                            // loads per loader wave and chunk
    static constexpr size_t XHALF = (size_t)4 * 64 * 16;                 // one wave's partial W H
    static constexpr size_t XBYTES = (size_t)2 * 2 * XHALF;             // [step parity][half]
    static constexpr size_t LDS_MAX = 160 * 1024;                        // gfx950: 160 KB per workgroup
    // output waves: one step's staged bf16 H (both halves) and U fragments, three steps deep
    static constexpr size_t STB = (size_t)(Ly::NKD + Ly::NKT) * 1024;
    // and the finished output tiles for the store waves: [step parity][rt][lane], 4 elements
    static constexpr size_t OTB = (size_t)4 * 64 * 4 * sizeof(typename E::T);
    static constexpr size_t STAGE = 3 * STB + 2 * OTB;
    static constexpr bool OUTW = (SLOT + UTSUB) * 2 + XBYTES + STAGE <= LDS_MAX;
    static constexpr int THREADS = OUTW ? 512 : 256;
    // waves per workgroup that read the records after the compute waves' last barrier and so
    // count themselves in for the segment's "read" count: the loaders, and the output waves
    static constexpr unsigned READERS = OUTW ? 4 : 2;
    // outputs in the compute waves instead: H^T Q^T halves [parity][writer][tile][lane]
    static constexpr size_t XOBYTES = (size_t)2 * 2 * 2 * 64 * 16;
    static constexpr size_t FIXED = XBYTES + (OUTW ? STAGE : XOBYTES);
    static constexpr int NS = (SLOT + UTSUB) * 4 + FIXED <= LDS_MAX ? 4 : ((SLOT + UTSUB) * 3 + FIXED <= LDS_MAX ? 3 : 2);
    static constexpr size_t O_X = NS * SLOT;                             // LDS offsets of the areas
    static constexpr size_t O_ST = O_X + XBYTES;                         // staging (output waves) or
    static constexpr size_t O_OT = O_ST + 3 * STB;                       //   and their output tiles, or
    static constexpr size_t O_XO = O_X + XBYTES;                         // H^T Q^T halves (in-wave outputs)
    static constexpr size_t O_UT = O_X + FIXED;
    static constexpr size_t LDS = O_UT + NS * UTSUB;
    static_assert(LDS <= LDS_MAX, "chain LDS");
    // a loader's loads still in flight when it waits for chunk c + 1: those of the NS - 2 later chunks
    static constexpr int WAITN = (NS - 2) * DMA_OPS;
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
// be made to wait on them.
// M0 is a reserved register, so clang warns about the clobber; the kernels that call dma16 use
// M0 for nothing else, and the asm sets it before each load.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, unsigned lds_base) {
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);   // wave-uniform by construction
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// Loader wave lw's share of chunk c's loads into slot s: BPW 1 KB blocks of the -W / Khat^T
// fragments (interleaved with the other loader's) and its half of the Ut tiles.
template <int D, class E>
__device__ __forceinline__ void chain_issue(unsigned char* smem, const unsigned char* rec, int s, int cg, int lw,
                                            int lane) {
    using C = ChainCfg<D, E>;
    using Ly = Layout<D, E>;
    const unsigned base = lds_addr(smem + (size_t)s * C::SLOT);
    // The column groups of a slice read the same fragments at about the same time; each starts at
    // a different block, so that their requests go to different L2 channels at any moment rather
    // than queueing eight deep on one (B=1 H=16 L=128K, chain alone: 2.0 -> 1.75 ms).
    const int rot = (cg * C::BPW / C::NCW) % C::BPW;   // < BPW
#pragma unroll
    for (int i = 0; i < C::BPW; ++i) {
        int ii = i + rot;
        ii = ii >= C::BPW ? ii - C::BPW : ii;
        const unsigned blk = (unsigned)(lw + 2 * ii) * 1024u;
        dma16(rec + blk + lane * 16, base + blk);
    }
    const unsigned ubase = lds_addr(smem + C::O_UT + (size_t)s * C::UTSUB);
    const unsigned char* ut = rec + Ly::A_UT + (size_t)cg * C::UTSUB;
#pragma unroll
    for (int i = 0; i < C::UTL; ++i) {
        const unsigned blk = (unsigned)(lw * C::UTL + i) * 1024u;
        dma16(ut + blk + lane * 16, ubase + blk);
    }
}

// Loader wave lw (0 or 1) of a chain workgroup. Iteration c (after barrier c - 1): issue chunk
// c + NS - 1 into the slot of chunk c - 1 (whose fragments the compute waves read before
// barrier c - 1), wait for chunk c + 1 (read by the compute waves after barrier c), barrier c.
// In a segmented call it first waits for the segment's prep count, and at the end counts itself
// in for the chain's: the count tells the prep stage that this launch has read its buffer.
template <int D, class E>
__device__ __forceinline__ void chain_loader(const PrefArgs& a, unsigned char* smem, const unsigned char* rec0, int nch,
                                             int cg, int lw, int lane) {
    using Ly = Layout<D, E>;
    using C = ChainCfg<D, E>;
    constexpr int NS = C::NS;
    if (a.flags) wait_count(a.flags, FL_PREP, (unsigned)a.sgi + 1);   // the segment's records are written
    for (int c = 0; c < NS - 1; ++c)
        chain_issue<D, E>(smem, rec0 + (size_t)min(c, nch - 1) * Ly::REC, c, cg, lw, lane);
    wait_vmcnt<0>();
    lds_barrier();
    for (int c = 0; c < nch; ++c) {
        const int cn = c + NS - 1;   // always issued (clamped to the last chunk): fixed counts
        chain_issue<D, E>(smem, rec0 + (size_t)min(cn, nch - 1) * Ly::REC, cn % NS, cg, lw, lane);
        wait_vmcnt<C::WAITN>();
        lds_barrier();
    }
    lds_barrier();   // matches the compute waves' last barrier
    wait_vmcnt<0>();   // no LDS write may land after the workgroup ends
    if (a.flags) publish_read(a.flags, FL_CHAIN, (unsigned)a.sgi + 1, C::READERS * a.BH * C::NCW, lane);
}

// Output tile (O^T, lane (j, m): O[token 16 rt + m][16 cg + 4 j .. + 3]) of token tile rt of the
// segment's chunk c; tokens past the end of the sequence are dropped.
template <int D, class E>
__device__ __forceinline__ void store_out(const PrefArgs& a, int bh, int cg, int c, int rt, int lane, const f32x4& v) {
    using T = typename E::T;
    const long t0 = (long)(a.c0 + c) * CH;
    const int n = (int)min((long)CH, a.L - t0);
    const __amdgpu_buffer_rsrc_t ro =
        buffer_rsrc(static_cast<T*>(a.o) + ((size_t)bh * a.L + t0) * D, n * D * (int)sizeof(T));
    const int j = lane >> 4, m = lane & 15;
    buffer_store4(ro, ((16 * rt + m) * D + 16 * cg + 4 * j) * (int)sizeof(T), make_float4(v[0], v[1], v[2], v[3]), T{});
}

// Packed output tile element of this lane: 4 elements of T (8 or 16 bytes)
template <class E>
using OutPack = typename std::conditional<sizeof(typename E::T) == 2, uint2, uint4>::type;
template <class E>
__device__ __forceinline__ OutPack<E> pack_out(const f32x4& v) {
    if constexpr (sizeof(typename E::T) == 2)
        return uint2{f2bf2(v[0], v[1]), f2bf2(v[2], v[3])};
    else
        return uint4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
}
template <int D, class E>
__device__ __forceinline__ void store_packed(const PrefArgs& a, int bh, int cg, int c, int rt, int lane, OutPack<E> x) {
    using T = typename E::T;
    const long t0 = (long)(a.c0 + c) * CH;
    const int n = (int)min((long)CH, a.L - t0);
    const __amdgpu_buffer_rsrc_t ro =
        buffer_rsrc(static_cast<T*>(a.o) + ((size_t)bh * a.L + t0) * D, n * D * (int)sizeof(T));
    const int j = lane >> 4, m = lane & 15;
    const int off = ((16 * rt + m) * D + 16 * cg + 4 * j) * (int)sizeof(T);
    if constexpr (sizeof(T) == 2) {
        typedef int i32x2_t __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(i32x2_t{(int)x.x, (int)x.y}, ro, off, 0, 0);
    } else {
        typedef int i32x4_t __attribute__((ext_vector_type(4)));
        __builtin_amdgcn_raw_buffer_store_b128(i32x4_t{(int)x.x, (int)x.y, (int)x.z, (int)x.w}, ro, off, 0, 0);
    }
}

// Compute wave HH of a chain workgroup: it owns state rows [HH Dk/2, (HH + 1) Dk/2) of column
// group cg. Per chunk c:
//   A  Hf = bf16(H); partial product P_HH = (-W)[:, half] Hf, with Ut folded into the
//      accumulators of token tiles 2 HH and 2 HH + 1; P_HH -> LDS; H *= chunk decay.
//   B  U = P_HH + P_other (fp32 addition is commutative, so both waves hold the same U);
//      H += Khat^T[half, :] bf16(U); chunk c + 1's -W and Khat^T fragments are read from its
//      slot (complete since barrier c), so neither product of the next step waits on LDS.
//   With output waves, bf16(H) is staged in A and bf16(U) in B. Without, B ends with the
//      outputs: H^T Q^T over the wave's half of d for the four token tiles, the other wave's
//      two to LDS, its own two scaled by e^g and U^T P^T added; the other wave's half for its
//      own tiles of chunk c - 1 (stored before barrier c) completes chunk c - 1's outputs.
// One barrier per step, between A and B: the partial products alternate between two LDS areas
// by step parity, so an area is rewritten only after the partner has passed the next barrier.
// Ut is read in A, before the barrier after which its slot may be refilled.
template <int D, class E, int HH>
__device__ __forceinline__ void chain_compute(const PrefArgs& a, unsigned char* smem, const unsigned char* rec0,
                                              int nch, int bh, int cg, int lane) {
    using T = typename E::T;
    using M = MM<E>;
    using Ly = Layout<D, E>;
    using C = ChainCfg<D, E>;
    using frag = typename M::frag;
    constexpr int NKD = Ly::NKD, NKT = Ly::NKT, NDT = Ly::NDT, NS = C::NS;
    constexpr int HKD = NKD / 2, HDT = NDT / 2;   // fragments / tiles of one row half
    // token tiles this wave finishes, and the P^T fragments they need
    constexpr int R[2] = {HH == 0 ? 0 : 1, HH == 0 ? 3 : 2};
    constexpr int RO[2] = {HH == 0 ? 1 : 0, HH == 0 ? 2 : 3};   // the other wave's
    constexpr int NP0 = Ly::kbmax(R[0]) + 1, NPF = NP0 + Ly::kbmax(R[1]) + 1;
    f32x4* X0 = reinterpret_cast<f32x4*>(smem + C::O_X);                   // [parity][half][rt][lane]
    constexpr size_t XPAR = 2 * C::XHALF / sizeof(f32x4);
    f32x4* XO = reinterpret_cast<f32x4*>(smem + C::O_XO);                  // [parity][writer][tile][lane]
    const int j = lane >> 4, m = lane & 15;
    const int col = 16 * cg + m;
    f32x4 H[HDT];   // lane (j, m): H[16 (HH HDT + t) + 4 j + e][col]
#pragma unroll
    for (int t = 0; t < HDT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            H[t][e] = a.h0 ? a.h0[((size_t)bh * D + 16 * (HH * HDT + t) + 4 * j + e) * D + col] : 0.f;

    // what a step reads from global memory, two chunks ahead
    struct Pre {
        frag qf[4][HKD];   // Q fragments, k = d over this wave's half, column = token
        frag pf[NPF];      // P^T fragments of tiles R[0], R[1]
        float eg[2];       // e^{g_r} of this lane's token in tiles R[0], R[1]
        unsigned dec, keep;
    };
    auto load = [&](Pre& p, int c) {
        c = min(c, nch - 1);   // past the segment: the last chunk again (unused)
        const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(rec0 + (size_t)c * Ly::REC, (int)Ly::REC);
        // the decay and keep flag first: a step needs them first, and waits are in issue order
        p.dec = buffer_load4(rr, (int)Ly::A_DEC);
        p.keep = buffer_load4(rr, (int)Ly::A_KEEP);
        if constexpr (C::OUTW) return;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int kk = 0; kk < HKD; ++kk)
                p.qf[rt][kk] = __builtin_bit_cast(
                    frag, buffer_load16(rr, (int)Ly::A_Q + (rt * NKD + HH * HKD + kk) * Ly::FR + lane * 16));
#pragma unroll
        for (int i = 0; i < NPF; ++i) {
            const int rt = i < NP0 ? R[0] : R[1], kt = i < NP0 ? i : i - NP0;
            p.pf[i] = __builtin_bit_cast(frag, buffer_load16(rr, (int)Ly::A_P + (rt * NKT + kt) * Ly::FR + lane * 16));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) p.eg[i] = __uint_as_float(buffer_load4(rr, (int)Ly::A_EG + (16 * R[i] + m) * 4));
    };

    // -W and Khat^T fragments of the chunk in slot s
    frag wf[4 * HKD], kf[HDT * NKT];
    auto read_slot = [&](int s) {
        const unsigned char* slot = smem + (size_t)s * C::SLOT;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int kk = 0; kk < HKD; ++kk)
                wf[rt * HKD + kk] = ld_frag<frag>(slot + Ly::A_W + (size_t)(rt * NKD + HH * HKD + kk) * Ly::FR, lane);
#pragma unroll
        for (int t = 0; t < HDT; ++t)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
                kf[t * NKT + kt] = ld_frag<frag>(slot + Ly::A_KH + (size_t)((HH * HDT + t) * NKT + kt) * Ly::FR, lane);
    };

    f32x4 on[2];     // chunk c - 1's own tiles without the other wave's half of H^T Q^T
    float egp[2];    // and their e^g
    // the records may be read only after this barrier: before it the loaders wait for the
    // segment's prep count (and acquire)
    lds_barrier();
    // NSET register sets: chunk c's loads are issued at the start of step c - NSET + 1 (two
    // for fp32 at Dk = 128, whose fragments are twice the size: four would spill)
    constexpr int NSET = sizeof(T) == 4 && D == 128 ? 2 : 4;
    Pre S[NSET];
#pragma unroll
    for (int i = 0; i < NSET - 1; ++i) load(S[i], i);
    const float bad = call_failed(a) ? __builtin_nanf("") : 0.f;   // NaN outputs after a timed-out wait
    read_slot(0);

    auto step = [&](int c, Pre& S, Pre& N) {
        load(N, c + NSET - 1);   // into the set of chunk c - 1, read in the step before
        f32x4* X = X0 + (c & 1) * XPAR;
        const unsigned char* us = smem + C::O_UT + (size_t)(c % NS) * C::UTSUB;
        const T* ut = reinterpret_cast<const T*>(us);   // [rt][lane][4]
        unsigned char* st = smem + C::O_ST + (size_t)(c % 3) * C::STB;   // (output waves)
        frag Hf[HKD];
#pragma unroll
        for (int kk = 0; kk < HKD; ++kk) {
            Hf[kk] = M::from_acc(H, kk);
            if constexpr (C::OUTW) st_frag(st + (size_t)(HH * HKD + kk) * 1024, lane, Hf[kk]);
        }
        f32x4 P[4];
        const float dec = __uint_as_float(S.dec);
        const unsigned keep = __builtin_amdgcn_readfirstlane(S.keep);
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
        lds_barrier();   // partial products exchanged; chunk c + 1's slot is complete
        f32x4 U[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const f32x4 po = X[((1 - HH) * 4 + rt) * 64 + lane];
            U[rt] = f32x4{P[rt][0] + po[0], P[rt][1] + po[1], P[rt][2] + po[2], P[rt][3] + po[3]};
        }
        frag Uf[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            Uf[kt] = M::from_acc(U, kt);
            if constexpr (C::OUTW)
                if (kt % 2 == HH) st_frag(st + (size_t)(NKD + kt) * 1024, lane, Uf[kt]);
        }
        if (keep) {   // a skipped chunk's update leaves the decayed state (its U still feeds its outputs)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int t = 0; t < HDT; ++t) H[t] = M::mma(kf[t * NKT + kt], Uf[kt], H[t]);
        }
        read_slot((c + 1) % NS);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (C::OUTW) return;
        // outputs of chunk c: H^T Q^T over this wave's half of d
        f32x4 qh[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            qh[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < HKD; ++kk) qh[rt] = M::mma(Hf[kk], S.qf[rt][kk], qh[rt]);
        }
        f32x4* xo = XO + ((size_t)((c & 1) * 2 + HH) * 2) * 64;
        xo[lane] = qh[RO[0]];
        xo[64 + lane] = qh[RO[1]];
        f32x4 oc[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float g = S.eg[i];
            oc[i] = f32x4{qh[R[i]][0] * g, qh[R[i]][1] * g, qh[R[i]][2] * g, qh[R[i]][3] * g};
#pragma unroll
            for (int kt = 0; kt <= Ly::kbmax(R[i]); ++kt) oc[i] = M::mma(Uf[kt], S.pf[i == 0 ? kt : NP0 + kt], oc[i]);
        }
        // chunk c - 1: the other wave's half, stored before barrier c
        if (c > 0) {
            const f32x4* xp = XO + ((size_t)(((c - 1) & 1) * 2 + 1 - HH) * 2) * 64;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const f32x4 x = xp[i * 64 + lane];
                store_out<D, E>(a, bh, cg, c - 1, R[i], lane,
                                f32x4{on[i][0] + egp[i] * x[0] + bad, on[i][1] + egp[i] * x[1] + bad,
                                      on[i][2] + egp[i] * x[2] + bad, on[i][3] + egp[i] * x[3] + bad});
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            on[i] = oc[i];
            egp[i] = S.eg[i];
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int c = 0; c < nch; c += NSET) {
#pragma unroll
        for (int u = 0; u < NSET; ++u)
            if (u == 0 || c + u < nch) step(c + u, S[u], S[(u + NSET - 1) % NSET]);
    }
    lds_barrier();   // the last step's H^T Q^T halves (or staged fragments) are in LDS
    if constexpr (!C::OUTW) {
        const int c = nch - 1;
        const f32x4* xp = XO + ((size_t)((c & 1) * 2 + 1 - HH) * 2) * 64;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const f32x4 x = xp[i * 64 + lane];
            store_out<D, E>(a, bh, cg, c, R[i], lane,
                            f32x4{on[i][0] + egp[i] * x[0] + bad, on[i][1] + egp[i] * x[1] + bad,
                                  on[i][2] + egp[i] * x[2] + bad, on[i][3] + egp[i] * x[3] + bad});
        }
    }
    if (call_failed(a))
#pragma unroll
        for (int t = 0; t < HDT; ++t) H[t] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
#pragma unroll
    for (int t = 0; t < HDT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            a.h_final[((size_t)bh * D + 16 * (HH * HDT + t) + 4 * j + e) * D + col] = H[t][e];
}

// Output wave HH of a chain workgroup (with output waves): it finishes token tiles {0, 3}
// (HH = 0) or {1, 2} of every chunk of the column group. Iteration c follows barrier c of the
// compute waves, after which step c - 1's staged bf16 H and U are complete: O^T of chunk c - 1 =
// e^g (H^T Q^T) + U^T P^T over all of d, then the loads of chunk c - 1 + NSET into the register
// set just used, then the tiles into LDS for the store waves (the last chunk's it stores
// itself). Its barrier sequence is the compute waves': the first, one per step, the last.
template <int D, class E, int HH>
__device__ __forceinline__ void chain_output(const PrefArgs& a, unsigned char* smem, const unsigned char* rec0,
                                             int nch, int bh, int cg, int lane) {
    using M = MM<E>;
    using Ly = Layout<D, E>;
    using C = ChainCfg<D, E>;
    using frag = typename M::frag;
    constexpr int NKD = Ly::NKD, NKT = Ly::NKT;
    constexpr int R[2] = {HH == 0 ? 0 : 1, HH == 0 ? 3 : 2};
    constexpr int NP0 = Ly::kbmax(R[0]) + 1, NPF = NP0 + Ly::kbmax(R[1]) + 1;
    const int m = lane & 15;
    struct Pre {
        frag qf[2][NKD];   // Q fragments of tiles R[0], R[1] (k = d, column = token)
        frag pf[NPF];      // P^T fragments of tiles R[0], R[1]
        float eg[2];       // e^{g_r} of this lane's token in tiles R[0], R[1]
    };
    auto load = [&](Pre& p, int c) {
        c = min(c, nch - 1);   // past the segment: the last chunk again (unused)
        const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(rec0 + (size_t)c * Ly::REC, (int)Ly::REC);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd)
                p.qf[i][kd] = __builtin_bit_cast(
                    frag, buffer_load16(rr, (int)Ly::A_Q + (R[i] * NKD + kd) * Ly::FR + lane * 16));
#pragma unroll
        for (int i = 0; i < NPF; ++i) {
            const int rt = i < NP0 ? R[0] : R[1], kt = i < NP0 ? i : i - NP0;
            p.pf[i] = __builtin_bit_cast(frag, buffer_load16(rr, (int)Ly::A_P + (rt * NKT + kt) * Ly::FR + lane * 16));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) p.eg[i] = __uint_as_float(buffer_load4(rr, (int)Ly::A_EG + (16 * R[i] + m) * 4));
    };
    float bad = 0.f;
    OutPack<E> res[2];
    auto out = [&](int c, const Pre& S) {
        const unsigned char* st = smem + C::O_ST + (size_t)(c % 3) * C::STB;
        frag Hf[NKD], Uf[NKT];
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) Hf[kd] = ld_frag<frag>(st + (size_t)kd * 1024, lane);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) Uf[kt] = ld_frag<frag>(st + (size_t)(NKD + kt) * 1024, lane);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) acc = M::mma(Hf[kd], S.qf[i][kd], acc);
            const float g = S.eg[i];
            acc = f32x4{acc[0] * g, acc[1] * g, acc[2] * g, acc[3] * g};
#pragma unroll
            for (int kt = 0; kt <= Ly::kbmax(R[i]); ++kt) acc = M::mma(Uf[kt], S.pf[i == 0 ? kt : NP0 + kt], acc);
            res[i] = pack_out<E>(f32x4{acc[0] + bad, acc[1] + bad, acc[2] + bad, acc[3] + bad});
        }
    };
    constexpr int NSET = 3;
    lds_barrier();   // the records may be read from here on (the loaders have seen the prep count)
    bad = call_failed(a) ? __builtin_nanf("") : 0.f;
    Pre S[NSET];
#pragma unroll
    for (int i = 0; i < NSET; ++i) load(S[i], i);
    // iteration cc = 0 .. nch: barrier cc (cc = nch: the compute waves' last), then chunk cc - 1
    for (int c = 0; c <= nch; c += NSET) {
#pragma unroll
        for (int u = 0; u < NSET; ++u) {
            const int cc = c + u;
            if (u == 0 || cc <= nch) {
                lds_barrier();
                if (cc > 0) {
                    Pre& P = S[(u + NSET - 1) % NSET];   // chunk cc - 1's set
                    out(cc - 1, P);
                    load(P, cc - 1 + NSET);
                    if (cc < nch) {
                        OutPack<E>* ot = reinterpret_cast<OutPack<E>*>(smem + C::O_OT + (size_t)((cc - 1) & 1) * C::OTB);
                        ot[R[0] * 64 + lane] = res[0];
                        ot[R[1] * 64 + lane] = res[1];
                    } else {
                        store_packed<D, E>(a, bh, cg, cc - 1, R[0], lane, res[0]);
                        store_packed<D, E>(a, bh, cg, cc - 1, R[1], lane, res[1]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    wait_vmcnt<0>();   // every record load used has returned
    if (a.flags) publish_read(a.flags, FL_CHAIN, (unsigned)a.sgi + 1, C::READERS * a.BH * C::NCW, lane);
}

// Store wave HH of a chain workgroup (with output waves): iteration c follows barrier c, after
// which the output tiles of chunk c - 2 are in LDS; it writes tiles {0, 3} (HH = 0) or {1, 2}
// to memory. It loads nothing, so it never waits for its stores.
template <int D, class E, int HH>
__device__ __forceinline__ void chain_storer(const PrefArgs& a, unsigned char* smem, int nch, int bh, int cg,
                                             int lane) {
    using C = ChainCfg<D, E>;
    constexpr int R[2] = {HH == 0 ? 0 : 1, HH == 0 ? 3 : 2};
    lds_barrier();
    for (int cc = 0; cc <= nch; ++cc) {
        lds_barrier();
        if (cc >= 2) {
            const OutPack<E>* ot = reinterpret_cast<const OutPack<E>*>(smem + C::O_OT + (size_t)(cc & 1) * C::OTB);
#pragma unroll
            for (int i = 0; i < 2; ++i) store_packed<D, E>(a, bh, cg, cc - 2, R[i], lane, ot[R[i] * 64 + lane]);
        }
    }
}

// One workgroup per CU (its LDS ring). Waves 0 and 1 compute (row half w); with output waves,
// waves 2 and 3 form the outputs, waves 4 and 5 load and waves 6 and 7 store the outputs, else
// waves 2 and 3 load. The roles run separate loops with the same barrier sequence.
template <int D, class E>
__global__ __launch_bounds__((ChainCfg<D, E>::THREADS)) void chain_kernel(PrefArgs a) {
    using Ly = Layout<D, E>;
    using C = ChainCfg<D, E>;
    extern __shared__ __align__(16) unsigned char smem[];
    // blockIdx -> (slice, column group) so that all column groups of one slice run on the same
    // XCD (workgroups are dealt to the 8 XCDs round-robin) and share its L2.
    const int xcd = blockIdx.x & 7, sl = blockIdx.x >> 3;
    const int cg = sl % C::NCW, bh = (sl / C::NCW) * 8 + xcd;
    if (bh >= a.BH) return;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const unsigned char* rec0 = a.ws + (size_t)bh * a.segcap * Ly::REC;
    constexpr int LW = C::OUTW ? 4 : 2;   // first loader wave
    if (C::OUTW && w >= 6) {
        if (w == 7)
            chain_storer<D, E, 1>(a, smem, a.nseg, bh, cg, lane);
        else
            chain_storer<D, E, 0>(a, smem, a.nseg, bh, cg, lane);
    } else if (w >= LW)
        chain_loader<D, E>(a, smem, rec0, a.nseg, cg, w - LW, lane);
    else if (C::OUTW && w == 3)
        chain_output<D, E, 1>(a, smem, rec0, a.nseg, bh, cg, lane);
    else if (C::OUTW && w == 2)
        chain_output<D, E, 0>(a, smem, rec0, a.nseg, bh, cg, lane);
    else if (w == 1)
        chain_compute<D, E, 1>(a, smem, rec0, a.nseg, bh, cg, lane);
    else
        chain_compute<D, E, 0>(a, smem, rec0, a.nseg, bh, cg, lane);
}

// h_final = h0 (or zeros) for L = 0
__global__ void copy_state_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

template <int D, class E>
struct Launch {
    using T = typename E::T;
    using Ly = Layout<D, E>;
    using CC = ChainCfg<D, E>;
    static constexpr size_t LDS_PREP = PrepCfg<D, E>::LDS;
    static constexpr size_t LDS_CHAIN = CC::LDS;
    // While the chain runs on some of the CUs, the prep stage beside it is held to three
    // workgroups per CU by asking for more than a quarter of the CU's 160 KB of LDS: more
    // concurrent prep work slows the latency-bound chain by more than it gains.
    static constexpr size_t LDS_BESIDE = 41 * 1024;
    static constexpr size_t lds_prep(bool beside) { return beside && LDS_PREP < LDS_BESIDE ? LDS_BESIDE : LDS_PREP; }

    // raise the dynamic-LDS limits once per process (every caller sets the same values)
    static bool attributes() {
        static const bool ok =
            hipFuncSetAttribute(reinterpret_cast<const void*>(&prep_kernel<D, E>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_prep(true)) == hipSuccess &&
            hipFuncSetAttribute(reinterpret_cast<const void*>(&chain_kernel<D, E>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_CHAIN) == hipSuccess;
        return ok;
    }
    static int chain_blocks(int BH) { return 8 * ((BH + 7) / 8) * CC::NCW; }
    static void prep(const PrefArgs& a, hipStream_t s, bool beside = false) {
        hipLaunchKernelGGL((prep_kernel<D, E>), dim3(a.nseg, a.BH), dim3(256), lds_prep(beside), s, a);
    }
    static void chain(const PrefArgs& a, hipStream_t s) {
        hipLaunchKernelGGL((chain_kernel<D, E>), dim3(chain_blocks(a.BH)), dim3(CC::THREADS), LDS_CHAIN, s, a);
    }
};

// A stream and an event per device, created on first use and kept for the process: the
// intra-chunk stage of later segments runs on it while the chain works on the current segment
// on the caller's stream.
struct StreamCtx {
    std::mutex mu;
    bool ready = false;
    int ncu = 0;   // compute units of the device
    hipStream_t sp = nullptr;
    hipEvent_t start = nullptr;
};

static StreamCtx g_ctx[64];

static bool init_ctx(StreamCtx& c, int dev) {
    if (c.ready) return true;
    if (hipDeviceGetAttribute(&c.ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
    if (hipStreamCreateWithFlags(&c.sp, hipStreamNonBlocking) != hipSuccess) return false;
    if (hipEventCreateWithFlags(&c.start, hipEventDisableTiming) != hipSuccess) return false;
    c.ready = true;
    return true;
}

template <int D, class E>
static int launch_prefill_t(PrefArgs a, long nch, size_t ws_bytes, hipStream_t stream) {
    using LN = Launch<D, E>;
    if (!LN::attributes()) return -1;
    const size_t rec = Layout<D, E>::REC * (size_t)a.BH;
    if (ws_bytes >= (size_t)nch * rec) {   // whole sequence in one segment, caller's stream only
        a.c0 = 0; a.nseg = (int)nch; a.segcap = (int)nch; a.flags = nullptr; a.sgi = 0;
        LN::prep(a, stream);
        LN::chain(a, stream);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    const int seg = (int)((ws_bytes - FLAG_BYTES) / (NBUF * rec));   // >= 1 (validated)
    const size_t buf = (size_t)seg * rec;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
    StreamCtx& cx = g_ctx[dev];
    std::lock_guard<std::mutex> lk(cx.mu);
    if (!init_ctx(cx, dev)) return -1;
    const bool beside = LN::chain_blocks(a.BH) < cx.ncu;   // the chain leaves CUs to prep
    unsigned char* ws0 = a.ws;
    const float* h0 = a.h0;
    // progress counters after the buffers, cleared on the caller's stream; the side stream
    // starts after that (and after the work already queued on the caller's stream)
    unsigned* flags = reinterpret_cast<unsigned*>(ws0 + NBUF * buf);
    static_assert(FL_WORDS * 4 <= FLAG_BYTES, "counters fit");
    hipLaunchKernelGGL(flags_reset_kernel, dim3(1), dim3(FL_WORDS), 0, stream, flags);
    bool ok = hipEventRecord(cx.start, stream) == hipSuccess && hipStreamWaitEvent(cx.sp, cx.start, 0) == hipSuccess;
    auto wait = [&](hipStream_t s, int which, int count) {
        return hipStreamWaitValue32(s, flags + which, (unsigned)count, hipStreamWaitValueGte, 0xffffffffu) == hipSuccess;
    };
    auto mark = [&](hipStream_t s, int which, int count) {
        return hipStreamWriteValue32(s, flags + which, (unsigned)count, 0) == hipSuccess;
    };
    const int nsegs = (int)((nch + seg - 1) / seg);
    for (int sgi = 0; ok && sgi < nsegs; ++sgi) {
        PrefArgs b = a;
        b.c0 = sgi * seg;
        b.nseg = (int)(nch - b.c0 < seg ? nch - b.c0 : seg);
        b.segcap = seg;
        b.ws = ws0 + (size_t)(sgi % NBUF) * buf;
        b.h0 = sgi == 0 ? h0 : a.h_final;   // later segments continue from the running state
        b.flags = flags;
        b.sgi = sgi;
        // prep rewrites a buffer once the chain of the segment NBUF back has read it; the count
        // it then writes (hipStreamWriteValue32, after its kernel on the side stream) makes its
        // records visible to the chain, which waits for it inside its kernel and publishes its
        // own count when its last wave is done, so consecutive chain launches follow each other
        // directly. Every wait, in a kernel or on a stream, is for work queued before it, so the
        // order holds even where streams share a hardware queue. When the chain occupies every
        // CU its workgroups could keep prep's from starting, so then the stream waits instead.
        if (sgi >= NBUF) ok = ok && wait(cx.sp, FL_CHAIN, sgi - NBUF + 1);
        LN::prep(b, cx.sp, beside);
        ok = ok && mark(cx.sp, FL_PREP, sgi + 1);
        // hand the side stream's commands to the GPU now: left to itself the runtime holds
        // them back, and the chain then waits for prep (B=1, H=16, L=128K: 2.44 -> 2.02 ms;
        // doing the same on the caller's stream slows the chain's launches instead)
        (void)hipStreamQuery(cx.sp);
        if (!beside) ok = ok && wait(stream, FL_PREP, sgi + 1);
        LN::chain(b, stream);
    }
    return ok && hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_prefill(const void* q, const void* k, const void* v, const float* beta, const float* log_alpha,
                   const unsigned char* keep, const float* h0, void* o, float* h_final, int BH, long L, int D,
                   int dtype, int band, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (L == 0) {
        const size_t n = (size_t)BH * D * D;
        if (h0 == h_final) return 0;
        hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, h0, h_final, n);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    const long nch = (L + CH - 1) / CH;
    PrefArgs a{q, k, v, beta, log_alpha, h0, o, h_final, static_cast<unsigned char*>(ws), L, BH, 0, 0, 0, keep, (int)nch,
               band};
    if (D == 128 && dtype == 0) return launch_prefill_t<128, BF16>(a, nch, ws_bytes, stream);
    if (D == 128) return launch_prefill_t<128, F32>(a, nch, ws_bytes, stream);
    if (dtype == 0) return launch_prefill_t<64, BF16>(a, nch, ws_bytes, stream);
    return launch_prefill_t<64, F32>(a, nch, ws_bytes, stream);
}

}  // namespace gdn
