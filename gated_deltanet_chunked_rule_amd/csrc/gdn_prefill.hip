// Chunked prefill of the gated delta rule on gfx950, in block-scan form.
//
// The SparseGDN article (fileenergy.com, section "Why GDN prefill is expensive") names three
// sources of chunked GDN prefill work: the intra-chunk delta-system solve, the sequential
// chunk-to-chunk state pass for each head, and the outputs computed from every chunk's start
// state. Per chunk of C = 64 tokens, with g the inclusive cumulative log-gate (restarting at each
// chunk) and the key-major state H (Dk x Dv) at chunk start, the token recurrence
//     H_r = a_r (I - beta_r k_r k_r^T) H_{r-1} + beta_r k_r v_r^T
// unrolls to (exactly, up to rounding):
//     A[r][s] = beta_r exp(g_r - g_s) k_r.k_s  (s < r),     T = (I + A)^-1
//     W = T diag(beta e^g) K,   Ut = T diag(beta) V,        U = Ut - W H
//     O = diag(e^g) Q H + P U,  P[r][s] = exp(g_r - g_s) q_r.k_s  (s <= r)
//     H' = e^{g_C} H + Khat^T U,  Khat[s] = exp(g_C - g_s) k_s
// i.e. the affine chunk map H' = A_c H + B_c of the article's skip-scan illustration (section on
// embedding the selector into FLA) with A_c = e^{g_C} I - Khat^T W and B_c = Khat^T Ut.
//
// Affine maps compose, so a block of consecutive chunks c = 1 .. m moves its start state to its
// end state by one map  H_end = Phi H_start + Psi  with  Phi = A_m ... A_1  and
// Psi = sum_c A_m ... A_{c+1} B_c. The sequential pass is cut at block boundaries:
//   map_kernel  (one workgroup per head and block, every block but the last, all in parallel):
//               the block's chunks from last to first, each one's intra-chunk solve and then, with
//               Z = (A_m ... A_{c+1})^T (from I) and Y = Khat Z,
//                   Psi += Y^T Ut,   Z <- e^{g_C} Z - W^T Y;
//               at the end Z = Phi^T. Phi goes to the workspace as matrix-core operands (bf16 as
//               a high and a low part), Psi as fp32 tiles.
//   scan_kernel (one workgroup per head and 16 value columns): H_{b+1} = Phi_b H_b + Psi_b over
//               the blocks in order, with fp32-accurate products; every block's start state to
//               the workspace.
//   out_kernel  (one workgroup per head and block, all in parallel): from the block's start
//               state, each chunk's intra-chunk solve again, then U, the outputs O and the next
//               state with the fp32 state held in registers; the last block writes h_final.
// Chunk-start states never reach memory, and the per-head sequential work shrinks from one step
// per chunk to one small product per block. With a single block (many heads, short sequences or
// no workspace) only out_kernel runs: the sequential pass per head in one workgroup.
//
// A log gate of -inf (a zero gate) clears the state before its token's write. Cumulative sums
// then cannot be differenced, so each token also carries the index of the last zero gate at or
// before it: exp(g_r - g_s) is taken over the finite gates only, and is zero when a zero gate
// lies in (s, r]. Finite log gates below -110 are taken as -110 (exp of any sum holding one is
// exactly zero in fp32). Only exponentials of non-positive differences are formed.
#include <atomic>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_launch.h"
#include "gdn_rows.h"

namespace gdn {

// ---------------------------------------------------------------------------------------------
// sizes and layouts
// ---------------------------------------------------------------------------------------------
constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
constexpr size_t up16(size_t x) { return (x + 15) / 16 * 16; }

template <int D, class E, int NW_ = 4>
struct Cfg {
    using T = typename E::T;
    using M = MM<E>;
    static constexpr int KB = M::KB;                          // k extent of one fragment
    static constexpr int FPD = KB / 16;                       // 16-wide tiles per fragment along k
    static constexpr int NDT = D / 16;                        // 16-wide tiles along d
    static constexpr int NKD = D / KB;                        // fragments along d
    static constexpr int NKT = CH / KB;                       // fragments along a chunk's tokens
    static constexpr int NW = NW_;                            // waves sharing the d (value) tiles
    static constexpr int NT = 64 * NW;                        // their threads
    static constexpr int VPW = NDT / NW;                      // d (and value) tiles per wave
    static_assert(NDT % NW == 0, "whole tiles per wave");
    static constexpr int SVPW = NDT / 4;                      // row tiles per wave of the scan
    static constexpr int NSPLIT = sizeof(T) == 2 ? 2 : 1;     // bf16 operands as high + low parts
    static constexpr int KP = row_stride<D, E>();             // row stride of staged rows (elements)
    static constexpr int AS = CH + 4;                         // row stride of A and T (floats)
    static constexpr size_t FR = 1024;                        // bytes per fragment (64 lanes x 16)
    static constexpr size_t REG = up16(cmax((size_t)CH * KP * sizeof(T), (size_t)CH * AS * 4));
    // per slice and block in the workspace: Phi operands, and Psi / the block's start state
    static constexpr size_t PHI = (size_t)NDT * NKD * NSPLIT * FR;   // 4 D^2 bytes
    static constexpr size_t HS = (size_t)NDT * NDT * FR;             // D^2 fp32, in 16 x 16 tiles
    static constexpr int kbmax(int rt) { return (16 * rt + 15) / KB; }   // last token fragment <= tile rt
    static constexpr int NPFR = [] {
        int c = 0;
        for (int rt = 0; rt < 4; ++rt) c += (16 * rt + 15) / KB + 1;
        return c;
    }();
};

// Waves per workgroup of the output kernel: four for bf16 (two workgroups share a CU, so one's
// serial phases overlap the other's matrix work), eight for fp32 at Dk = 128 (its operands
// need the registers of two waves per value tile).
template <int D, class E>
constexpr int out_waves() { return D == 128 && sizeof(typename E::T) == 4 ? 8 : 4; }

// The map kernel holds two fp32 state blocks, so at Dk = 128 it runs eight waves, one value tile
// each. With bf16 it works on chunks in pairs: each half of the workgroup (four waves) does the
// intra-chunk solve of one chunk of the pair in its own LDS slot, so the two serial solves run
// side by side, and then all eight waves apply both chunks to the state in order.
template <int D, class E>
struct MapCfg {
    static constexpr bool PAIR = D == 128 && sizeof(typename E::T) == 2;
    static constexpr int NWS = D == 128 ? 8 : 4;     // waves holding the state
    static constexpr int NWP = PAIR ? 4 : NWS;       // waves per chunk's solve
    static constexpr int NH = PAIR ? 2 : 1;          // chunks per iteration
};

// per-token gate arrays of the chunk in LDS
struct Gates {
    float g[CH];     // cumulative log gate over the finite gates, in log2 units (times log2 e)
    int rho[CH];     // last token <= r with a zero gate (log a = -inf), or -1
    float b[CH];     // beta
    float nbe[CH];   // -beta e^{g_r} (zero after a zero gate)
    float kh[CH];    // e^{g_C - g_s} (zero before the chunk's last zero gate)
    float eg[CH];    // e^{g_r} (zero after a zero gate)
    float dec;       // e^{g_C}
    float pad[3];
};

// fp32 inputs, whose bound is tight: the cumulative log gates also carry their low parts (g + glo
// is the exact prefix sum, see wave_scan2), so that differences of them keep fp32 precision where
// the sums themselves are large (strong decay: a chunk's log gates summing to -10^3)
struct GatesLo : Gates {
    float glo[CH];
};
template <class E>
using GatesOf = std::conditional_t<sizeof(typename E::T) == 4, GatesLo, Gates>;

// LDS of a workgroup of the map (OUT = false) or output (OUT = true) kernel:
//   OUT:  Q rows | K rows, then T | V rows, then A, then -W fragments | Khat^T fragments |
//         P^T fragments | gates of two chunks (the current one and the next, by chunk parity)
//   map:  K rows | V rows, then A, then -W^T fragments | T | Ut fragments | gates
template <int D, class E, bool OUT>
struct Lds {
    using C = Cfg<D, E>;
    static constexpr size_t REG = C::REG;
    static constexpr size_t O_Q = 0;
    static constexpr size_t O_K = OUT ? REG : 0;
    static constexpr size_t O_T = OUT ? REG : REG * 2;
    static constexpr size_t O_V = OUT ? 2 * REG : REG;         // V rows, then A, then the W fragments
    static constexpr size_t O_KH = 3 * REG;                    // OUT: Khat^T fragments [dt][kt]
    static constexpr size_t O_P = O_KH + (size_t)C::NDT * C::NKT * C::FR;   // OUT: P^T fragments [rt][kt]
    static constexpr size_t O_UT = 3 * REG;                    // map: Ut fragments [kt][vt]
    static constexpr size_t O_G = OUT ? O_P + (size_t)4 * C::NKT * C::FR : O_UT + (size_t)C::NKT * C::NDT * C::FR;
    static constexpr size_t GSZ = up16(sizeof(GatesOf<E>));
    static constexpr size_t BYTES = O_G + (OUT ? 2 : 1) * GSZ;
    static_assert(BYTES <= 160 * 1024, "LDS");
};

struct PrefArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* beta;
    const float* log_alpha;
    const float* h0;
    const unsigned char* keep;   // [BH][nch] chunk keep mask, or NULL (keep all)
    void* o;
    float* h_final;
    unsigned char* ws;           // per slice: Phi of blocks 0 .. NB-2, then the NB state slots
    long L;
    int BH;
    int nch;                     // chunks per slice
    int m;                       // chunks per block
    int NB;                      // blocks per slice
    int band;                    // 16 x 16 blocks of T kept below the diagonal (3: all, exact)
};

// bytes per slice of the blocks' "map is not zero" flags (one int per block but the last)
__host__ __device__ __forceinline__ size_t flag_bytes(int NB) { return NB <= 1 ? 0 : ((size_t)(NB - 1) * 4 + 255) / 256 * 256; }

template <int D, class E>
__device__ __forceinline__ size_t slice_ws(const PrefArgs& a) {
    using C = Cfg<D, E>;
    return (size_t)(a.NB - 1) * C::PHI + (size_t)a.NB * C::HS + flag_bytes(a.NB);
}
template <int D, class E>
__device__ __forceinline__ unsigned char* ws_phi(const PrefArgs& a, int bh, int b) {
    return a.ws + (size_t)bh * slice_ws<D, E>(a) + (size_t)b * Cfg<D, E>::PHI;
}
// state slot s of a slice: slot 0 holds H_0, slot b + 1 first Psi_b (map_kernel), then H_{b+1}
template <int D, class E>
__device__ __forceinline__ f32x4* ws_hs(const PrefArgs& a, int bh, int s) {
    using C = Cfg<D, E>;
    return reinterpret_cast<f32x4*>(a.ws + (size_t)bh * slice_ws<D, E>(a) + (size_t)(a.NB - 1) * C::PHI +
                                    (size_t)s * C::HS);
}

// flag of block b (< NB - 1) of a slice: nonzero when its map's transition Phi_b is not zero
template <int D, class E>
__device__ __forceinline__ int* ws_flag(const PrefArgs& a, int bh, int b) {
    using C = Cfg<D, E>;
    return reinterpret_cast<int*>(a.ws + (size_t)bh * slice_ws<D, E>(a) + (size_t)(a.NB - 1) * C::PHI +
                                  (size_t)a.NB * C::HS) + b;
}

__device__ __forceinline__ unsigned keep_chunk(const PrefArgs& a, int bh, int c) {
    return a.keep ? (unsigned)__builtin_amdgcn_readfirstlane(a.keep[(size_t)bh * a.nch + c] != 0) : 1u;
}

// ---------------------------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------------------------
// A value the compiler must treat as unknown from here on. Taking the lane index through this at
// the top of every chunk iteration keeps the per-lane LDS addresses, masks and selector
// fragments derived from it inside the loop: hoisted out of the loop they would all stay live
// across every phase of it (a few hundred registers) and spill, while recomputing them costs a
// handful of integer instructions per use.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// inclusive max-scan over the 64 lanes of a wave (values >= -1)
__device__ __forceinline__ int wave_max_scan(int x, int /*lane*/) {
    return wave_scan_dpp(x, -1, [](int a, int b) { return max(a, b); });
}

// 2^x by the hardware's base-2 exponential (what expf(x) reduces to after scaling x by log2 e)
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Gate arrays of a chunk, computed by one wave (lane = token; past the end la = 0, bt = 0).
// The cumulative log gates are kept in log2 units, so every factor exp(g_r - g_s) is one base-2
// exponential of a difference. A finite log gate below -110 is taken as -110: every factor whose
// interval holds it is exactly zero in fp32 either way, and the cumulative sums stay small
// enough to keep their precision (a gate of, say, -1e6 would leave later sums with no bits for
// the other gates). upd = false (a skipped chunk of the output kernel) sets Khat's
// factors e^{g_C - g} to zero, so the state update adds nothing to the decayed state.
template <class G>
__device__ __forceinline__ void gate_scan(G* gt, float la, float bt, int lane, bool upd = true) {
    constexpr float LOG2E = 1.44269504088896341f;
    const bool zero = la == -__builtin_inff();
    if constexpr (std::is_same<G, GatesLo>::value) {
        // g + lo exactly; scaled to log2 units with the product's rounding error kept in lo. No
        // contraction here: fused into a later subtraction (gC - g as fma(-gn, LOG2E, gC)), the
        // product would enter unrounded where the pair's bookkeeping assumes the rounded g, and
        // e^{g_C - g_s} would be off by up to half an ulp of the sums (e.g. 7.5e-5 for the last
        // token's own factor, which must be exactly 1, where a chunk's sums reach 10^3).
#pragma clang fp contract(off)
        float lo;
        const float gn = wave_scan2(zero ? 0.f : floor_log_gate(la), lo);
        const float g = gn * LOG2E;
        lo = __builtin_fmaf(lo, LOG2E, __builtin_fmaf(gn, LOG2E, -g));
        const int rho = wave_max_scan(zero ? lane : -1, lane);
        const float gC = wave_last(g), gClo = wave_last(lo);
        const int rhoC = __builtin_amdgcn_readlane(rho, 63);
        const float eg = rho < 0 ? exp2_hw(g + lo) : 0.f;
        gt->g[lane] = g;
        gt->glo[lane] = lo;
        gt->rho[lane] = rho;
        gt->b[lane] = bt;
        gt->nbe[lane] = -bt * eg;
        gt->kh[lane] = upd && rhoC <= lane ? exp2_hw((gC - g) + (gClo - lo)) : 0.f;
        gt->eg[lane] = eg;
        if (lane == 0) gt->dec = rhoC < 0 ? exp2_hw(gC + gClo) : 0.f;
    } else {
        const float g = wave_scan(zero ? 0.f : floor_log_gate(la), lane) * LOG2E;
        const int rho = wave_max_scan(zero ? lane : -1, lane);
        const float gC = wave_last(g);
        const int rhoC = __builtin_amdgcn_readlane(rho, 63);
        const float eg = rho < 0 ? exp2_hw(g) : 0.f;
        gt->g[lane] = g;
        gt->rho[lane] = rho;
        gt->b[lane] = bt;
        gt->nbe[lane] = -bt * eg;
        gt->kh[lane] = upd && rhoC <= lane ? exp2_hw(gC - g) : 0.f;
        gt->eg[lane] = eg;
        if (lane == 0) gt->dec = rhoC < 0 ? exp2_hw(gC) : 0.f;
    }
}

// The part of an operand fragment that one 16 x 16 accumulator tile fills: elements 4 h .. 4 h + 3
// of each lane for bf16 (h = which of the fragment's two tiles), the whole fragment for fp32.
// `lo` stores the rounding residual x - bf16(x) instead (bf16 only).
template <class E>
__device__ __forceinline__ void st_tile_part(unsigned char* frag, int lane, int h, const f32x4& t, bool lo = false) {
    if constexpr (sizeof(typename E::T) == 2) {
        float x[4] = {t[0], t[1], t[2], t[3]};
        if (lo) {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] -= bf2f(f2bf(x[e]));
        }
        *reinterpret_cast<uint2*>(frag + lane * 16 + h * 8) = uint2{f2bf2(x[0], x[1]), f2bf2(x[2], x[3])};
    } else {
        *reinterpret_cast<f32x4*>(frag + lane * 16) = t;
    }
}

// residual fragment of from_acc(t, kb): x - bf16(x) per element (bf16 only)
template <class E>
__device__ __forceinline__ typename MM<E>::frag lo_from_acc(const f32x4* t, int kb) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float y = t[2 * kb + i][e];
            x[4 * i + e] = y - bf2f(f2bf(y));
        }
    return MM<E>::pack(x);
}

__device__ __forceinline__ f32x4 scale4(const f32x4& t, float s) { return f32x4{t[0] * s, t[1] * s, t[2] * s, t[3] * s}; }

// ---------------------------------------------------------------------------------------------
// one chunk's rows in flight
// ---------------------------------------------------------------------------------------------
// Q and K rows for LDS (Q only for the output kernel), the wave's own value tiles of V as row
// fragments straight from memory (only its own tiles are transposed, so V never goes through
// LDS), and for wave 0 the gates. Loads go through buffer resources over the chunk's valid
// tokens: rows past the end of the sequence read as zero. A bf16 V fragment holds 8 adjacent
// columns per lane (one 16-byte load): lane (j, m) takes row m at columns 8 j .. 8 j + 7 of its
// 32-column group, the order v_unit_cols transposes.
template <int D, class E, bool OUT, int NW>
struct Fetch {
    using C = Cfg<D, E, NW>;
    using T = typename E::T;
    using frag = typename MM<E>::frag;
    static constexpr int NGW = C::VPW >= C::FPD ? C::VPW / C::FPD : 1;   // fragment groups of V a wave owns
    RowRegs<D, E, C::NT> rq, rk;
    frag vf[NGW][4];   // V row fragments [own group][token tile]
    float la, bt;
    unsigned kp = 1;   // OUT: the chunk's keep flag (nonzero: its update is kept)
    int n;             // valid tokens
    size_t tok0;       // first token of the chunk in its slice's rows
    size_t kidx;       // the chunk's entry in the keep mask
    // the wave that loads (and scans) the gates: wave 0 for the map kernel; for the output kernel
    // the last wave, which has no block of T to form in the first step after the substitution
    static constexpr int GW = OUT ? NW - 1 : 0;
    __device__ __forceinline__ void start(const PrefArgs& a, int bh, int c) {
        const long t0 = (long)c * CH;
        n = (int)min((long)CH, a.L - t0);
        tok0 = (size_t)bh * a.L + t0;
        kidx = (size_t)bh * a.nch + c;
    }
    __device__ __forceinline__ void load_k(const PrefArgs& a, int tid) {
        rk.load(static_cast<const T*>(a.k) + tok0 * D, n, tid);
    }
    __device__ __forceinline__ void load_q(const PrefArgs& a, int tid) {
        rq.load(static_cast<const T*>(a.q) + tok0 * D, n, tid);
    }
    __device__ __forceinline__ void load_v(const PrefArgs& a, int tid, int w) {
        const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(static_cast<const T*>(a.v) + tok0 * D, n * D * (int)sizeof(T));
        const int lane = tid & 63, j = lane >> 4, m = lane & 15;
        const int g0 = C::VPW * w / C::FPD;
#pragma unroll
        for (int gi = 0; gi < NGW; ++gi)
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                if constexpr (sizeof(T) == 2) {
                    const int e0 = (16 * st + m) * D + (g0 + gi) * C::KB + 8 * j;   // element offset
                    vf[gi][st] = __builtin_bit_cast(frag, buffer_load16(rv, e0 * 2));
                } else {
                    const int e0 = (16 * st + m) * D + (g0 + gi) * C::KB + 4 * j;
                    vf[gi][st] = __builtin_bit_cast(frag, buffer_load16(rv, e0 * 4));
                }
            }
    }
    __device__ __forceinline__ void load_gates(const PrefArgs& a, int tid) {
        if ((tid >> 6) == GW) {   // lane = token
            const __amdgpu_buffer_rsrc_t rl = buffer_rsrc(a.log_alpha + tok0, n * 4);
            const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(a.beta + tok0, n * 4);
            la = __uint_as_float(buffer_load4(rl, (tid & 63) * 4));
            bt = __uint_as_float(buffer_load4(rb, (tid & 63) * 4));
            if constexpr (OUT) kp = a.keep ? (unsigned)a.keep[kidx] : 1u;
        }
    }
    __device__ __forceinline__ void issue(const PrefArgs& a, int bh, int c, bool rows, int tid, int w) {
        start(a, bh, c);
        if (rows) {
            load_k(a, tid);
            if constexpr (OUT) load_q(a, tid);
            load_v(a, tid, w);
        }
        load_gates(a, tid);
    }
};

// Inverse off-diagonal block (bj + LVL, bj) of T = (I + A)^-1 (16 x 16 blocks, fp32):
//     T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
// on fp32 MFMA; every T_kj with k < i must be final. Called by one whole wave; all its loads
// are issued before the first product.
template <int AS, int LVL>
__device__ __forceinline__ void inverse_block(const float* Am, float* Tm, int bj, int j, int m) {
    const int bi = bj + LVL;
    f32x4 av[LVL], bv[LVL];
#pragma unroll
    for (int d = 0; d < LVL; ++d) {
        const int bk = bj + d;
        const float4 x = *reinterpret_cast<const float4*>(Am + (16 * bi + m) * AS + 16 * bk + 4 * j);
        av[d] = f32x4{x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[d][e] = Tm[(16 * bk + 4 * j + e) * AS + 16 * bj + m];
    }
    const float4 t = *reinterpret_cast<const float4*>(Tm + (16 * bi + m) * AS + 16 * bi + 4 * j);
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < LVL; ++d) x = MM<F32>::mma(av[d], bv[d], x);
    const f32x4 y = MM<F32>::mma(f32x4{t.x, t.y, t.z, t.w}, x, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int e = 0; e < 4; ++e) Tm[(16 * bi + 4 * j + e) * AS + 16 * bj + m] = -y[e];
}

// Steps s = 4 S .. 4 S + 3 of the forward substitution of a diagonal 16 x 16 block of T (block
// origin i0), lane (c, g) = (lane / 4, lane % 4) holding rows 4 g .. 4 g + 3 of column c in x:
// the lane of the quad with g = S owns row s, and the quad broadcast gives its final value.
template <int S, int AS>
__device__ __forceinline__ void subst_stage(const float* Am, int i0, int g, float (&x)[4]) {
    float4 av[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = *reinterpret_cast<const float4*>(Am + (i0 + 4 * g + i) * AS + i0 + 4 * S);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float v = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x[k]), S * 0x55, 0xF, 0xF, false));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ak = k == 0 ? av[i].x : k == 1 ? av[i].y : k == 2 ? av[i].z : av[i].w;
            x[i] = fmaf(-ak, v, x[i]);
        }
    }
}

// The lower-left 32 x 32 quadrant of T from its two diagonal 32 x 32 blocks (each already
// inverted):  T_ij = -sum_{k=2}^{i} T_ik X_kj  with  X_kj = sum_{l=j}^{1} A_kl T_lj,
// i in {2, 3}, j in {0, 1}; wave q computes tile (2 + q / 2, q % 2), recomputing the X it needs
// (so the quadrant takes one barrier). fp32 MFMA; all four diagonal blocks and T_10, T_32 must be
// final.
template <int AS>
__device__ __forceinline__ void inverse_quadrant(const float* Am, float* Tm, int q, int j, int m) {
    const bool i3 = (q >> 1) != 0;   // scalars
    const int bj = q & 1, bi = i3 ? 3 : 2;
    auto arow = [&](const float* X, int r, int l) {   // A operand: tile (r, l), lane (m, j): row m, k = 4 j ..
        const float4 x = *reinterpret_cast<const float4*>(X + (16 * r + m) * AS + 16 * l + 4 * j);
        return f32x4{x.x, x.y, x.z, x.w};
    };
    auto bcol = [&](int l, int c) {   // B operand: tile (l, c) of T, lane (m, j): k = 4 j + e, column m
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = Tm[(16 * l + 4 * j + e) * AS + 16 * c + m];
        return v;
    };
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const f32x4 a2j = arow(Am, 2, bj), tjj = bcol(bj, bj), ti2 = arow(Tm, bi, 2);
    f32x4 x2 = MM<F32>::mma(a2j, tjj, z);
    if (bj == 0) x2 = MM<F32>::mma(arow(Am, 2, 1), bcol(1, 0), x2);
    f32x4 y = MM<F32>::mma(ti2, x2, z);
    if (i3) {
        f32x4 x3 = MM<F32>::mma(arow(Am, 3, bj), tjj, z);
        if (bj == 0) x3 = MM<F32>::mma(arow(Am, 3, 1), bcol(1, 0), x3);
        y = MM<F32>::mma(arow(Tm, 3, 3), x3, y);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) Tm[(16 * bi + 4 * j + e) * AS + 16 * bj + m] = -y[e];
}

// B operand that transposes a bf16 V fragment of Fetch::load_v on the matrix core: element e of
// lane (j, n) is 1 where 8 j + e = n + 16 q, so the product lands columns 16 q .. 16 q + 15 of
// the fragment's 32-column group in an accumulator tile (exact: one nonzero term per output).
__device__ __forceinline__ bf16x8 v_unit_cols(int j, int n, int q) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 8 * j + e == n + 16 * q ? 1.f : 0.f;
    return MM<BF16>::pack(x);
}

// ---------------------------------------------------------------------------------------------
// the intra-chunk solve, shared by both kernels
// ---------------------------------------------------------------------------------------------
// From the chunk's rows and gates in LDS (after a barrier), wave w:
//   - row tile w of the Gram matrix K K^T, masked and gated into A (the blocks on and below the
//     diagonal), and for OUT the P^T tiles of query tile w, gated and packed as fragments; the
//     operand fragments of tile w are loaded once and those of each key tile once for both;
//   - its own d tiles of K transposed on the matrix core (scaled by -beta e^g into `kbe`, and
//     for OUT by e^{g_C - g} into the Khat^T fragments) and its own value tiles of V from `vf`
//     (scaled by beta into `vb`);
// then T = (I + A)^-1 blocked by 16: the diagonal blocks by forward substitution, then (exact)
// the two 32 x 32 diagonal blocks and the quadrant below them, or (band < 3) the blocks within
// `band` of the diagonal level by level, the others zero. Returns after the barrier that
// completes T. Wave w owns d (and value) tiles VPW w .. VPW w + VPW - 1. The chunk's gate arrays
// are `gt`. The last wave has no block of T to form in the step after the diagonal substitution
// and runs `side()` there instead (work of its own that touches none of the solve's LDS).
template <int D, class E, bool OUT, int NW, class Side>
__device__ __forceinline__ void intra_solve(unsigned char* smem, const GatesOf<E>* gt, int band, int w, int lane, Side&& side,
                                            const typename MM<E>::frag (&vf)[Fetch<D, E, OUT, NW>::NGW][4],
                                            typename MM<E>::frag (&kbe)[Cfg<D, E, NW>::VPW][Cfg<D, E, NW>::NKT],
                                            typename MM<E>::frag (&vb)[Cfg<D, E, NW>::VPW][Cfg<D, E, NW>::NKT]) {
    using C = Cfg<D, E, NW>;
    using L = Lds<D, E, OUT>;
    using M = MM<E>;
    using T = typename E::T;
    using frag = typename M::frag;
    constexpr int KB = C::KB, FPD = C::FPD, NKD = C::NKD, NKT = C::NKT, VPW = C::VPW, KP = C::KP, AS = C::AS;
    const int j = lane >> 4, m = lane & 15;
    const T* Kr = reinterpret_cast<const T*>(smem + L::O_K);
    const T* Qr = reinterpret_cast<const T*>(smem + L::O_Q);
    float* Tm = reinterpret_cast<float*>(smem + L::O_T);
    float* Am = reinterpret_cast<float*>(smem + L::O_V);

    // Row tile rw of the Gram matrix and row tile rp of P^T: only their tiles on and below the
    // diagonal are formed (st <= rw, st <= rp). With four waves wave w takes Gram row w and P^T
    // row 3 - w, five tiles each; with eight, waves 0-3 take the Gram rows and waves 4-7 the P^T
    // rows (the map kernel, which has no P^T, splits each Gram row over two waves). Every branch
    // below is on scalars.
    constexpr bool SPLIT = C::NW == 8;
    const int rw = w & 3, rp = SPLIT ? rw : 3 - rw;
    const bool do_gram = !OUT || !SPLIT || w < 4;
    const bool do_p = OUT && (!SPLIT || w >= 4);
    constexpr int NST = !OUT && SPLIT ? 2 : 4;               // key tiles per wave
    const int st0 = !OUT && SPLIT ? 2 * (w >> 2) : 0;
    // operands of row tiles rw (K) and rp (Q), and the gates of this lane's rows: r = 16 rw + m in
    // the transposed Gram tiles and r = 16 rp + m in the P^T tiles (accumulator columns in both)
    frag kw[NKD], qw[NKD];
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
        if (do_gram) kw[kd] = row_frag_raw<E>(Kr + (16 * rw + m) * KP, kd * KB, j);
        if constexpr (OUT)
            if (do_p) qw[kd] = row_frag_raw<E>(Qr + (16 * rp + m) * KP, kd * KB, j);
    }
    const float grw = gt->g[16 * rw + m], brw = gt->b[16 * rw + m];
    const int rhow = gt->rho[16 * rw + m];
    const float grm = gt->g[16 * rp + m];
    const int rhom = gt->rho[16 * rp + m];
    // fp32 inputs: the exponents g_r - g_s of the gate factors with the sums' low parts
    constexpr bool LO = std::is_same<GatesOf<E>, GatesLo>::value;
    f32x4 pt[4];
#pragma unroll
    for (int i = 0; i < NST; ++i) {
        const int st = st0 + i;
        const bool g_on = do_gram && st <= rw, p_on = do_p && st <= rp;
        pt[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!g_on && !p_on) continue;
        frag kf[NKD];
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) kf[kd] = row_frag_raw<E>(Kr + (16 * st + m) * KP, kd * KB, j);
        if (g_on) {
            // Gram tile (rw, st), transposed: lane (j, n) holds k_s . k_r at s = 16 st + 4 j + e,
            // r = 16 rw + n, so that the four A[r][s] of a lane are adjacent in A's row r (one
            // 16-byte store); A[r][s] = beta_r exp(g_r - g_s) k_r.k_s for s < r
            f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) g = M::mma(kf[kd], kw[kd], g);
            const int r = 16 * rw + m;
            const float4 gs4 = *reinterpret_cast<const float4*>(gt->g + 16 * st + 4 * j);
            const float gs[4] = {gs4.x, gs4.y, gs4.z, gs4.w};
            float av[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 16 * st + 4 * j + e;
                if constexpr (LO) {
                    const float d = (grw - gs[e]) + (gt->glo[r] - gt->glo[s]);
                    av[e] = (s < r && s >= rhow) ? brw * exp2_hw(d) * g[e] : 0.f;
                } else {
                    av[e] = (s < r && s >= rhow) ? brw * exp2_hw(grw - gs[e]) * g[e] : 0.f;
                }
            }
            *reinterpret_cast<float4*>(Am + r * AS + 16 * st + 4 * j) = make_float4(av[0], av[1], av[2], av[3]);
        }
        if constexpr (OUT) {
            if (p_on) {
                // P^T tile (st, rp): lane (j, n) holds exp(g_r - g_s) q_r.k_s at s = 16 st + 4 j + e,
                // r = 16 rp + n (zero for s > r or a zero gate in (s, r])
                f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kd = 0; kd < NKD; ++kd) p = M::mma(kf[kd], qw[kd], p);
                const float4 gs4 = *reinterpret_cast<const float4*>(gt->g + 16 * st + 4 * j);
                const float gs[4] = {gs4.x, gs4.y, gs4.z, gs4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s2 = 16 * st + 4 * j + e, r = 16 * rp + m;
                    if constexpr (LO) {
                        const float d = (grm - gs[e]) + (gt->glo[r] - gt->glo[s2]);
                        pt[i][e] = (s2 <= r && s2 >= rhom) ? exp2_hw(d) * p[e] : 0.f;
                    } else {
                        pt[i][e] = (s2 <= r && s2 >= rhom) ? exp2_hw(grm - gs[e]) * p[e] : 0.f;
                    }
                }
            }
        }
    }
    if constexpr (OUT) {
        // P^T fragments [rt = rp][kt]: the B operand (k = s, column r) of O^T += U^T P^T
        if (do_p) {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) st_frag(smem + L::O_P + (size_t)(rp * NKT + kt) * C::FR, lane, M::from_acc(pt, kt));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // rows to columns: tile st of d (value) tile dt, lane (j, n) holding rows 16 st + 4 j .. + 3
    // of column 16 dt + n. K (bf16) with gfx950's transposing LDS reads, V (in registers) and
    // fp32 K on the matrix core.
#pragma unroll
    for (int t = 0; t < VPW; ++t) {
        const int dt = VPW * w + t;
        frag sel;
        if constexpr (sizeof(T) == 2) sel = v_unit_cols(j, m, dt % FPD);
        else sel = unit_cols<E>(j, m, dt % FPD);
        f32x4 kc[4], vc[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            if constexpr (sizeof(T) != 2)
                kc[st] = M::mma(row_frag_raw<E>(Kr + (16 * st + m) * KP, KB * (dt / FPD), j), sel, f32x4{0.f, 0.f, 0.f, 0.f});
            vc[st] = M::mma(vf[VPW >= FPD ? t / FPD : 0][st], sel, f32x4{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            if constexpr (sizeof(T) == 2) {
                const frag kr = tr_frag(Kr, KP, KB * kt, 16 * dt, j, m);
                kbe[t][kt] = scale_frag(kr, gt->nbe + KB * kt, j);
                if constexpr (OUT) st_frag(smem + L::O_KH + (size_t)(dt * NKT + kt) * C::FR, lane, scale_frag(kr, gt->kh + KB * kt, j));
            } else {
                kbe[t][kt] = cols_frag<E>(&kc[FPD * kt], gt->nbe + KB * kt, j);
                if constexpr (OUT)
                    st_frag(smem + L::O_KH + (size_t)(dt * NKT + kt) * C::FR, lane, cols_frag<E>(&kc[FPD * kt], gt->kh + KB * kt, j));
            }
            vb[t][kt] = cols_frag<E>(&vc[FPD * kt], gt->b + KB * kt, j);
        }
    }
    // Diagonal block rw of T by forward substitution in outer-product order, by the wave that
    // formed A's diagonal tile (rw, rw) above: it reads only its own LDS writes, so it needs no
    // barrier and overlaps the other waves' tiles (T_ii is stored once K's rows are free). Lane
    // (c, g) = (lane / 4, lane % 4) holds rows 4 g .. 4 g + 3 of column c. Step s takes the final
    // x_s from the lane of its quad that owns row s (a quad broadcast) and updates every row of
    // the lane with A[r][s] (zero on and above the diagonal, so rows at or before s are left as
    // they are); A is read four columns at a time.
    const bool diag = do_gram && st0 <= rw && rw < st0 + NST;   // scalar; every wave when NW = 4
    float xd[4];
    if (C::NW == 4 || diag) {
        asm volatile("" ::: "memory");
        const int i0 = 16 * rw, g = lane & 3, c = lane >> 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) xd[i] = 4 * g + i == c ? 1.f : 0.f;
        subst_stage<0, AS>(Am, i0, g, xd);
        subst_stage<1, AS>(Am, i0, g, xd);
        subst_stage<2, AS>(Am, i0, g, xd);
        subst_stage<3, AS>(Am, i0, g, xd);
    }
#pragma unroll
    for (int t = 0; t < VPW; ++t)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            asm volatile("" : "+v"(kbe[t][kt]));
            asm volatile("" : "+v"(vb[t][kt]));
        }
    lds_sync();   // A is complete, and K rows are no longer read (OUT: T takes their space)
    // T's blocks (0, 1) and (2, 3) above the diagonal are zero (the token fragments of 32 that
    // the products with T read cover them; no other block above the diagonal is read), and so
    // are, for the block-adjacent approximation, the blocks more than `band` below it
    const int tid = 64 * w + lane;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
        constexpr int NZ = C::NT < 256 ? 256 / C::NT : 1;   // elements per thread
        const int bi = b >> 2, bj = b & 3;                   // compile-time block, scalar test
        if (((bj == bi + 1 && (bi & 1) == 0) || bi - bj > band) && (C::NT <= 256 || w < 4)) {
#pragma unroll
            for (int z = 0; z < NZ; ++z) {
                const int el = tid + (NZ > 1 ? C::NT * z : 0);
                Tm[(16 * bi + (el >> 4)) * AS + 16 * bj + (el & 15)] = 0.f;
            }
        }
    }
    if (C::NW == 4 || diag) {
        const int i0 = 16 * rw, g = lane & 3, c = lane >> 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) Tm[(i0 + 4 * g + i) * AS + i0 + c] = xd[i];
    }
    lds_sync();
    if (band >= 3) {
        // exact: blocks (1, 0) and (3, 2), then the lower-left quadrant
        if (w < 2) inverse_block<AS, 1>(Am, Tm, 2 * w, j, m);
        else if (w == NW - 1) side();
        lds_sync();
        if (w < 4) inverse_quadrant<AS>(Am, Tm, w, j, m);
        lds_sync();
    } else {
        // block-adjacent: the blocks within `band` of the diagonal, level by level
        if (w + 1 < 4 && 1 <= band) inverse_block<AS, 1>(Am, Tm, w, j, m);
        else if (w == NW - 1) side();
        lds_sync();
        if (w + 2 < 4 && 2 <= band) inverse_block<AS, 2>(Am, Tm, w, j, m);
        lds_sync();
    }
}

// ---------------------------------------------------------------------------------------------
// map_kernel: (Phi, Psi) of one block of chunks
// ---------------------------------------------------------------------------------------------
// Wave w holds columns VPW w .. VPW w + VPW - 1 (16 wide) of Z (Dk x Dk, rows l) and the same
// rows of Psi (Dk x Dv), fp32 in accumulator registers:
//   Z[t][lt]   lane (j, n): Z[16 lt + 4 j + e][16 (VPW w + t) + n]
//   Psi[t][vt] lane (j, n): Psi[16 (VPW w + t) + 4 j + e][16 vt + n]
// Per kept chunk (last to first):  Y = Khat Z (Z as high + low bf16 parts),  Psi += Y^T Ut,
// Z <- e^{g_C} Z - W^T Y. A skipped chunk (SparseGDN: the state only decays) is Z <- e^{g_C} Z.
// Each iteration takes NH chunks (c, c - 1, ...); half h of the workgroup solves chunk c - h in
// LDS slot h (a half with no chunk, or a skipped one, runs through the same barriers on whatever
// its slot holds, and nothing reads the result).
// Khat = diag(e^{g_C - g}) K over a chunk's staged K rows, in place, by NT threads: each element
// rounded once from its product, the value the state steps' operand loads would otherwise form
// per use.
template <int D, class E, int NT>
__device__ __forceinline__ void scale_rows(typename E::T* R, const float* kh, int tid) {
    using T = typename E::T;
    constexpr int KP = row_stride<D, E>(), EPU = 4 / (int)sizeof(T) * 2;   // elements per 8 bytes
    constexpr int UPR = D / EPU, N = CH * UPR / NT;
    static_assert(CH * UPR % NT == 0, "whole units per thread");
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int u = tid + NT * i, r = u / UPR;
        uint2* p = reinterpret_cast<uint2*>(R + r * KP + (u % UPR) * EPU);
        const float sc = kh[r];
        if constexpr (sizeof(T) == 2) {   // four bf16
            const float4 x = load4(reinterpret_cast<const T*>(p));
            store4(reinterpret_cast<T*>(p), make_float4(x.x * sc, x.y * sc, x.z * sc, x.w * sc));
        } else {                          // two fp32
            const uint2 y = *p;
            *p = uint2{__float_as_uint(__uint_as_float(y.x) * sc), __float_as_uint(__uint_as_float(y.y) * sc)};
        }
    }
}

template <int D, class E>
constexpr size_t map_lds() {
    return MapCfg<D, E>::NH * ((Lds<D, E, false>::BYTES + 255) / 256 * 256);
}

template <int D, class E>
__global__ __launch_bounds__(512) void map_kernel(PrefArgs a) {
    using MC = MapCfg<D, E>;
    using C = Cfg<D, E, MC::NWS>;    // the state's distribution over the waves
    using CP = Cfg<D, E, MC::NWP>;   // the solve's, within a half
    using L = Lds<D, E, false>;
    using M = MM<E>;
    using T = typename E::T;
    using frag = typename M::frag;
    constexpr int KB = C::KB, NKD = C::NKD, NKT = C::NKT, NDT = C::NDT, VPW = C::VPW, KP = C::KP, AS = C::AS;
    constexpr int NH = MC::NH;
    constexpr size_t SLOT = (L::BYTES + 255) / 256 * 256;
    extern __shared__ __align__(16) unsigned char smem[];
    const int b = blockIdx.x, bh = blockIdx.y;
    const int lane0 = threadIdx.x & 63, j0 = lane0 >> 4, m0 = lane0 & 15;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = NH == 2 ? w / 4 : 0, hw = NH == 2 ? w % 4 : w;   // scalars
    const int c0 = b * a.m, c1 = min(a.nch, c0 + a.m);   // chunks [c0, c1), processed last to first
    unsigned char* my = smem + (size_t)half * SLOT;      // this half's slot
    __shared__ unsigned zf[MC::NWS];                     // per wave: its columns of Z are all zero

    f32x4 Z[VPW][NDT], Psi[VPW][NDT];
#pragma unroll
    for (int t = 0; t < VPW; ++t)
#pragma unroll
        for (int lt = 0; lt < NDT; ++lt) {
            Psi[t][lt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) Z[t][lt][e] = (16 * lt + 4 * j0 + e == 16 * (VPW * w + t) + m0) ? 1.f : 0.f;
        }

    // whether this wave's columns of Z are all exactly zero (the same answer in every lane)
    auto z_zero = [&]() {
        unsigned nz = 0;
#pragma unroll
        for (int t = 0; t < VPW; ++t)
#pragma unroll
            for (int lt = 0; lt < NDT; ++lt)
#pragma unroll
                for (int e = 0; e < 4; ++e) nz |= __float_as_uint(Z[t][lt][e]) & 0x7fffffffu;
        return __builtin_amdgcn_ballot_w64(nz != 0u) == 0;
    };

    Fetch<D, E, false, MC::NWP> fx;
    bool zero = false;   // the composed transition is exactly zero (scalar)
    unsigned keep = 0;
    if (c1 - 1 - half >= c0) {
        keep = keep_chunk(a, bh, c1 - 1 - half);
        fx.issue(a, bh, c1 - 1 - half, keep, 64 * hw + lane0, hw);
    }
    for (int c = c1 - 1; c >= c0; c -= NH) {
        const int lane = opaque(threadIdx.x & 63), j = lane >> 4, m = lane & 15, htid = 64 * hw + lane;
        const int mine = c - half;                     // this half's chunk (scalar)
        T* Kr = reinterpret_cast<T*>(my + L::O_K);
        GatesOf<E>* gt = reinterpret_cast<GatesOf<E>*>(my + L::O_G);
        if (mine >= c0) {
            if (keep) fx.rk.store(Kr, fx.n, htid);
            if (hw == 0) gate_scan(gt, fx.la, fx.bt, lane);
        }
        lds_sync();
        // the iteration's chunks and whether each updates the state (scalars, the same in every wave)
        unsigned kp[NH];
        bool any = false;
#pragma unroll
        for (int p = 0; p < NH; ++p) {
            kp[p] = c - p >= c0 ? keep_chunk(a, bh, c - p) : 0u;
            any = any || kp[p];
        }
        if (any) {
            frag kbe[CP::VPW][NKT], vb[CP::VPW][NKT];
            intra_solve<D, E, false, MC::NWP>(my, gt, a.band, hw, lane, [] {}, fx.vf, kbe, vb);
            // -W (token tiles x this wave's d tiles) and Ut (x its value tiles) of the half's
            // chunk, then the fragments the state step reads: -W^T [dt][kt] (A: rows d, k = token)
            // and Ut [kt][vt] (B: k = token, columns v). A (in the V-row space) was last read
            // before intra_solve's final barrier.
            const float* Tm = reinterpret_cast<const float*>(my + L::O_T);
            f32x4 wn[CP::VPW][4], ua[CP::VPW][4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                frag Tf[NKT];
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
                    if (kt <= C::kbmax(rt)) Tf[kt] = row_frag_f32<E>(Tm + (16 * rt + m) * AS, kt * KB, j);
#pragma unroll
                for (int t = 0; t < CP::VPW; ++t) {
                    wn[t][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    ua[t][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kt = 0; kt < NKT; ++kt)
                        if (kt <= C::kbmax(rt)) {
                            wn[t][rt] = M::mma(Tf[kt], kbe[t][kt], wn[t][rt]);
                            ua[t][rt] = M::mma(Tf[kt], vb[t][kt], ua[t][rt]);
                        }
                }
            }
#pragma unroll
            for (int t = 0; t < CP::VPW; ++t)
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    const int dt = CP::VPW * hw + t;
                    st_frag(my + L::O_V + (size_t)(dt * NKT + kt) * C::FR, lane, M::from_acc(wn[t], kt));
                    st_frag(my + L::O_UT + (size_t)(kt * NDT + dt) * C::FR, lane, M::from_acc(ua[t], kt));
                }
            // the solve is done with this half's K rows: scale them into Khat for the state steps
            if (mine >= c0 && (half ? kp[NH - 1] : kp[0])) scale_rows<D, E, 64 * MC::NWP>(Kr, gt->kh, 64 * hw + lane);
        }
        lds_sync();
        // the next iteration's rows and gates load while this one's state steps run
        if (mine - NH >= c0) {
            keep = keep_chunk(a, bh, mine - NH);
            fx.issue(a, bh, mine - NH, keep, htid, hw);
        }
#pragma unroll
        for (int p = 0; p < NH; ++p) {
            if (c - p < c0) break;   // scalar
            // A wave's step touches only its columns of Z and its rows of Psi; once those columns
            // are exactly zero, Y's columns are zero and the step leaves both as they are (with
            // strong decay, the pair's second step after the first has underflowed Z).
            if (p > 0 && z_zero()) continue;
            const unsigned char* sl = smem + (size_t)p * SLOT;
            const T* Ks = reinterpret_cast<const T*>(sl + L::O_K);
            const Gates* gs = reinterpret_cast<const Gates*>(sl + L::O_G);
            const float dec = gs->dec;
            if (!kp[p]) {
#pragma unroll
                for (int t = 0; t < VPW; ++t)
#pragma unroll
                    for (int lt = 0; lt < NDT; ++lt) Z[t][lt] = scale4(Z[t][lt], dec);
                continue;
            }
            // Y = Khat Z
            f32x4 Y[VPW][4];
#pragma unroll
            for (int t = 0; t < VPW; ++t)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) Y[t][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) {
                frag zh[VPW], zl[VPW];
#pragma unroll
                for (int t = 0; t < VPW; ++t) {
                    zh[t] = M::from_acc(Z[t], kd);
                    if constexpr (C::NSPLIT == 2) zl[t] = lo_from_acc<E>(Z[t], kd);
                }
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const frag kf = row_frag_raw<E>(Ks + (16 * rt + m) * KP, kd * KB, j);   // Khat rows
#pragma unroll
                    for (int t = 0; t < VPW; ++t) {
                        Y[t][rt] = M::mma(kf, zh[t], Y[t][rt]);
                        if constexpr (C::NSPLIT == 2) Y[t][rt] = M::mma(kf, zl[t], Y[t][rt]);
                    }
                }
            }
            frag Yf[VPW][NKT];
#pragma unroll
            for (int t = 0; t < VPW; ++t)
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) Yf[t][kt] = M::from_acc(Y[t], kt);
            // Psi += Y^T Ut
#pragma unroll
            for (int vt = 0; vt < NDT; ++vt)
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    const frag uf = ld_frag<frag>(sl + L::O_UT + (size_t)(kt * NDT + vt) * C::FR, lane);
#pragma unroll
                    for (int t = 0; t < VPW; ++t) Psi[t][vt] = M::mma(Yf[t][kt], uf, Psi[t][vt]);
                }
            // Z <- e^{g_C} Z - W^T Y
#pragma unroll
            for (int lt = 0; lt < NDT; ++lt) {
#pragma unroll
                for (int t = 0; t < VPW; ++t) Z[t][lt] = scale4(Z[t][lt], dec);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    const frag wf = ld_frag<frag>(sl + L::O_V + (size_t)(lt * NKT + kt) * C::FR, lane);
#pragma unroll
                    for (int t = 0; t < VPW; ++t) Z[t][lt] = M::mma(wf, Yf[t][kt], Z[t][lt]);
                }
            }
        }
        // Once every column of Z is exactly zero the earlier chunks cannot change Phi or Psi
        // (each of their steps multiplies Z), so the block's map is complete. With strong decay
        // this happens after a chunk or two: the product of a chunk's gates falls below fp32's
        // smallest subnormal.
        const bool wzero = z_zero();
        if (lane0 == 0) zf[w] = wzero ? 1u : 0u;
        lds_sync();   // the slots are free for the next chunks
        unsigned done = 1u;
#pragma unroll
        for (int i = 0; i < MC::NWS; ++i) done &= zf[i];
        if (__builtin_amdgcn_readfirstlane(done)) {   // the same decision in every wave
            zero = true;
            break;
        }
    }
    // Phi = Z^T as A operands (rows i = this wave's columns of Z, k = l), unless it is zero (the
    // flag says so and the pass over blocks does not read it), and Psi as tiles
    unsigned char* phi = ws_phi<D, E>(a, bh, b);
    f32x4* psi = ws_hs<D, E>(a, bh, b + 1);
    if (threadIdx.x == 0) *ws_flag<D, E>(a, bh, b) = zero ? 0 : 1;
#pragma unroll
    for (int t = 0; t < VPW; ++t) {
        const int it = VPW * w + t;
        if (!zero) {
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) {
                st_frag(phi + ((size_t)(it * NKD + kd) * C::NSPLIT) * C::FR, lane0, M::from_acc(Z[t], kd));
                if constexpr (C::NSPLIT == 2)
                    st_frag(phi + ((size_t)(it * NKD + kd) * 2 + 1) * C::FR, lane0, lo_from_acc<E>(Z[t], kd));
            }
        }
#pragma unroll
        for (int vt = 0; vt < NDT; ++vt) psi[(it * NDT + vt) * 64 + lane0] = Psi[t][vt];
    }
}

// ---------------------------------------------------------------------------------------------
// scan_kernel: block start states
// ---------------------------------------------------------------------------------------------
// One workgroup per slice and 16 value columns vt; wave w holds row tiles VPW w .. of H[:, vt].
// Step b: H_{b+1} = Phi_b H_b + Psi_b, the products as high and low bf16 parts
// (Phi_hi H_hi + Phi_lo H_hi + Phi_hi H_lo), which keeps fp32 accuracy; the waves exchange their
// rows of H as operand fragments through LDS (double-buffered by step parity).
template <int D, class E>
__global__ __launch_bounds__(256) void scan_kernel(PrefArgs a) {
    using C = Cfg<D, E>;
    using M = MM<E>;
    using frag = typename M::frag;
    constexpr int NKD = C::NKD, NDT = C::NDT, VPW = C::SVPW, FPD = C::FPD, NS = C::NSPLIT;
    __shared__ __align__(16) unsigned char hb[2 * NKD * NS * 1024];
    // Workgroup L of the 1-D grid takes value tile vt of slice bh. Workgroups go to the 8 XCDs in
    // turn (L mod 8), and each reads all of its slice's Phi_b: with a multiple of 8 slices the
    // NDT tiles of a slice share an XCD (and its L2), else the plain order.
    const int L = blockIdx.x;
    const bool xcd = a.BH % 8 == 0;
    const int vt = xcd ? (L >> 3) % NDT : L % NDT;
    const int bh = xcd ? ((L >> 3) / NDT) * 8 + (L & 7) : L / NDT;
    const int tid = threadIdx.x, lane = tid & 63, j = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    f32x4 H[VPW];
#pragma unroll
    for (int t = 0; t < VPW; ++t) {
        const int lt = VPW * w + t;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            H[t][e] = a.h0 ? a.h0[((size_t)bh * D + 16 * lt + 4 * j + e) * D + 16 * vt + m] : 0.f;
        ws_hs<D, E>(a, bh, 0)[(lt * NDT + vt) * 64 + lane] = H[t];
    }
    // A block whose map is zero leaves H_{b+1} = Psi_b, which its slot already holds: such blocks
    // are skipped, and H is reloaded from the slot before the next block that needs it. The flags
    // of 64 blocks at a time come in one load (lane i takes block b0 + i) and one ballot, so the
    // pass does not wait on one flag read per block. Phi_b and Psi_b do not depend on H: the next
    // live block's are loaded while this block's product runs (within the same 64 flags).
    frag ph[VPW][NKD][NS], pn[VPW][NKD][NS];   // this block's and the next live block's Phi operands
    f32x4 ps[VPW], psn[VPW];                   // their Psi tiles
    auto load_block = [&](int bb, frag (&p)[VPW][NKD][NS], f32x4 (&q)[VPW]) {
        const unsigned char* phi = ws_phi<D, E>(a, bh, bb);
        const f32x4* slot = ws_hs<D, E>(a, bh, bb + 1);
#pragma unroll
        for (int t = 0; t < VPW; ++t) {
            const int it = VPW * w + t;
            q[t] = slot[(it * NDT + vt) * 64 + lane];
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd)
#pragma unroll
                for (int s = 0; s < NS; ++s) p[t][kd][s] = ld_frag<frag>(phi + ((size_t)(it * NKD + kd) * NS + s) * 1024, lane);
        }
    };
    bool have = true;   // H holds H_b (scalar)
    int steps = 0;      // products formed so far: the LDS buffer alternates with them
    int pre = -1;       // the block whose operands are in pn / psn (scalar)
    unsigned long long live = 0;   // nonzero flags of blocks b0 .. b0 + 63 (bit i: block b0 + i)
    for (int b = 0; b + 1 < a.NB; ++b) {
        if ((b & 63) == 0) {
            const int nf = min(64, a.NB - 1 - b);
            const __amdgpu_buffer_rsrc_t rf = buffer_rsrc(ws_flag<D, E>(a, bh, b), nf * 4);
            live = __builtin_amdgcn_ballot_w64(buffer_load4(rf, lane * 4) != 0u);
        }
        if (((live >> (b & 63)) & 1ull) == 0) {
            have = false;
            continue;
        }
        if (!have) {
#pragma unroll
            for (int t = 0; t < VPW; ++t) H[t] = ws_hs<D, E>(a, bh, b)[((VPW * w + t) * NDT + vt) * 64 + lane];
        }
        f32x4* slot = ws_hs<D, E>(a, bh, b + 1);
        if (pre == b) {
#pragma unroll
            for (int t = 0; t < VPW; ++t) {
                ps[t] = psn[t];
#pragma unroll
                for (int kd = 0; kd < NKD; ++kd)
#pragma unroll
                    for (int s = 0; s < NS; ++s) ph[t][kd][s] = pn[t][kd][s];
            }
        } else {
            load_block(b, ph, ps);
        }
        // the next live block of this window, if any: its operands load during this product
        const unsigned long long above = (b & 63) == 63 ? 0ull : live >> ((b & 63) + 1);
        if (above != 0ull) {
            pre = b + 1 + (int)__builtin_ctzll(above);
            load_block(pre, pn, psn);
        }
        f32x4 acc[VPW];
#pragma unroll
        for (int t = 0; t < VPW; ++t) acc[t] = ps[t];
        unsigned char* buf = hb + (size_t)(steps & 1) * NKD * NS * 1024;
        ++steps;
        have = true;
#pragma unroll
        for (int t = 0; t < VPW; ++t) {
            const int lt = VPW * w + t;
#pragma unroll
            for (int s = 0; s < NS; ++s) st_tile_part<E>(buf + (size_t)((lt / FPD) * NS + s) * 1024, lane, lt % FPD, H[t], s == 1);
        }
        lds_sync();
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) {
            frag hf[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) hf[s] = ld_frag<frag>(buf + (size_t)(kd * NS + s) * 1024, lane);
#pragma unroll
            for (int t = 0; t < VPW; ++t) {
                acc[t] = M::mma(ph[t][kd][0], hf[0], acc[t]);
                if constexpr (NS == 2) {
                    acc[t] = M::mma(ph[t][kd][1], hf[0], acc[t]);
                    acc[t] = M::mma(ph[t][kd][0], hf[1], acc[t]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < VPW; ++t) {
            H[t] = acc[t];
            slot[((VPW * w + t) * NDT + vt) * 64 + lane] = H[t];
        }
    }
}

// ---------------------------------------------------------------------------------------------
// out_kernel: outputs and the final state of one block
// ---------------------------------------------------------------------------------------------
// Wave w holds value columns VPW w .. VPW w + VPW - 1 (16 wide) of the fp32 state:
//   H[t][lt] lane (j, n): H[16 lt + 4 j + e][16 (VPW w + t) + n]
// Per chunk, after the intra-chunk solve:
//   U = Ut - W H;  O^T = e^g (H^T Q^T) + U^T P^T (stored);  H <- e^{g_C} H + Khat^T U
// (a skipped chunk's update leaves the decayed state; its outputs still use U). SKIP: the
// launch has a keep mask; a skipped chunk's Khat is zero (its gate scan zeroes e^{g_C - g}), so
// the same fused update leaves e^{g_C} H exactly.
template <int D, class E, bool SKIP>
__global__ __launch_bounds__(512) void out_kernel(PrefArgs a) {
    using C = Cfg<D, E, out_waves<D, E>()>;
    using L = Lds<D, E, true>;
    using M = MM<E>;
    using T = typename E::T;
    using frag = typename M::frag;
    constexpr int KB = C::KB, FPD = C::FPD, NKD = C::NKD, NKT = C::NKT, NDT = C::NDT, VPW = C::VPW, KP = C::KP,
                  AS = C::AS;
    extern __shared__ __align__(16) unsigned char smem[];
    const int b = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, j = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c0 = b * a.m, c1 = min(a.nch, c0 + a.m);
    T* Qr = reinterpret_cast<T*>(smem + L::O_Q);
    T* Kr = reinterpret_cast<T*>(smem + L::O_K);
    const float* Tm = reinterpret_cast<const float*>(smem + L::O_T);
    constexpr int GW = Fetch<D, E, true, C::NW>::GW;   // the wave that loads and scans the gates

    // the block's start state: h0 (or zeros) for a single block, else the scan's slot
    f32x4 H[VPW][NDT];
#pragma unroll
    for (int t = 0; t < VPW; ++t) {
        const int vt = VPW * w + t;
#pragma unroll
        for (int lt = 0; lt < NDT; ++lt) {
            if (a.NB > 1) {
                H[t][lt] = ws_hs<D, E>(a, bh, b)[(lt * NDT + vt) * 64 + lane];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    H[t][lt][e] = a.h0 ? a.h0[((size_t)bh * D + 16 * lt + 4 * j + e) * D + 16 * vt + m] : 0.f;
            }
        }
    }

    Fetch<D, E, true, C::NW> fx;
    fx.issue(a, bh, c0, true, tid, w);
    for (int c = c0; c < c1; ++c) {
        const int tid = 64 * w + opaque(threadIdx.x & 63), lane = tid & 63, j = lane >> 4, m = lane & 15;
        const int n = fx.n;
        // the gate arrays of chunk c and of chunk c + 1 (two LDS slots by chunk parity)
        GatesOf<E>* gt = reinterpret_cast<GatesOf<E>*>(smem + L::O_G + (size_t)((c - c0) & 1) * L::GSZ);
        GatesOf<E>* gn = reinterpret_cast<GatesOf<E>*>(smem + L::O_G + (size_t)((c - c0 + 1) & 1) * L::GSZ);
        fx.rq.store(Qr, n, tid);
        fx.rk.store(Kr, n, tid);
        // the first chunk's gates are scanned here; every later chunk's during the solve of the
        // chunk before it (side work of wave GW, below)
        if (c == c0 && w == GW) gate_scan(gt, fx.la, fx.bt, lane, !SKIP || fx.kp != 0u);
        // the next chunk's K and Q rows and gates load while this whole chunk runs (their
        // registers are free once stored); its V fragments follow once the solve has used this
        // chunk's (after W and Ut)
        const bool more = c + 1 < c1;
        if (more) {
            fx.start(a, bh, c + 1);
            fx.load_gates(a, tid);
            fx.load_k(a, tid);
            fx.load_q(a, tid);
        }
        lds_sync();
        frag kbe[VPW][NKT], vb[VPW][NKT];
        // The solve up to W and Ut is this workgroup's serial path; the other workgroup on the CU
        // is usually in its matrix-heavy state phase then. A higher wave priority lets the solve's
        // dependent steps issue first, and the state phase takes the idle cycles between them.
        __builtin_amdgcn_s_setprio(2);
        intra_solve<D, E, true, C::NW>(smem, gt, a.band, w, lane, [&] {
            if (more) gate_scan(gn, fx.la, fx.bt, lane, !SKIP || fx.kp != 0u);
        }, fx.vf, kbe, vb);
        // -W fragments [rt][kd] (A: rows token, k = d), each d tile filling its part, and Ut
        f32x4 U[VPW][4];
        {
            f32x4 wt[4][VPW];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                frag Tf[NKT];
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
                    if (kt <= C::kbmax(rt)) Tf[kt] = row_frag_f32<E>(Tm + (16 * rt + m) * AS, kt * KB, j);
#pragma unroll
                for (int t = 0; t < VPW; ++t) {
                    wt[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
                    U[t][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kt = 0; kt < NKT; ++kt)
                        if (kt <= C::kbmax(rt)) {
                            wt[rt][t] = M::mma(kbe[t][kt], Tf[kt], wt[rt][t]);
                            U[t][rt] = M::mma(Tf[kt], vb[t][kt], U[t][rt]);
                        }
                }
            }
            // A (in the V-row space) was last read before intra_solve's final barrier
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int t = 0; t < VPW; ++t) {
                    const int dt = VPW * w + t;
                    st_tile_part<E>(smem + L::O_V + (size_t)(rt * NKD + dt / FPD) * C::FR, lane, dt % FPD, wt[rt][t]);
                }
        }
        lds_sync();
        __builtin_amdgcn_s_setprio(0);
        if (more) fx.load_v(a, tid, w);   // apart from the burst of K and Q loads at the top
        const float dec = gt->dec;
        // U = Ut - W H
        frag Hf[VPW][NKD];
#pragma unroll
        for (int t = 0; t < VPW; ++t)
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) Hf[t][kd] = M::from_acc(H[t], kd);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) {
                const frag wf = ld_frag<frag>(smem + L::O_V + (size_t)(rt * NKD + kd) * C::FR, lane);
#pragma unroll
                for (int t = 0; t < VPW; ++t) U[t][rt] = M::mma(wf, Hf[t][kd], U[t][rt]);
            }
        frag Uf[VPW][NKT];
#pragma unroll
        for (int t = 0; t < VPW; ++t)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) Uf[t][kt] = M::from_acc(U[t], kt);
        // O^T = e^g (H^T Q^T) + U^T P^T, lane (j, n): O[16 rt + n][16 vt + 4 j .. + 3], and
        // H <- e^{g_C} H + Khat^T U (H itself is no longer read: the products use Hf). The two
        // are interleaved, two value tiles of the update per output tile, so that the update's
        // independent products fill the output's dependent chains. When e^{g_C} is exactly zero
        // (strong decay: the chunk's gates multiply below fp32's smallest subnormal) the decayed
        // state is zero and the update starts from zero instead of scaling H: one straight-line
        // copy of the loop per case, chosen by a scalar branch.
        const long t0 = (long)c * CH;
        const __amdgpu_buffer_rsrc_t ro =
            buffer_rsrc(static_cast<T*>(a.o) + ((size_t)bh * a.L + t0) * D, n * D * (int)sizeof(T));
        auto outputs_and_update = [&](auto dz) {
            constexpr bool DZ = decltype(dz)::value;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 ot[VPW];
#pragma unroll
                for (int t = 0; t < VPW; ++t) ot[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kd = 0; kd < NKD; ++kd) {
                    const frag qf = row_frag_raw<E>(Qr + (16 * rt + m) * KP, kd * KB, j);
#pragma unroll
                    for (int t = 0; t < VPW; ++t) ot[t] = M::mma(Hf[t][kd], qf, ot[t]);
                }
#pragma unroll
                for (int l = 0; l < NDT / 4; ++l) {
                    const int lt = (NDT / 4) * rt + l;
#pragma unroll
                    for (int t = 0; t < VPW; ++t) H[t][lt] = DZ ? f32x4{0.f, 0.f, 0.f, 0.f} : scale4(H[t][lt], dec);
#pragma unroll
                    for (int kt = 0; kt < NKT; ++kt) {
                        const frag kf = ld_frag<frag>(smem + L::O_KH + (size_t)(lt * NKT + kt) * C::FR, lane);
#pragma unroll
                        for (int t = 0; t < VPW; ++t) H[t][lt] = M::mma(kf, Uf[t][kt], H[t][lt]);
                    }
                }
                const float eg = gt->eg[16 * rt + m];
#pragma unroll
                for (int t = 0; t < VPW; ++t) ot[t] = scale4(ot[t], eg);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
                    if (kt <= C::kbmax(rt)) {
                        const frag pf = ld_frag<frag>(smem + L::O_P + (size_t)(rt * NKT + kt) * C::FR, lane);
#pragma unroll
                        for (int t = 0; t < VPW; ++t) ot[t] = M::mma(Uf[t][kt], pf, ot[t]);
                    }
#pragma unroll
                for (int t = 0; t < VPW; ++t)
                    buffer_store4(ro, ((16 * rt + m) * D + 16 * (VPW * w + t) + 4 * j) * (int)sizeof(T),
                                  make_float4(ot[t][0], ot[t][1], ot[t][2], ot[t][3]), T{});
                __builtin_amdgcn_sched_barrier(0);   // keeps each tile's operand loads in its step
            }
        };
        if (__builtin_amdgcn_readfirstlane(__float_as_uint(dec)) == 0u) outputs_and_update(std::true_type{});
        else outputs_and_update(std::false_type{});
        lds_sync();   // the chunk's LDS is free for the next one
    }
    if (b == a.NB - 1) {
#pragma unroll
        for (int t = 0; t < VPW; ++t)
#pragma unroll
            for (int lt = 0; lt < NDT; ++lt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.h_final[((size_t)bh * D + 16 * lt + 4 * j + e) * D + 16 * (VPW * w + t) + m] = H[t][lt][e];
    }
}

// h_final = h0 (or zeros) for L = 0
__global__ void copy_state_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

// ---------------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------------
static int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return n;
}

// bytes of workspace per slice for NB blocks (none for one block)
static size_t ws_per_slice(int NB, int D) { return NB <= 1 ? 0 : (size_t)(2 * NB - 1) * 4 * D * D + flag_bytes(NB); }

// Blocks per slice: one where the slices alone give every CU a workgroup (the sequential pass per
// head in one workgroup, no map work), else enough for about two output workgroups per CU, at
// most one per chunk.
static long preferred_blocks(long BH, long nch) {
    const int ncu = device_cus() > 0 ? device_cus() : 256;
    if (BH >= ncu) return 1;
    long nb = (2L * ncu + BH - 1) / BH;
    return nb < nch ? nb : nch;
}

size_t prefill_workspace_bytes(long BH, long L, int D, int /*dtype*/) {
    const long nch = (L + CH - 1) / CH;
    if (nch == 0) return 0;
    long nb = preferred_blocks(BH, nch);
    const long m = (nch + nb - 1) / nb;
    nb = (nch + m - 1) / m;
    return (size_t)BH * ws_per_slice((int)nb, D);
}

// no workspace is needed: the whole sequence then runs as one block per slice
size_t prefill_workspace_min_bytes(long, long, int, int) { return 0; }

// Static scratch for the prefill entry point that allocates nothing: it holds that call's block
// maps and block start states, laid out as a caller's workspace. Each device holds its own copy
// from the time the library's code is loaded on it until the process ends.
static __device__ __align__(256) unsigned char scratch[GDN_PREFILL_NOALLOC_MAX_BYTES];

int prefill_scratch(void** ptr) {
    constexpr int MAXDEV = 64;
    static std::atomic<void*> addr[MAXDEV];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAXDEV) return -1;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        // the device address of this device's copy (the array's name is only a host-side handle)
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return -1;
        addr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return 0;
}

// Optional per-kernel timing: HIP events recorded around each launch on the caller's stream.
namespace {
struct StageTimer {
    struct Rec {
        int stage, dev;
        hipEvent_t begin, end;
    };
    std::mutex mu;
    std::atomic<bool> on{false};
    std::vector<std::pair<int, hipEvent_t>> pool;   // (device, event): events belong to a device
    std::vector<Rec> rec;
    hipEvent_t get(int dev) {
        for (size_t i = pool.size(); i-- > 0;)
            if (pool[i].first == dev) {
                hipEvent_t e = pool[i].second;
                pool.erase(pool.begin() + (long)i);
                return e;
            }
        hipEvent_t e = nullptr;
        return hipEventCreate(&e) == hipSuccess ? e : nullptr;
    }
};
StageTimer& timer() {
    static StageTimer t;
    return t;
}
// launches one kernel through f(), bracketed by events when timing is on; true if the launch
// was accepted
template <class F>
bool timed(int stage, hipStream_t s, F&& f) {
    StageTimer& t = timer();
    if (!t.on.load(std::memory_order_relaxed)) {
        f();
        return hipGetLastError() == hipSuccess;
    }
    std::lock_guard<std::mutex> g(t.mu);
    int dev = 0;
    (void)hipGetDevice(&dev);
    hipEvent_t e0 = t.get(dev), e1 = t.get(dev);
    if (e0 && e1) (void)hipEventRecord(e0, s);
    f();
    const bool ok = hipGetLastError() == hipSuccess;
    if (e0 && e1) {
        (void)hipEventRecord(e1, s);
        t.rec.push_back({stage, dev, e0, e1});
    } else {   // an event could not be created: this launch goes untimed
        if (e0) t.pool.push_back({dev, e0});
        if (e1) t.pool.push_back({dev, e1});
    }
    return ok;
}
}  // namespace

void prefill_timing(bool enable) { timer().on.store(enable); }

int prefill_kernel_times(float* ms, int* launches) {
    StageTimer& t = timer();
    std::lock_guard<std::mutex> g(t.mu);
    float sum[3] = {0.f, 0.f, 0.f};
    int cnt[3] = {0, 0, 0};
    bool ok = true;
    for (auto& r : t.rec) {
        float x = 0.f;
        if (hipEventSynchronize(r.end) != hipSuccess || hipEventElapsedTime(&x, r.begin, r.end) != hipSuccess) ok = false;
        sum[r.stage] += x;
        cnt[r.stage] += 1;
        t.pool.push_back({r.dev, r.begin});
        t.pool.push_back({r.dev, r.end});
    }
    t.rec.clear();
    for (int i = 0; i < 3; ++i) {
        if (ms) ms[i] = sum[i];
        if (launches) launches[i] = cnt[i];
    }
    return ok ? 0 : -1;
}

template <int D, class E>
struct Launch {
    static bool attributes() {
        static const bool ok =
            hipFuncSetAttribute(reinterpret_cast<const void*>(&map_kernel<D, E>), hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)map_lds<D, E>()) == hipSuccess &&
            hipFuncSetAttribute(reinterpret_cast<const void*>(&out_kernel<D, E, false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lds<D, E, true>::BYTES) == hipSuccess &&
            hipFuncSetAttribute(reinterpret_cast<const void*>(&out_kernel<D, E, true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lds<D, E, true>::BYTES) == hipSuccess;
        return ok;
    }
    static int run(const PrefArgs& a, hipStream_t s) {
        if (!attributes()) return -1;
        constexpr size_t lds_map = map_lds<D, E>(), lds_out = Lds<D, E, true>::BYTES;
        if (a.NB > 1) {
            if (!timed(0, s, [&] {
                    hipLaunchKernelGGL((map_kernel<D, E>), dim3(a.NB - 1, a.BH), dim3(64 * MapCfg<D, E>::NWS), lds_map,
                                       s, a);
                }))
                return -1;
            if (!timed(1, s, [&] { hipLaunchKernelGGL((scan_kernel<D, E>), dim3(D / 16 * a.BH), dim3(256), 0, s, a); }))
                return -1;
        }
        return timed(2, s, [&] {
                   if (a.keep)
                       hipLaunchKernelGGL((out_kernel<D, E, true>), dim3(a.NB, a.BH), dim3(64 * out_waves<D, E>()),
                                          lds_out, s, a);
                   else
                       hipLaunchKernelGGL((out_kernel<D, E, false>), dim3(a.NB, a.BH), dim3(64 * out_waves<D, E>()),
                                          lds_out, s, a);
               })
                   ? 0
                   : -1;
    }
};

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
    // as many blocks as preferred and as the workspace holds
    long nb = preferred_blocks(BH, nch);
    while (nb > 1 && (size_t)BH * ws_per_slice((int)nb, D) > ws_bytes) --nb;
    const long m = (nch + nb - 1) / nb;
    nb = (nch + m - 1) / m;
    PrefArgs a{q, k, v, beta, log_alpha, h0, keep, o, h_final, static_cast<unsigned char*>(ws), L, BH, (int)nch, (int)m,
               (int)nb, band};
    if (D == 128 && dtype == 0) return Launch<128, BF16>::run(a, stream);
    if (D == 128) return Launch<128, F32>::run(a, stream);
    if (dtype == 0) return Launch<64, BF16>::run(a, stream);
    return Launch<64, F32>::run(a, stream);
}

}  // namespace gdn
