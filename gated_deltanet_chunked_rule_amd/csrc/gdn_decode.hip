// Recurrent decode step of the gated delta rule on gfx950.
//
// One generated token per sequence costs a constant amount of work, independent of how many
// tokens came before (AI RnD Day channel post, tgstat.ru, section "Linear attention"). With the
// key-major state H = S^T (Dk x Dv) the token update S_t = a S (I - beta k k^T) + beta v k^T is
//     p = H^T k,   r = H^T q              (one pass over H, both reductions at once)
//     u = beta (v - a p)
//     H <- a H + k u^T                     (rank-1 update, written back in place)
//     o = S_t q = a r + u (k^T q)
// so the state is read from HBM once and written once: the kernel is bound by HBM bandwidth.
//
// Work split: one 1024-thread workgroup per (sequence, head). Thread t owns 4 consecutive value
// columns (one 16-byte vector per state row) of D/RG rows, rows interleaved so that every wave-wide
// load or store covers whole, adjacent 512-byte (D=128) or 256-byte (D=64) rows. The whole 64 KB
// (D=128) state block lives in registers between the read and the write, at 4 rows (16 VGPRs) per
// thread, which leaves room for many workgroups per CU to keep HBM busy (with 256 threads per
// slice the state takes 64 VGPRs per thread and the step ran about 12% slower).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int D, class E>
__global__ __launch_bounds__(1024) void decode_kernel(const typename E::T* __restrict__ q,
                                                     const typename E::T* __restrict__ k,
                                                     const typename E::T* __restrict__ v,
                                                     const float* __restrict__ beta,
                                                     const float* __restrict__ log_alpha,
                                                     float* __restrict__ state,
                                                     typename E::T* __restrict__ o) {
    constexpr int CG = D / 4;          // column groups of 4
    constexpr int THREADS = 1024;
    constexpr int RG = THREADS / CG;   // row groups
    constexpr int RPT = D / RG;        // rows per thread
    constexpr int NW = THREADS / 64;   // waves per workgroup
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    const size_t slice = blockIdx.x;

    __shared__ float sk[D], sq[D];
    __shared__ float4 red_p[NW][CG], red_r[NW][CG];
    __shared__ float s_kq;

    const typename E::T* qs = q + slice * D;
    const typename E::T* ks = k + slice * D;
    if (t < D) { sk[t] = E::load(ks + t); sq[t] = E::load(qs + t); }

    float* H = state + slice * (size_t)D * D;
    f32x4 h[RPT];
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr)
        h[rr] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(H + (size_t)(rr * RG + rg) * D) + cg);
    __syncthreads();

    // k^T q by wave 0
    if (t < 64) {
        float acc = 0.f;
        for (int i = t; i < D; i += 64) acc += sk[i] * sq[i];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (t == 0) s_kq = acc;
    }

    float4 p = make_float4(0.f, 0.f, 0.f, 0.f), r = p;
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
        const int i = rr * RG + rg;
        const float ki = sk[i], qi = sq[i];
        p.x += h[rr][0] * ki; p.y += h[rr][1] * ki; p.z += h[rr][2] * ki; p.w += h[rr][3] * ki;
        r.x += h[rr][0] * qi; r.y += h[rr][1] * qi; r.z += h[rr][2] * qi; r.w += h[rr][3] * qi;
    }
    // reduce over the row groups of this wave (lanes that share cg)
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
        p.x += __shfl_xor(p.x, off); p.y += __shfl_xor(p.y, off);
        p.z += __shfl_xor(p.z, off); p.w += __shfl_xor(p.w, off);
        r.x += __shfl_xor(r.x, off); r.y += __shfl_xor(r.y, off);
        r.z += __shfl_xor(r.z, off); r.w += __shfl_xor(r.w, off);
    }
    const int w = t / 64, lane = t % 64;
    if (lane < CG) { red_p[w][cg] = p; red_r[w][cg] = r; }
    __syncthreads();
    p = red_p[0][cg]; r = red_r[0][cg];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) {
        const float4 a = red_p[ww][cg], b = red_r[ww][cg];
        p.x += a.x; p.y += a.y; p.z += a.z; p.w += a.w;
        r.x += b.x; r.y += b.y; r.z += b.z; r.w += b.w;
    }

    const float bt = beta[slice];
    const float a = __expf(log_alpha[slice]);
    const float4 vv = load4(v + slice * D + cg * 4);
    float4 u;
    u.x = bt * (vv.x - a * p.x); u.y = bt * (vv.y - a * p.y);
    u.z = bt * (vv.z - a * p.z); u.w = bt * (vv.w - a * p.w);

#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
        const int i = rr * RG + rg;
        const float ki = sk[i];
        f32x4 x;
        x[0] = a * h[rr][0] + ki * u.x; x[1] = a * h[rr][1] + ki * u.y;
        x[2] = a * h[rr][2] + ki * u.z; x[3] = a * h[rr][3] + ki * u.w;
        __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(H + (size_t)i * D) + cg);
    }
    if (rg == 0) {
        const float kq = s_kq;
        float4 out;
        out.x = a * r.x + u.x * kq; out.y = a * r.y + u.y * kq;
        out.z = a * r.z + u.z * kq; out.w = a * r.w + u.w * kq;
        store4(o + slice * D + cg * 4, out);
    }
}

int launch_decode(const void* q, const void* k, const void* v, const float* beta, const float* log_alpha,
                  float* state, void* o, long slices, int D, int dtype, hipStream_t stream) {
    dim3 grid((unsigned)slices), block(1024);
#define GDN_DEC(DD, EE)                                                                                   \
    hipLaunchKernelGGL((decode_kernel<DD, EE>), grid, block, 0, stream, (const EE::T*)q, (const EE::T*)k, \
                       (const EE::T*)v, beta, log_alpha, state, (EE::T*)o)
    if (D == 128 && dtype == 0) GDN_DEC(128, BF16);
    else if (D == 128) GDN_DEC(128, F32);
    else if (D == 64 && dtype == 0) GDN_DEC(64, BF16);
    else GDN_DEC(64, F32);
#undef GDN_DEC
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gdn
