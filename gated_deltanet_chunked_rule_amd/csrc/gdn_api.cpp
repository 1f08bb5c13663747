// C ABI of libgdn.so: argument validation, then launches on the caller's stream.
// Every check runs before any launch, so an error return means nothing was enqueued.
#include <hip/hip_runtime.h>
#include <atomic>
#include <climits>
#include <cstdint>
#include <cstring>

#include "../../include/gdn.h"
#include "gdn_launch.h"

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range rng(const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

bool aligned(const void* p, uintptr_t to) { return (reinterpret_cast<uintptr_t>(p) & (to - 1)) == 0; }

// per-device check that the current device is gfx950: 0 unknown, 1 ok, -1 not gfx950
std::atomic<int> g_dev_ok[64];

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GDN_ERR_LAUNCH;
    if (dev < 64) {
        const int st = g_dev_ok[dev].load(std::memory_order_relaxed);
        if (st == 1) return GDN_OK;
        if (st == -1) return GDN_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GDN_ERR_LAUNCH;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_dev_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
    return ok ? GDN_OK : GDN_ERR_DEVICE;
}

int check_dims(long B, long H, long L, int Dk, int Dv, int dtype) {
    if (dtype != GDN_BF16 && dtype != GDN_F32) return GDN_ERR_DTYPE;
    if (Dk != Dv || (Dk != 64 && Dk != 128)) return GDN_ERR_SHAPE;
    if (B < 1 || H < 1 || L < 0) return GDN_ERR_SHAPE;
    if (B * H > 65535) return GDN_ERR_SHAPE;                 // workgroup grid rows
    if (L > (long)INT_MAX - 64) return GDN_ERR_SHAPE;
    return GDN_OK;
}

int validate_prefill(const void* q, const void* k, const void* v, const float* beta, const float* log_alpha,
                     const unsigned char* keep, bool skip, const float* h0, void* o, float* h_final, int B, int H,
                     int L, int Dk, int Dv, int dtype, void* workspace, size_t workspace_bytes, bool delta) {
    int st = check_dims(B, H, L, Dk, Dv, dtype);
    if (st != GDN_OK) return st;
    // the smallest workspace the entry point accepts (0: none needed)
    const size_t need = delta ? gdn::prefill_workspace_min_bytes((long)B * H, L, Dk, dtype)
                              : gdn::linattn_workspace_min_bytes((long)B * H, L, Dk);
    if (!h_final) return GDN_ERR_NULL;
    if (L > 0 && (!q || !k || !v || !o)) return GDN_ERR_NULL;   // L = 0 reads no token data
    if (delta && L > 0 && (!beta || !log_alpha)) return GDN_ERR_NULL;
    if (!delta && beta) return GDN_ERR_NULL;        // log_alpha is optional without the delta term
    if (skip && L > 0 && !keep) return GDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, beta, log_alpha, h0, o, h_final};
    for (const void* p : ptrs)
        if (p && !aligned(p, 16)) return GDN_ERR_ALIGN;
    const size_t esz = dtype == GDN_BF16 ? 2 : 4;
    const size_t BH = (size_t)B * H;
    const size_t tok = BH * (size_t)L;
    if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
    // a workspace is optional where none is needed, but one that is handed over is used
    const bool use_ws = workspace && workspace_bytes > 0;
    if (use_ws && !aligned(workspace, 256)) return GDN_ERR_ALIGN;
    const size_t nchk = ((size_t)L + 63) / 64;
    const Range in[] = {rng(q, tok * Dk * esz), rng(k, tok * Dk * esz), rng(v, tok * Dv * esz),
                        rng(beta, beta ? tok * 4 : 0), rng(log_alpha, log_alpha ? tok * 4 : 0),
                        rng(keep, keep ? BH * nchk : 0), rng(h0, h0 ? BH * Dk * Dv * 4 : 0)};
    const Range ro = rng(o, tok * Dv * esz), rh = rng(h_final, BH * Dk * Dv * 4);
    const Range rw = rng(workspace, use_ws ? workspace_bytes : 0);
    for (int i = 0; i < 7; ++i) {
        if (overlap(ro, in[i]) || overlap(rw, in[i])) return GDN_ERR_ALIAS;
        if (i == 6 && h0 == h_final) continue;  // in-place state update is allowed
        if (overlap(rh, in[i])) return GDN_ERR_ALIAS;
    }
    if (overlap(ro, rh) || overlap(ro, rw) || overlap(rh, rw)) return GDN_ERR_ALIAS;
    return GDN_OK;
}

// the gated delta-rule prefill entry points
int prefill(const void* q, const void* k, const void* v, const float* beta, const float* log_alpha,
            const unsigned char* keep, bool skip, const float* h0, void* o, float* h_final, int B, int H, int L,
            int Dk, int Dv, int dtype, void* workspace, size_t workspace_bytes, void* stream, int band = 3) {
    if (band < 0 || band > 3) return GDN_ERR_SHAPE;
    int st = validate_prefill(q, k, v, beta, log_alpha, keep, skip, h0, o, h_final, B, H, L, Dk, Dv, dtype,
                              workspace, workspace_bytes, true);
    if (st != GDN_OK) return st;
    st = check_device();
    if (st != GDN_OK) return st;
    return gdn::launch_prefill(q, k, v, beta, log_alpha, keep, h0, o, h_final, B * H, L, Dk, dtype, band,
                               workspace, workspace_bytes, static_cast<hipStream_t>(stream)) == 0
               ? GDN_OK
               : GDN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int gdn_prefill_timing(int enable) {
    gdn::prefill_timing(enable != 0);
    return GDN_OK;
}

int gdn_prefill_kernel_times(float* ms, int* launches) {
    return gdn::prefill_kernel_times(ms, launches) == 0 ? GDN_OK : GDN_ERR_LAUNCH;
}

const char* gdn_status_string(int status) {
    switch (status) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL or a forbidden one is set";
        case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: unsupported shape";
        case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: unsupported dtype";
        case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: pointer not 16-byte (workspace: 256-byte) aligned";
        case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS: an output overlaps an input or another output";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
        case GDN_ERR_LAUNCH: return "GDN_ERR_LAUNCH: HIP runtime error";
        case GDN_ERR_DEVICE: return "GDN_ERR_DEVICE: current device is not gfx950";
        case GDN_ERR_SCRATCH:
            return "GDN_ERR_SCRATCH: scratch_bytes exceeds the library's static scratch (GDN_PREFILL_NOALLOC_MAX_BYTES)";
        default: return "unknown status";
    }
}

size_t gdn_prefill_workspace_size(int B, int H, int L, int Dk, int Dv, int dtype) {
    if (check_dims(B, H, L, Dk, Dv, dtype) != GDN_OK) return 0;
    return gdn::prefill_workspace_bytes((long)B * H, L, Dk, dtype);
}

int gdn_prefill_fwd(const void* q, const void* k, const void* v, const float* beta, const float* log_alpha,
                    const float* h0, void* o, float* h_final, int B, int H, int L, int Dk, int Dv, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
    return prefill(q, k, v, beta, log_alpha, nullptr, false, h0, o, h_final, B, H, L, Dk, Dv, dtype, workspace,
                   workspace_bytes, stream);
}

int gdn_prefill_fwd_noalloc(const void* q, const void* k, const void* v, const float* beta, const float* log_alpha,
                            const float* h0, void* o, float* h_final, int B, int H, int L, int Dk, int Dv, int dtype,
                            size_t scratch_bytes, void* stream) {
    if (scratch_bytes > GDN_PREFILL_NOALLOC_MAX_BYTES) return GDN_ERR_SCRATCH;
    // the arguments first (no workspace: none is required), then the scratch's address
    int st = validate_prefill(q, k, v, beta, log_alpha, nullptr, false, h0, o, h_final, B, H, L, Dk, Dv, dtype,
                              nullptr, 0, true);
    if (st != GDN_OK) return st;
    st = check_device();
    if (st != GDN_OK) return st;
    void* ws = nullptr;
    if (scratch_bytes > 0 && gdn::prefill_scratch(&ws) != 0) return GDN_ERR_LAUNCH;
    return gdn::launch_prefill(q, k, v, beta, log_alpha, nullptr, h0, o, h_final, B * H, L, Dk, dtype, 3, ws,
                               scratch_bytes, static_cast<hipStream_t>(stream)) == 0
               ? GDN_OK
               : GDN_ERR_LAUNCH;
}

int gdn_prefill_skip_fwd(const void* q, const void* k, const void* v, const float* beta, const float* log_alpha,
                         const unsigned char* keep, const float* h0, void* o, float* h_final, int B, int H, int L,
                         int Dk, int Dv, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return prefill(q, k, v, beta, log_alpha, keep, true, h0, o, h_final, B, H, L, Dk, Dv, dtype, workspace,
                   workspace_bytes, stream);
}

int gdn_prefill_banded_fwd(const void* q, const void* k, const void* v, const float* beta, const float* log_alpha,
                           const float* h0, void* o, float* h_final, int B, int H, int L, int Dk, int Dv, int dtype,
                           int band, void* workspace, size_t workspace_bytes, void* stream) {
    return prefill(q, k, v, beta, log_alpha, nullptr, false, h0, o, h_final, B, H, L, Dk, Dv, dtype, workspace,
                   workspace_bytes, stream, band);
}

int linattn_prefill_fwd(const void* q, const void* k, const void* v, const float* beta, const float* log_alpha,
                        const float* h0, void* o, float* h_final, int B, int H, int L, int Dk, int Dv, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
    int st = validate_prefill(q, k, v, beta, log_alpha, nullptr, false, h0, o, h_final, B, H, L, Dk, Dv, dtype,
                              workspace, workspace_bytes, false);
    if (st != GDN_OK) return st;
    st = check_device();
    if (st != GDN_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int rc = L == 0 ? gdn::launch_prefill(q, k, v, nullptr, nullptr, nullptr, h0, o, h_final, B * H, 0, Dk,
                                                dtype, 3, workspace, workspace_bytes, s)
                          : gdn::launch_linattn(q, k, v, log_alpha, h0, o, h_final, B * H, L, Dk, dtype, workspace,
                                                workspace_bytes, s);
    return rc == 0 ? GDN_OK : GDN_ERR_LAUNCH;
}

size_t linattn_prefill_workspace_size(int B, int H, int L, int Dk, int Dv, int dtype) {
    if (check_dims(B, H, L, Dk, Dv, dtype) != GDN_OK) return 0;
    return gdn::linattn_workspace_bytes((long)B * H, L, Dk);
}

size_t gla_prefill_workspace_size(int B, int H, int L, int Dk, int Dv, int dtype) {
    if (check_dims(B, H, L, Dk, Dv, dtype) != GDN_OK) return 0;
    return gdn::gla_workspace_bytes((long)B * H, L, Dk);
}

int gla_prefill_fwd(const void* q, const void* k, const void* v, const float* log_alpha, const float* h0, void* o,
                    float* h_final, int B, int H, int L, int Dk, int Dv, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
    int st = check_dims(B, H, L, Dk, Dv, dtype);
    if (st != GDN_OK) return st;
    if (!h_final) return GDN_ERR_NULL;
    if (L > 0 && (!q || !k || !v || !o || !log_alpha)) return GDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, log_alpha, h0, o, h_final};
    for (const void* p : ptrs)
        if (p && !aligned(p, 16)) return GDN_ERR_ALIGN;
    const size_t need = gdn::gla_workspace_min_bytes((long)B * H, L, Dk);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return GDN_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return GDN_ERR_ALIGN;
    }
    const size_t esz = dtype == GDN_BF16 ? 2 : 4;
    const size_t BH = (size_t)B * H, tok = BH * (size_t)L;
    const Range in[] = {rng(q, tok * Dk * esz), rng(k, tok * Dk * esz), rng(v, tok * Dv * esz),
                        rng(log_alpha, log_alpha ? tok * Dk * 4 : 0), rng(h0, h0 ? BH * Dk * Dv * 4 : 0)};
    const Range ro = rng(o, tok * Dv * esz), rh = rng(h_final, BH * Dk * Dv * 4);
    const Range rw = rng(workspace, workspace && need ? workspace_bytes : 0);
    for (int i = 0; i < 5; ++i) {
        if (overlap(ro, in[i]) || overlap(rw, in[i])) return GDN_ERR_ALIAS;
        if (i == 4 && h0 == h_final) continue;  // in-place state update is allowed
        if (overlap(rh, in[i])) return GDN_ERR_ALIAS;
    }
    if (overlap(ro, rh) || overlap(ro, rw) || overlap(rh, rw)) return GDN_ERR_ALIAS;
    st = check_device();
    if (st != GDN_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int rc = L == 0 ? gdn::launch_prefill(q, k, v, nullptr, nullptr, nullptr, h0, o, h_final, B * H, 0, Dk,
                                                dtype, 3, workspace, workspace_bytes, s)
                          : gdn::launch_gla(q, k, v, log_alpha, h0, o, h_final, B * H, L, Dk, dtype, workspace,
                                            workspace_bytes, s);
    return rc == 0 ? GDN_OK : GDN_ERR_LAUNCH;
}

size_t linattn_bidir_workspace_size(int B, int H, int L, int Dk, int Dv, int dtype) {
    if (check_dims(B, H, L, Dk, Dv, dtype) != GDN_OK) return 0;
    return gdn::bidir_workspace_bytes((long)B * H, L, Dk, dtype);
}

int linattn_bidir_fwd(const void* q, const void* k, const void* v, void* o, float* kv_out, int B, int H, int L,
                      int Dk, int Dv, int dtype, int flags, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_dims(B, H, L, Dk, Dv, dtype);
    if (st != GDN_OK) return st;
    if (flags & ~(GDN_BIDIR_NORMALIZE | GDN_BIDIR_ELU1)) return GDN_ERR_SHAPE;
    if (L > 0 && (!q || !k || !v || !o)) return GDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, o, kv_out};
    for (const void* p : ptrs)
        if (p && !aligned(p, 16)) return GDN_ERR_ALIGN;
    const size_t need = gdn::bidir_workspace_bytes((long)B * H, L, Dk, dtype);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return GDN_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return GDN_ERR_ALIGN;
    }
    const size_t esz = dtype == GDN_BF16 ? 2 : 4;
    const size_t BH = (size_t)B * H, tok = BH * (size_t)L;
    const Range in[] = {rng(q, tok * Dk * esz), rng(k, tok * Dk * esz), rng(v, tok * Dv * esz)};
    const Range ro = rng(o, tok * Dv * esz), rk = rng(kv_out, kv_out ? BH * Dk * Dv * 4 : 0);
    const Range rw = rng(workspace, workspace && need ? workspace_bytes : 0);
    for (const Range& r : in)
        if (overlap(ro, r) || overlap(rk, r) || overlap(rw, r)) return GDN_ERR_ALIAS;
    if (overlap(ro, rk) || overlap(ro, rw) || overlap(rk, rw)) return GDN_ERR_ALIAS;
    st = check_device();
    if (st != GDN_OK) return st;
    return gdn::launch_bidir(q, k, v, o, kv_out, (int)BH, L, Dk, dtype, flags, workspace,
                             static_cast<hipStream_t>(stream)) == 0
               ? GDN_OK
               : GDN_ERR_LAUNCH;
}

int gdn_decode_step(const void* q, const void* k, const void* v, const float* beta, const float* log_alpha,
                    float* state, void* o, int N, int H, int Dk, int Dv, int dtype, void* stream) {
    if (dtype != GDN_BF16 && dtype != GDN_F32) return GDN_ERR_DTYPE;
    if (Dk != Dv || (Dk != 64 && Dk != 128) || N < 1 || H < 1) return GDN_ERR_SHAPE;
    if ((long)N * H > INT_MAX) return GDN_ERR_SHAPE;
    if (!q || !k || !v || !beta || !log_alpha || !state || !o) return GDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, beta, log_alpha, state, o};
    for (const void* p : ptrs)
        if (!aligned(p, 16)) return GDN_ERR_ALIGN;
    const size_t esz = dtype == GDN_BF16 ? 2 : 4;
    const size_t S = (size_t)N * H;
    const Range in[] = {rng(q, S * Dk * esz), rng(k, S * Dk * esz), rng(v, S * Dv * esz), rng(beta, S * 4),
                        rng(log_alpha, S * 4)};
    const Range rs = rng(state, S * Dk * Dv * 4), ro = rng(o, S * Dv * esz);
    for (const Range& r : in)
        if (overlap(rs, r) || overlap(ro, r)) return GDN_ERR_ALIAS;
    if (overlap(rs, ro)) return GDN_ERR_ALIAS;
    int st = check_device();
    if (st != GDN_OK) return st;
    return gdn::launch_decode(q, k, v, beta, log_alpha, state, o, (long)S, Dk, dtype,
                              static_cast<hipStream_t>(stream)) == 0
               ? GDN_OK
               : GDN_ERR_LAUNCH;
}

}  // extern "C"
