// Kernel launchers behind the C ABI (internal to libgdn; arguments are validated by the caller).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gdn {

int launch_decode(const void* q, const void* k, const void* v, const float* beta, const float* log_alpha,
                  float* state, void* o, long slices, int D, int dtype, hipStream_t stream);

size_t prefill_workspace_bytes(long BH, long L, int D, int dtype);      // preferred
size_t prefill_workspace_min_bytes(long BH, long L, int D, int dtype);  // smallest accepted

// keep: [BH][ceil(L/64)] chunk keep mask (nonzero = apply the chunk's state update), or NULL (all)
// band: 16 x 16 blocks of the intra-chunk inverse kept below its diagonal, 0 .. 3 (3 = exact)
// L = 0 copies h0 (or zeros) to h_final.
int launch_prefill(const void* q, const void* k, const void* v, const float* beta, const float* log_alpha,
                   const unsigned char* keep, const float* h0, void* o, float* h_final, int BH, long L, int D,
                   int dtype, int band, void* ws, size_t ws_bytes, hipStream_t stream);

// Device address of the current device's copy of the static prefill scratch
// (GDN_PREFILL_NOALLOC_MAX_BYTES bytes), looked up once per device; 0 or -1.
int prefill_scratch(void** ptr);

// Per-kernel timing of launch_prefill: when on, HIP events bracket each launch on its stream.
// prefill_kernel_times waits for them and returns summed ms and launch counts per stage (block
// maps, pass over blocks, outputs), then clears the record.
void prefill_timing(bool enable);
int prefill_kernel_times(float* ms, int* launches);

// Causal linear attention, plain (log_alpha NULL) or with a per-token decay, block-parallel.
// The workspace holds each block's state tiles (one block per slice at the minimum; a smaller
// workspace means fewer, longer blocks).
size_t linattn_workspace_bytes(long BH, long L, int D);      // preferred
size_t linattn_workspace_min_bytes(long BH, long L, int D);  // smallest accepted
int launch_linattn(const void* q, const void* k, const void* v, const float* log_alpha, const float* h0, void* o,
                   float* h_final, int BH, long L, int D, int dtype, void* ws, size_t ws_bytes, hipStream_t stream);

// Gated linear attention with a gate per key dimension: log_alpha [BH][L][D]; same workspace
// scheme with a D-vector of summed log gates per block.
size_t gla_workspace_bytes(long BH, long L, int D);
size_t gla_workspace_min_bytes(long BH, long L, int D);
int launch_gla(const void* q, const void* k, const void* v, const float* log_alpha, const float* h0, void* o,
               float* h_final, int BH, long L, int D, int dtype, void* ws, size_t ws_bytes, hipStream_t stream);

// Bidirectional linear attention. kv_out: [BH][D][D] fp32 or NULL. flags bit 0: divide by Z,
// bit 1: phi = elu + 1 (else identity). The workspace is bidir_workspace_bytes(...) bytes.
size_t bidir_workspace_bytes(long BH, long L, int D, int dtype);
int launch_bidir(const void* q, const void* k, const void* v, void* o, float* kv_out, int BH, long L, int D,
                 int dtype, int flags, void* ws, hipStream_t stream);

}  // namespace gdn
