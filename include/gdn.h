/*
 * gdn.h - C ABI of libgdn.so: causal linear attention in its gated delta-rule form
 * (Gated DeltaNet) and plain causal linear attention, as hand-written HIP for gfx950.
 *
 * The operations (per batch b and head h, state S a Dv x Dk matrix, t = 1..L):
 *
 *   gated delta rule   S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *                      o_t = S_t q_t,  a_t = exp(log_alpha_t).
 *       Gated DeltaNet is the layer the forpes.ru GigaChat linearisation article names among
 *       linear-attention variants (section "Overview") and whose prefill the SparseGDN article
 *       (fileenergy.com) analyses. Its prefill here is chunked exactly as that article's
 *       section "Why GDN prefill is expensive" describes: an intra-chunk delta-system solve, a
 *       sequential pass over chunks for each head, and outputs from each chunk's start state.
 *   plain linear attn  S_t = S_{t-1} + v_t k_t^T, o_t = S_t q_t  (AI RnD Day channel post,
 *       tgstat.ru, section "Linear attention"; the associativity trick of the datadaily.news
 *       overview, section "Linear attention").
 *   decode step        one token of the gated delta rule applied to a stored state in place
 *       (constant work per generated token, AI RnD Day post, section "Linear attention").
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, contiguous row-major, and
 *     16-byte aligned. The library never allocates, frees or synchronises device memory.
 *   - States are stored key-major: element [i][j] of a [Dk][Dv] block is S[j][i].
 *   - Outputs use the state that already contains token t (inclusive causality). No softmax
 *     scale and no normaliser are applied; q and k are used exactly as given.
 *   - dtype (GDN_BF16 or GDN_F32) is the element type of q, k, v and o. beta, log_alpha and
 *     every state are always fp32.
 *   - Launches are asynchronous on `stream` (a hipStream_t passed as void*; NULL = the null
 *     stream). A return of GDN_OK means the work was enqueued. The library never allocates
 *     device memory and uses no stream but the caller's.
 *   - Errors are returned as negative status codes; validation happens before any launch, so
 *     on an error nothing was enqueued and no output was touched.
 *   - Supported sizes: Dk = Dv in {64, 128}; the chunk length is fixed at 64 tokens; any
 *     L >= 0 (a ragged last chunk is handled exactly).
 *   - Concurrent calls on different streams must not share output or workspace buffers.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

enum {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,       /* a required pointer is NULL, or a forbidden one is not */
    GDN_ERR_SHAPE = -2,      /* unsupported B, H, L, N, Dk or Dv */
    GDN_ERR_DTYPE = -3,      /* dtype not GDN_BF16 / GDN_F32 */
    GDN_ERR_ALIGN = -4,      /* a pointer is not 16-byte aligned */
    GDN_ERR_ALIAS = -5,      /* an output overlaps an input or another output */
    GDN_ERR_WORKSPACE = -6,  /* workspace missing or smaller than the size query returned */
    GDN_ERR_LAUNCH = -7,     /* the HIP runtime refused a launch or a device query */
    GDN_ERR_DEVICE = -8,     /* the current device is not a gfx950 GPU */
    GDN_ERR_SCRATCH = -9     /* more static scratch requested than the library holds */
};

/* Human-readable name of a status code (static string, never NULL). */
const char *gdn_status_string(int status);

/* Preferred bytes of device workspace for gdn_prefill_fwd, gdn_prefill_skip_fwd and
 * gdn_prefill_banded_fwd at this shape.
 * The prefill cuts each (batch, head) sequence into NB blocks of whole 64-token chunks. Each
 * block's affine state map (the composition of its chunks' maps S -> A S + B, SparseGDN article,
 * section on embedding the selector into FLA) is formed for all blocks in parallel, a short
 * sequential pass over the blocks gives every block's start state, and the blocks' outputs are
 * then formed in parallel. The workspace holds, per (batch, head), the maps of NB - 1 blocks, NB
 * block-start states and a flag per map (whether its transition is zero):
 * (2 NB - 1) * 4 * Dk * Dv + F bytes, F = 4 (NB - 1) rounded up to a multiple of 256 (F = 0 for
 * NB = 1). The preferred NB gives about two
 * output workgroups per compute unit of the current device (one block, i.e. no workspace, when
 * the (batch, head) slices alone give every compute unit one). Any workspace is accepted, none
 * included: the call uses the largest NB up to the preferred one whose bytes fit, and with no
 * workspace each slice runs its chunks in sequence in one workgroup. Results depend on NB only
 * through rounding. Returns 0 for an unsupported shape or L = 0. */
size_t gdn_prefill_workspace_size(int B, int H, int L, int Dk, int Dv, int dtype);

/* Per-kernel timing of the gated delta-rule prefill, for benchmarks. After
 * gdn_prefill_timing(1), every gdn_prefill_fwd, gdn_prefill_skip_fwd and gdn_prefill_banded_fwd
 * call records a HIP event before and after each of its kernels on the caller's stream, until
 * gdn_prefill_timing(0). gdn_prefill_kernel_times waits for the recorded events, writes the
 * summed milliseconds of the block-map, block-pass and output kernels to ms[0..2] and their
 * launch counts to launches[0..2] (either pointer may be NULL), and clears the record. The
 * events are host objects the library keeps in a pool until the process ends (no device
 * memory). Returns GDN_OK, or GDN_ERR_LAUNCH if an event could not be read (its time then
 * counts as 0). Timing is process-wide state: calls from several host threads share it. */
int gdn_prefill_timing(int enable);
int gdn_prefill_kernel_times(float *ms, int *launches);

/*
 * Chunked prefill of the gated delta rule.
 *   q, k        [B,H,L,Dk] dtype        v, o   [B,H,L,Dv] dtype   (may be NULL when L = 0)
 *   beta        [B,H,L] fp32            log_alpha [B,H,L] fp32 (log of the forget gate, <= 0
 *                                        in normal use; exp(log_alpha) is the gate; -inf is a
 *                                        zero gate, which clears the state before the token's write;
 *                                        a finite log gate below -110 is taken as -110, whose gate,
 *                                        like that of any sum holding it, is exactly 0 in fp32)
 *   h0          [B,H,Dk,Dv] fp32 initial state, or NULL for zeros
 *   h_final     [B,H,Dk,Dv] fp32 final state; may equal h0 (in-place update), any other
 *               overlap is GDN_ERR_ALIAS
 *   workspace   device buffer, 256-byte aligned, or NULL; gdn_prefill_workspace_size(...) bytes
 *               preferred (see above); scratch, reusable once the call's work completes
 * Up to three kernels run in order on `stream` (block maps, the pass over blocks, outputs); the
 * library keeps no state between calls and waits for nothing outside the stream's order.
 * L = 0 copies h0 (or zeros) into h_final. Non-finite inputs other than a log gate of -inf
 * propagate; they are not checked.
 */
int gdn_prefill_fwd(const void *q, const void *k, const void *v,
                    const float *beta, const float *log_alpha, const float *h0,
                    void *o, float *h_final,
                    int B, int H, int L, int Dk, int Dv, int dtype,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Size of the device array that gdn_prefill_fwd_noalloc uses as its workspace (80 MiB). */
#define GDN_PREFILL_NOALLOC_MAX_BYTES ((size_t)80 << 20)

/*
 * gdn_prefill_fwd for callers that cannot allocate device memory: code under HIP graph capture,
 * serving loops that must not call hipMalloc, harnesses that forbid allocation. The arguments and
 * results are those of gdn_prefill_fwd, except that the workspace is the first scratch_bytes
 * bytes of a static array the library holds on each device (GDN_PREFILL_NOALLOC_MAX_BYTES bytes,
 * held from the library's first use on that device until the process ends). scratch_bytes plays
 * the part of workspace_bytes: pass gdn_prefill_workspace_size(...) for the preferred block
 * count, any smaller value (0 included) for fewer blocks. Given the same number of bytes, results
 * are bitwise those of gdn_prefill_fwd with a workspace of that size.
 * A scratch_bytes above GDN_PREFILL_NOALLOC_MAX_BYTES is rejected with GDN_ERR_SCRATCH before
 * anything is enqueued. On a 256-CU MI355X the preferred size of every shape fits (the largest,
 * at D = 128 and B*H = 255, is 79.8 MiB). The call allocates nothing: the first call on a
 * device looks up that device's copy of the array once (hipGetSymbolAddress).
 * Every call on one device shares that device's array and leaves the last call's contents in it;
 * nothing in it needs clearing (each call writes what it reads). Calls on one device whose work
 * can overlap (different streams, or host threads) race on the array: order them on one stream.
 */
int gdn_prefill_fwd_noalloc(const void *q, const void *k, const void *v,
                            const float *beta, const float *log_alpha, const float *h0,
                            void *o, float *h_final, int B, int H, int L, int Dk, int Dv,
                            int dtype, size_t scratch_bytes, void *stream);

/*
 * The gated delta rule with skipped chunk updates (SparseGDN article, fileenergy.com: events the
 * selector drops only decay the state; outputs exist for every token, taken from chunk-start
 * snapshots; its scan_with_skips illustration). Tokens form chunks of 64 (the last one
 * ragged); for chunk c of slice (b, h):
 *   outputs: the gated delta rule run token by token from the chunk-start state;
 *   next chunk-start state: that run's final state if keep[(b*H + h)*ceil(L/64) + c] != 0,
 *                           else the chunk-start state times exp(sum of the chunk's log_alpha).
 *   keep        [B,H,ceil(L/64)] uint8 device array (any alignment; read, never written); NULL
 *               only when L = 0. A head-pair selector is expressed by repeating its mask.
 * All other arguments, the workspace and the stream behaviour as gdn_prefill_fwd. With every
 * keep byte nonzero and the same workspace size the result equals gdn_prefill_fwd's bit for bit.
 * A skipped chunk's state map is a scalar decay, so blocks of skipped chunks cost little in the
 * map stage.
 */
int gdn_prefill_skip_fwd(const void *q, const void *k, const void *v,
                         const float *beta, const float *log_alpha, const unsigned char *keep,
                         const float *h0, void *o, float *h_final,
                         int B, int H, int L, int Dk, int Dv, int dtype,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * The gated delta rule with the block-adjacent intra-chunk solve (SparseGDN article,
 * fileenergy.com, section on two-level sparsity: the delta system inside a chunk is solved only
 * across neighbouring blocks, a fixed structured approximation). Each 64-token chunk's inverse
 * T = (I + A)^-1 is formed in 16 x 16 blocks; blocks more than `band` block rows below the
 * diagonal are set to zero instead of computed (their terms drop out of W and U), the others are
 * the exact inverse's blocks. band in 0 .. 3; band = 3 is gdn_prefill_fwd bit for bit at the
 * same workspace size (other values: GDN_ERR_SHAPE). All other arguments, the workspace and the
 * stream as gdn_prefill_fwd.
 */
int gdn_prefill_banded_fwd(const void *q, const void *k, const void *v,
                           const float *beta, const float *log_alpha, const float *h0,
                           void *o, float *h_final,
                           int B, int H, int L, int Dk, int Dv, int dtype, int band,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Chunked prefill of causal linear attention without the delta term (the forpes.ru article on
 * linear attention, its recurrent form and the decay modifications listed after it):
 *   S_t = a_t S_{t-1} + v_t k_t^T,   o_t = S_t q_t,   a_t = exp(log_alpha_t),
 * i.e. per chunk  O = diag(e^g) Q H0 + (Q K^T masked causally, diagonal included, times
 * e^{g_r - g_s}) V  and  H <- e^{g_C} H0 + (e^{g_C - g} K)^T V  with g the in-chunk prefix
 * sum of log_alpha. log_alpha NULL means a = 1 (plain linear attention, AI RnD Day channel
 * post, tgstat.ru, section "Linear attention"). Log gates must be <= 0; one of -inf (a = 0)
 * clears the state before the token's write, and any log gate below -110 is taken as -110, whose
 * exponential (and that of every sum containing it) is exactly 0 in fp32, so it acts as a = 0
 * too. NaN propagates. Same argument list as gdn_prefill_fwd; beta
 * must be NULL. The scalar transition lets the sequence be split into blocks of chunks whose
 * contributions to the state are summed in parallel; the workspace holds one Dk x Dv fp32
 * state and 4 bytes per block and (batch, head): at least B*H*(Dk*Dv*4 + 4) bytes when L > 0,
 * linattn_prefill_workspace_size(...) preferred (more blocks). Results depend on the block
 * split only through the order of fp32 sums. Runs on `stream` only; L = 0 copies h0 (or zeros)
 * into h_final.
 */
int linattn_prefill_fwd(const void *q, const void *k, const void *v,
                        const float *beta, const float *log_alpha, const float *h0,
                        void *o, float *h_final,
                        int B, int H, int L, int Dk, int Dv, int dtype,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Preferred bytes of device workspace for linattn_prefill_fwd at this shape (blocks of chunks
 * for about 512 workgroups per stage); 0 for an unsupported shape or L = 0. */
size_t linattn_prefill_workspace_size(int B, int H, int L, int Dk, int Dv, int dtype);

/*
 * Gated linear attention with a gate per key dimension (the forpes.ru article's survey of
 * linearised models: GLA, its gating applied over the key vectors):
 *   S_t = S_{t-1} diag(a_t) + v_t k_t^T,   o_t = S_t q_t,   a_t[i] = exp(log_alpha[t][i]),
 * i.e. in the stored key-major state H = S^T, row i decays by a_t[i] before the write.
 *   log_alpha   [B,H,L,Dk] fp32 (required when L > 0), <= 0: any magnitude is supported (every
 *               factor the kernel forms is exp of a non-positive sum); -inf (a = 0) closes the
 *               dimension, and log gates below -110 are taken as -110, which acts the same way
 *               (its exponential is exactly 0 in fp32). NaN propagates.
 * All other arguments as linattn_prefill_fwd; the workspace holds one Dk x Dv fp32 state and a
 * Dk-vector of summed log gates per block and (batch, head): at least B*H*(Dk*Dv*4 + Dk*4) bytes
 * when L > 0, gla_prefill_workspace_size(...) preferred. Runs on `stream` only; L = 0 copies h0
 * (or zeros) into h_final.
 */
int gla_prefill_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                    const float *h0, void *o, float *h_final,
                    int B, int H, int L, int Dk, int Dv, int dtype,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Preferred bytes of device workspace for gla_prefill_fwd at this shape; 0 for an unsupported
 * shape or L = 0. */
size_t gla_prefill_workspace_size(int B, int H, int L, int Dk, int Dv, int dtype);

/*
 * Bidirectional (non-causal) linear attention with a kernel feature map and an optional
 * normaliser (the datadaily.news overview, section "Linear attention", its linear_attention
 * function): per batch b and head h, over the whole sequence,
 *   KV = sum_n phi(k_n) v_n^T  (Dk x Dv),   o_n = KV^T phi(q_n),
 *   and with GDN_BIDIR_NORMALIZE  o_n /= Z_n,  Z_n = phi(q_n) . sum_m phi(k_m).
 *   phi(x) = elu(x) + 1 (x + 1 for x > 0, exp(x) otherwise) with GDN_BIDIR_ELU1, else phi(x) = x
 *   (features already applied by the caller).
 *   q, k        [B,H,L,Dk] dtype        v, o   [B,H,L,Dv] dtype   (may be NULL when L = 0)
 *   kv_out      [B,H,Dk,Dv] fp32 (key-major, element [i][j] = KV[i][j]), or NULL; L = 0 gives zeros
 *   flags       GDN_BIDIR_NORMALIZE | GDN_BIDIR_ELU1 (other bits: GDN_ERR_SHAPE)
 *   workspace   device buffer, 256-byte aligned, at least linattn_bidir_workspace_size(...) bytes
 *               (none needed when L = 0); scratch, reusable once the call's work completes
 * phi is evaluated in fp32 and rounded to dtype before the products; the sums accumulate in
 * fp32 in a fixed order (results are bitwise reproducible). A zero Z gives IEEE inf/NaN
 * outputs, as the division does; positive features (GDN_BIDIR_ELU1) keep Z > 0. Runs on
 * `stream` only.
 */
enum { GDN_BIDIR_NORMALIZE = 1, GDN_BIDIR_ELU1 = 2 };

size_t linattn_bidir_workspace_size(int B, int H, int L, int Dk, int Dv, int dtype);

int linattn_bidir_fwd(const void *q, const void *k, const void *v, void *o, float *kv_out,
                      int B, int H, int L, int Dk, int Dv, int dtype, int flags,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * One recurrent decode step of the gated delta rule for N independent sequences:
 *   q, k [N,H,Dk] dtype;  v, o [N,H,Dv] dtype;  beta, log_alpha [N,H] fp32;
 *   state [N,H,Dk,Dv] fp32, read and overwritten IN PLACE with the state after the token.
 * Each call streams the state from HBM once and writes it back once.
 */
int gdn_decode_step(const void *q, const void *k, const void *v,
                    const float *beta, const float *log_alpha, float *state,
                    void *o, int N, int H, int Dk, int Dv, int dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
