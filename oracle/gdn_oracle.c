/*
 * fp64 CPU oracle for causal linear attention in its gated delta-rule form (Gated DeltaNet)
 * and for plain causal linear attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library. It shares no code, header, table or helper with the HIP library;
 * the product path never calls it.
 *
 * What it computes (per batch b and head h independently, token by token, in fp64):
 *
 *   Gated delta rule. The state S is a Dv x Dk matrix (math orientation, S[j][i]).
 *       S_t = a_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   a_t = exp(log_alpha_t)
 *       o_t = S_t q_t
 *   written out with the rank-1 product expanded, as the code below does:
 *       s = S_{t-1} k_t;  S_t = a_t (S_{t-1} - beta_t s k_t^T) + beta_t v_t k_t^T.
 *   The forget gate a_t multiplies the decayed old state only, not the new write.
 *
 *   Plain causal linear attention (the alpha = 1 case with no delta term), the update printed
 *   in the AI RnD Day channel post (tgstat.ru, section "Linear attention"):
 *       S_t = S_{t-1} + v_t k_t^T,   o_t = S_t q_t.
 *   The output uses the state that already contains token t (inclusive causality) and no
 *   softmax scale or normaliser is applied.
 *
 *   Decay-only gated linear attention (linear attention with a per-token decay, one of the
 *   modifications the forpes.ru article on linear attention lists after the recurrent form):
 *       S_t = a_t S_{t-1} + v_t k_t^T,   o_t = S_t q_t,   a_t = exp(log_alpha_t).
 *
 *   Gated linear attention with a gate per key dimension (the forpes.ru article's survey of
 *   linearised models: GLA, its gating applied over the key vectors):
 *       S_t = S_{t-1} diag(a_t) + v_t k_t^T,   o_t = S_t q_t,   a_t[i] = exp(log_alpha_t[i]),
 *   i.e. key dimension i of the state decays by its own factor a_t[i] before the write.
 *
 *   Gated delta rule with skipped chunk updates (the SparseGDN article, fileenergy.com: the
 *   selector's skipped events, and its scan_with_skips illustration in the section on embedding
 *   the selector into an FLA pipeline). Tokens are grouped into chunks of C; at the start of
 *   chunk c the state S_c is the chunk's snapshot. Every token's output is the gated delta rule
 *   run token by token from the snapshot through the chunk (outputs exist for every token,
 *   skipped chunk or not). The state carried to the next chunk is the result of that run when
 *   keep[c] != 0, and otherwise the snapshot only decayed: exp(sum of the chunk's log_alpha) S_c.
 *
 *   Decode step: the gated delta-rule update above applied once to a stored state.
 *
 *   Bidirectional (non-causal) linear attention, the kernel-feature-map form of the datadaily.news
 *   overview (section "Linear attention", its linear_attention function): every token sees the
 *   whole sequence,
 *       KV = sum_n phi(k_n) v_n^T (Dk x Dv),  out_n = KV^T phi(q_n),
 *       Z_n = phi(q_n) . sum_m phi(k_m),      out_n / Z_n when normalising,
 *   with phi the identity or elu(x) + 1 (x for x > 0, exp(x) otherwise).
 *
 * Storage orientation. Initial, final and decode states are stored key-major: element
 * [i][j] of a [Dk][Dv] block equals S[j][i]. This matches the chunk-level map S -> A S + B of
 * the SparseGDN article's skip-scan illustration (fileenergy.com, section on embedding the
 * selector into an FLA pipeline), with the state's key dimension as the row index.
 *
 * Layouts (all row-major, fp64):
 *   q, k [B,H,L,Dk]; v, o [B,H,L,Dv]; beta, log_alpha [B,H,L]; h0, h_final [B,H,Dk,Dv];
 *   the per-key-dimension log_alpha of gated linear attention [B,H,L,Dk].
 *   h0 == NULL means a zero initial state.
 * nthreads <= 0 uses the OpenMP default. Returns the number of threads used.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* S (Dv x Dk) <- key-major block X (Dk x Dv), or zeros. */
static void load_state(double *S, const double *X, int Dk, int Dv)
{
    for (int j = 0; j < Dv; ++j)
        for (int i = 0; i < Dk; ++i)
            S[(size_t)j * Dk + i] = X ? X[(size_t)i * Dv + j] : 0.0;
}

static void store_state(double *X, const double *S, int Dk, int Dv)
{
    for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j)
            X[(size_t)i * Dv + j] = S[(size_t)j * Dk + i];
}

/* o = S q */
static void read_out(double *o, const double *S, const double *q, int Dk, int Dv)
{
    for (int j = 0; j < Dv; ++j) {
        double acc = 0.0;
        const double *row = S + (size_t)j * Dk;
        for (int i = 0; i < Dk; ++i) acc += row[i] * q[i];
        o[j] = acc;
    }
}

/* One gated delta-rule token: S <- a (S - beta (S k) k^T) + beta v k^T. `sk` is scratch (Dv). */
static void gdn_token(double *S, double *sk, const double *k, const double *v,
                      double beta, double log_alpha, int Dk, int Dv)
{
    const double a = exp(log_alpha);
    for (int j = 0; j < Dv; ++j) {
        double acc = 0.0;
        const double *row = S + (size_t)j * Dk;
        for (int i = 0; i < Dk; ++i) acc += row[i] * k[i];
        sk[j] = acc;
    }
    for (int j = 0; j < Dv; ++j) {
        double *row = S + (size_t)j * Dk;
        const double dj = beta * sk[j];
        const double wj = beta * v[j];
        for (int i = 0; i < Dk; ++i) row[i] = a * (row[i] - dj * k[i]) + wj * k[i];
    }
}

/* One decay-only gated linear-attention token: S <- a S + v k^T. */
static void gla_token(double *S, const double *k, const double *v, double log_alpha, int Dk, int Dv)
{
    const double a = exp(log_alpha);
    for (int j = 0; j < Dv; ++j) {
        double *row = S + (size_t)j * Dk;
        for (int i = 0; i < Dk; ++i) row[i] = a * row[i] + v[j] * k[i];
    }
}

/* One gated linear-attention token, a gate per key dimension: S[j][i] <- a[i] S[j][i] + v[j] k[i]. */
static void gla_vec_token(double *S, double *a, const double *k, const double *v, const double *log_alpha,
                          int Dk, int Dv)
{
    for (int i = 0; i < Dk; ++i) a[i] = exp(log_alpha[i]);
    for (int j = 0; j < Dv; ++j) {
        double *row = S + (size_t)j * Dk;
        for (int i = 0; i < Dk; ++i) row[i] = a[i] * row[i] + v[j] * k[i];
    }
}

/* One plain linear-attention token: S <- S + v k^T. */
static void la_token(double *S, const double *k, const double *v, int Dk, int Dv)
{
    for (int j = 0; j < Dv; ++j) {
        double *row = S + (size_t)j * Dk;
        for (int i = 0; i < Dk; ++i) row[i] += v[j] * k[i];
    }
}

int oracle_gdn_prefill(const double *q, const double *k, const double *v,
                       const double *beta, const double *log_alpha, const double *h0,
                       double *o, double *h_final,
                       int B, int H, int L, int Dk, int Dv, int nthreads)
{
    const int used = set_threads(nthreads);
    const long nslice = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long s = 0; s < nslice; ++s) {
        double *S = (double *)malloc(sizeof(double) * ((size_t)Dk * Dv + Dv));
        double *sk = S + (size_t)Dk * Dv;
        load_state(S, h0 ? h0 + (size_t)s * Dk * Dv : NULL, Dk, Dv);
        for (int t = 0; t < L; ++t) {
            const size_t tok = (size_t)s * L + t;
            gdn_token(S, sk, k + tok * Dk, v + tok * Dv, beta[tok], log_alpha[tok], Dk, Dv);
            read_out(o + tok * Dv, S, q + tok * Dk, Dk, Dv);
        }
        store_state(h_final + (size_t)s * Dk * Dv, S, Dk, Dv);
        free(S);
    }
    return used;
}

int oracle_linattn_prefill(const double *q, const double *k, const double *v, const double *h0,
                           double *o, double *h_final,
                           int B, int H, int L, int Dk, int Dv, int nthreads)
{
    const int used = set_threads(nthreads);
    const long nslice = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long s = 0; s < nslice; ++s) {
        double *S = (double *)malloc(sizeof(double) * (size_t)Dk * Dv);
        load_state(S, h0 ? h0 + (size_t)s * Dk * Dv : NULL, Dk, Dv);
        for (int t = 0; t < L; ++t) {
            const size_t tok = (size_t)s * L + t;
            la_token(S, k + tok * Dk, v + tok * Dv, Dk, Dv);
            read_out(o + tok * Dv, S, q + tok * Dk, Dk, Dv);
        }
        store_state(h_final + (size_t)s * Dk * Dv, S, Dk, Dv);
        free(S);
    }
    return used;
}

/* Decay-only gated linear attention: as oracle_linattn_prefill, with log_alpha [B,H,L]. */
int oracle_gla_prefill(const double *q, const double *k, const double *v, const double *log_alpha,
                       const double *h0, double *o, double *h_final,
                       int B, int H, int L, int Dk, int Dv, int nthreads)
{
    const int used = set_threads(nthreads);
    const long nslice = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long s = 0; s < nslice; ++s) {
        double *S = (double *)malloc(sizeof(double) * (size_t)Dk * Dv);
        load_state(S, h0 ? h0 + (size_t)s * Dk * Dv : NULL, Dk, Dv);
        for (int t = 0; t < L; ++t) {
            const size_t tok = (size_t)s * L + t;
            gla_token(S, k + tok * Dk, v + tok * Dv, log_alpha[tok], Dk, Dv);
            read_out(o + tok * Dv, S, q + tok * Dk, Dk, Dv);
        }
        store_state(h_final + (size_t)s * Dk * Dv, S, Dk, Dv);
        free(S);
    }
    return used;
}

/* Gated linear attention with a gate per key dimension: log_alpha [B,H,L,Dk]; the rest as
 * oracle_linattn_prefill. */
int oracle_gla_vec_prefill(const double *q, const double *k, const double *v, const double *log_alpha,
                           const double *h0, double *o, double *h_final,
                           int B, int H, int L, int Dk, int Dv, int nthreads)
{
    const int used = set_threads(nthreads);
    const long nslice = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long s = 0; s < nslice; ++s) {
        double *S = (double *)malloc(sizeof(double) * ((size_t)Dk * Dv + Dk));
        double *a = S + (size_t)Dk * Dv;
        load_state(S, h0 ? h0 + (size_t)s * Dk * Dv : NULL, Dk, Dv);
        for (int t = 0; t < L; ++t) {
            const size_t tok = (size_t)s * L + t;
            gla_vec_token(S, a, k + tok * Dk, v + tok * Dv, log_alpha + tok * Dk, Dk, Dv);
            read_out(o + tok * Dv, S, q + tok * Dk, Dk, Dv);
        }
        store_state(h_final + (size_t)s * Dk * Dv, S, Dk, Dv);
        free(S);
    }
    return used;
}

/* Gated delta rule with skipped chunk updates. keep [B,H,ceil(L/C)] (nonzero = keep); the rest as
 * oracle_gdn_prefill. */
int oracle_gdn_prefill_skip(const double *q, const double *k, const double *v,
                            const double *beta, const double *log_alpha, const double *h0,
                            const int *keep, int C, double *o, double *h_final,
                            int B, int H, int L, int Dk, int Dv, int nthreads)
{
    const int used = set_threads(nthreads);
    const long nslice = (long)B * H;
    const int nch = (L + C - 1) / C;
#pragma omp parallel for schedule(dynamic, 1)
    for (long s = 0; s < nslice; ++s) {
        double *S = (double *)malloc(sizeof(double) * ((size_t)2 * Dk * Dv + Dv));
        double *snap = S + (size_t)Dk * Dv;
        double *sk = snap + (size_t)Dk * Dv;
        load_state(S, h0 ? h0 + (size_t)s * Dk * Dv : NULL, Dk, Dv);
        for (int c = 0; c < nch; ++c) {
            memcpy(snap, S, sizeof(double) * (size_t)Dk * Dv);
            double gsum = 0.0;
            for (int t = c * C; t < L && t < (c + 1) * C; ++t) {
                const size_t tok = (size_t)s * L + t;
                gdn_token(S, sk, k + tok * Dk, v + tok * Dv, beta[tok], log_alpha[tok], Dk, Dv);
                read_out(o + tok * Dv, S, q + tok * Dk, Dk, Dv);
                gsum += log_alpha[tok];
            }
            if (!keep[(size_t)s * nch + c]) {
                const double d = exp(gsum);
                for (size_t e = 0; e < (size_t)Dk * Dv; ++e) S[e] = d * snap[e];
            }
        }
        store_state(h_final + (size_t)s * Dk * Dv, S, Dk, Dv);
        free(S);
    }
    return used;
}

/* Decode: q,k [N,H,Dk]; v, o [N,H,Dv]; beta, log_alpha [N,H]; state [N,H,Dk,Dv] updated in place. */
int oracle_gdn_decode_step(const double *q, const double *k, const double *v,
                           const double *beta, const double *log_alpha, double *state,
                           double *o, int N, int H, int Dk, int Dv, int nthreads)
{
    const int used = set_threads(nthreads);
    const long nslice = (long)N * H;
#pragma omp parallel for schedule(static)
    for (long s = 0; s < nslice; ++s) {
        double *S = (double *)malloc(sizeof(double) * ((size_t)Dk * Dv + Dv));
        double *sk = S + (size_t)Dk * Dv;
        double *st = state + (size_t)s * Dk * Dv;
        load_state(S, st, Dk, Dv);
        gdn_token(S, sk, k + (size_t)s * Dk, v + (size_t)s * Dv, beta[s], log_alpha[s], Dk, Dv);
        read_out(o + (size_t)s * Dv, S, q + (size_t)s * Dk, Dk, Dv);
        store_state(st, S, Dk, Dv);
        free(S);
    }
    return used;
}

/* phi(x) = elu(x) + 1 when elu1, else x. */
static double feature(double x, int elu1)
{
    if (!elu1) return x;
    return x > 0.0 ? x + 1.0 : exp(x);
}

/* Bidirectional linear attention. flags bit 0: divide by Z; bit 1: phi = elu + 1 (else identity).
 * q, k [B,H,L,Dk]; v, o [B,H,L,Dv]; kv [B,H,Dk,Dv] (KV, key-major, may be NULL). */
int oracle_linattn_bidir(const double *q, const double *k, const double *v, double *o, double *kv,
                         int B, int H, int L, int Dk, int Dv, int flags, int nthreads)
{
    const int used = set_threads(nthreads);
    const long nslice = (long)B * H;
    const int norm = flags & 1, elu1 = (flags >> 1) & 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (long s = 0; s < nslice; ++s) {
        double *KV = (double *)calloc((size_t)Dk * Dv + Dk + Dk, sizeof(double));
        double *ksum = KV + (size_t)Dk * Dv;
        double *fq = ksum + Dk;
        /* KV = sum_n phi(k_n) v_n^T and the key sum, over the whole sequence */
        for (int t = 0; t < L; ++t) {
            const double *kt = k + ((size_t)s * L + t) * Dk;
            const double *vt = v + ((size_t)s * L + t) * Dv;
            for (int i = 0; i < Dk; ++i) {
                const double fk = feature(kt[i], elu1);
                ksum[i] += fk;
                for (int j = 0; j < Dv; ++j) KV[(size_t)i * Dv + j] += fk * vt[j];
            }
        }
        /* out_n = KV^T phi(q_n), then / Z_n */
        for (int t = 0; t < L; ++t) {
            const double *qt = q + ((size_t)s * L + t) * Dk;
            double *ot = o + ((size_t)s * L + t) * Dv;
            double z = 0.0;
            for (int i = 0; i < Dk; ++i) {
                fq[i] = feature(qt[i], elu1);
                z += fq[i] * ksum[i];
            }
            for (int j = 0; j < Dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < Dk; ++i) acc += fq[i] * KV[(size_t)i * Dv + j];
                ot[j] = norm ? acc / z : acc;
            }
        }
        if (kv) memcpy(kv + (size_t)s * Dk * Dv, KV, sizeof(double) * (size_t)Dk * Dv);
        free(KV);
    }
    return used;
}
