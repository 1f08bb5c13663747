"""An independent fp64 NumPy evaluation of the gated delta rule in chunked (WY) form.

Used only as a pin for the token-by-token oracle: it reaches the same result by a
different algorithm, so agreement to ~1e-12 checks both. It follows the three stages the
SparseGDN article (fileenergy.com, section "Why GDN prefill is expensive") names: an
intra-chunk delta-system solve, a sequential pass over chunks per head, and outputs from
the chunk-start state; the chunk-to-chunk step is the affine map S -> A S + B of that
article's skip-scan illustration (section on embedding the selector into FLA).

Per chunk of n tokens with cumulative log-gate g (restarting at 0 each chunk) and
chunk-start key-major state H0 (Dk x Dv):
    A[r,s] = beta_r exp(g_r - g_s) k_r.k_s  (s < r);   T = (I + A)^-1
    W = T diag(beta exp(g)) K;   Ut = T diag(beta) V;   U = Ut - W H0
    O = diag(exp(g)) Q H0 + P U,  P[r,s] = exp(g_r - g_s) q_r.k_s  (s <= r)
    H_n = exp(g_n) H0 + Khat^T U,  Khat[s] = exp(g_n - g_s) k_s
"""
import numpy as np


def gdn_chunked(q, k, v, beta, log_alpha, h0=None, C=64):
    """q,k [L,Dk]; v [L,Dv]; beta, log_alpha [L]; h0 [Dk,Dv] key-major or None."""
    L, Dk = q.shape
    Dv = v.shape[1]
    H = np.zeros((Dk, Dv)) if h0 is None else np.array(h0, dtype=np.float64)
    o = np.zeros((L, Dv))
    for c0 in range(0, L, C):
        sl = slice(c0, min(L, c0 + C))
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        n = Q.shape[0]
        g = np.cumsum(log_alpha[sl])
        D = g[:, None] - g[None, :]
        lower = np.tril(np.ones((n, n), dtype=bool))
        Gam = np.where(lower, np.exp(np.where(lower, D, 0.0)), 0.0)
        A = np.tril(b[:, None] * (K @ K.T) * Gam, -1)
        T = np.linalg.inv(np.eye(n) + A)
        W = T @ ((b * np.exp(g))[:, None] * K)
        Ut = T @ (b[:, None] * V)
        U = Ut - W @ H
        P = (Q @ K.T) * Gam
        o[sl] = np.exp(g)[:, None] * (Q @ H) + P @ U
        Khat = np.exp(g[-1] - g)[:, None] * K
        H = np.exp(g[-1]) * H + Khat.T @ U
    return o, H


def linattn_chunked(q, k, v, h0=None, C=64):
    """Plain causal linear attention, chunked: O = Q H0 + (Q K^T masked) V, H += K^T V."""
    L, Dk = q.shape
    Dv = v.shape[1]
    H = np.zeros((Dk, Dv)) if h0 is None else np.array(h0, dtype=np.float64)
    o = np.zeros((L, Dv))
    for c0 in range(0, L, C):
        sl = slice(c0, min(L, c0 + C))
        Q, K, V = q[sl], k[sl], v[sl]
        o[sl] = Q @ H + np.tril(Q @ K.T) @ V
        H = H + K.T @ V
    return o, H
