"""fp64 chunked form of the gated delta rule with the block-adjacent intra-chunk solve
(test infrastructure only; see the package docstring for who may use it).

The SparseGDN article (fileenergy.com, section on its two-level sparsity) cuts the intra-chunk
delta-system solve down to the couplings between neighbouring blocks, a fixed structured
approximation. The plainest reading, taken here: the chunk's inverse T = (I + A)^-1 is formed
in 16 x 16 blocks and its blocks more than `band` block rows below the diagonal are replaced by
zero; the rest are the exact inverse's blocks. band = 3 (C = 64) keeps everything and is the
exact rule.

Steps per head and chunk (the chunked WY form; H is the key-major state, H = S^T, Dk x Dv):
    g = inclusive prefix sum of log_alpha over the chunk, gC its last value
    A[r, s] = beta_r exp(g_r - g_s) k_r . k_s for s < r (else 0);  T = (I + A)^-1, then banded
    W = T diag(beta e^g) K;   U~ = T diag(beta) V;   U = U~ - W H
    O = diag(e^g) Q H + ((Q K^T) masked to s <= r, times exp(g_r - g_s)) U
    H <- e^gC H + (diag(e^(gC - g)) K)^T U
The matrix inverse and products are NumPy's (fp64); nothing is fused or reordered.
"""
from __future__ import annotations

import numpy as np


def band_mask(n: int, band: int, block: int = 16) -> np.ndarray:
    """True where block row minus block column lies in [0, band] (the kept part, lower side)."""
    bi = np.arange(n)[:, None] // block
    bj = np.arange(n)[None, :] // block
    return (bi - bj >= 0) & (bi - bj <= band)


def chunk_inverse(k, beta, g, band: int = 3, block: int = 16):
    """T = (I + A)^-1 of one chunk with blocks beyond `band` below the diagonal set to zero."""
    n = len(beta)
    gamma = np.exp(np.minimum(g[:, None] - g[None, :], 0.0))   # only s <= r is kept below (exponent <= 0)
    A = np.tril(beta[:, None] * gamma * (k @ k.T), -1)
    T = np.linalg.inv(np.eye(n) + A)
    return np.where(band_mask(n, band, block), T, 0.0), A


def gdn_prefill_banded(q, k, v, beta, log_alpha, h0=None, band: int = 3, chunk: int = 64, block: int = 16):
    """q, k [B,H,L,Dk]; v [B,H,L,Dv]; beta, log_alpha [B,H,L]; h0 [B,H,Dk,Dv] (key-major) or None.
    Returns (o [B,H,L,Dv], h_final [B,H,Dk,Dv]) in fp64."""
    q, k, v, beta, log_alpha = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta, log_alpha))
    B, Hh, L, Dk = q.shape
    Dv = v.shape[-1]
    o = np.zeros((B, Hh, L, Dv))
    hf = np.zeros((B, Hh, Dk, Dv))
    for b in range(B):
        for h in range(Hh):
            H = np.zeros((Dk, Dv)) if h0 is None else np.array(h0[b, h], dtype=np.float64)
            for t0 in range(0, L, chunk):
                sl = slice(t0, min(L, t0 + chunk))
                qc, kc, vc, bc = q[b, h, sl], k[b, h, sl], v[b, h, sl], beta[b, h, sl]
                g = np.cumsum(log_alpha[b, h, sl])
                T, _ = chunk_inverse(kc, bc, g, band, block)
                W = T @ ((bc * np.exp(g))[:, None] * kc)
                U = T @ (bc[:, None] * vc) - W @ H
                P = np.tril(qc @ kc.T) * np.tril(np.exp(np.minimum(g[:, None] - g[None, :], 0.0)))
                o[b, h, sl] = np.exp(g)[:, None] * (qc @ H) + P @ U
                H = np.exp(g[-1]) * H + (np.exp(g[-1] - g)[:, None] * kc).T @ U
            hf[b, h] = H
    return o, hf
