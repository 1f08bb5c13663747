"""Pins for the oracle's chunked form with the block-adjacent intra-chunk solve (CPU only).

The chunked form (oracle/banded.py) is pinned to the token-by-token recurrence (the C oracle)
when the band keeps every block, and wherever the approximation is exact by construction: a
chunk inside one 16-token block, chunks of at most 32 tokens with band >= 1, beta = 0 (no delta
system). The band itself is pinned to the block structure of a triangular inverse: the kept
diagonal blocks are the inverses of the diagonal blocks of I + A, the first sub-diagonal block
is -T_ii A_i,i-1 T_i-1,i-1, and the rest are zero. Every band on general inputs is pinned to a
second formulation that never forms T: windows of the token recurrence (see
_windowed_chunk_form).
"""
import numpy as np
import pytest

import oracle
from oracle.banded import chunk_inverse


def _inputs(seed, B, H, L, D, long_memory=True):
    r = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q, k = unit(r.standard_normal((B, H, L, D))), unit(r.standard_normal((B, H, L, D)))
    v = r.standard_normal((B, H, L, D))
    beta = 1 / (1 + np.exp(-r.standard_normal((B, H, L))))
    la = -r.uniform(0, 0.05, (B, H, L)) if long_memory else -np.log1p(np.exp(r.standard_normal((B, H, L)) + 2))
    h0 = 0.1 * r.standard_normal((B, H, D, D))
    return q, k, v, beta, la, h0


@pytest.mark.parametrize("L", [1, 17, 64, 65, 200])
def test_full_band_is_the_recurrence(L):
    q, k, v, beta, la, h0 = _inputs(L, 2, 2, L, 16)
    o, hf = oracle.gdn_prefill_banded(q, k, v, beta, la, h0, band=3)
    ro, rh = oracle.gdn_prefill(q, k, v, beta, la, h0)
    np.testing.assert_allclose(o, ro, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(hf, rh, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("band", [0, 1, 2])
def test_exact_where_no_block_is_dropped(band):
    # one block per chunk (chunk of 16 tokens): every band is exact
    q, k, v, beta, la, h0 = _inputs(3, 1, 2, 80, 8)
    o, hf = oracle.gdn_prefill_banded(q, k, v, beta, la, h0, band=band, chunk=16)
    ro, rh = oracle.gdn_prefill(q, k, v, beta, la, h0)
    np.testing.assert_allclose(o, ro, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(hf, rh, rtol=1e-10, atol=1e-12)
    # beta = 0: no delta system at all
    z = np.zeros_like(beta)
    o, hf = oracle.gdn_prefill_banded(q, k, v, z, la, h0, band=band)
    ro, rh = oracle.gdn_prefill(q, k, v, z, la, h0)
    np.testing.assert_allclose(o, ro, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(hf, rh, rtol=1e-10, atol=1e-12)


def test_two_blocks_band_one_is_exact():
    q, k, v, beta, la, h0 = _inputs(4, 1, 2, 32, 8)
    o, hf = oracle.gdn_prefill_banded(q, k, v, beta, la, h0, band=1)
    ro, rh = oracle.gdn_prefill(q, k, v, beta, la, h0)
    np.testing.assert_allclose(o, ro, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(hf, rh, rtol=1e-10, atol=1e-12)


def test_banded_inverse_block_structure():
    r = np.random.default_rng(7)
    k = r.standard_normal((64, 16)) / 4
    beta = r.uniform(0.2, 0.9, 64)
    g = np.cumsum(-r.uniform(0, 0.05, 64))
    T3, A = chunk_inverse(k, beta, g, band=3)
    np.testing.assert_allclose(T3 @ (np.eye(64) + A), np.eye(64), atol=1e-12)
    blk = lambda M, i, j: M[16 * i:16 * i + 16, 16 * j:16 * j + 16]
    for band in (0, 1, 2):
        T, _ = chunk_inverse(k, beta, g, band=band)
        for i in range(4):
            Tii = np.linalg.inv(np.eye(16) + blk(A, i, i))
            np.testing.assert_allclose(blk(T, i, i), Tii, rtol=1e-12, atol=1e-14)
            for j in range(4):
                if j > i or i - j > band:
                    assert not blk(T, i, j).any()
                elif i - j == 1:
                    ref = -Tii @ blk(A, i, j) @ np.linalg.inv(np.eye(16) + blk(A, j, j))
                    np.testing.assert_allclose(blk(T, i, j), ref, rtol=1e-10, atol=1e-14)
                else:
                    np.testing.assert_array_equal(blk(T, i, j), blk(T3, i, j))


def test_band_is_an_approximation_with_long_memory():
    """Dropping blocks changes the result when keys interact across blocks (no pin for the value)."""
    q, k, v, beta, la, h0 = _inputs(9, 1, 1, 128, 16)
    o0, _ = oracle.gdn_prefill_banded(q, k, v, beta, la, h0, band=0)
    o3, _ = oracle.gdn_prefill_banded(q, k, v, beta, la, h0, band=3)
    assert np.abs(o0 - o3).max() > 1e-3 * np.abs(o3).max()


def _windowed_chunk_form(q, k, v, beta, la, h0, band, chunk=64, block=16):
    """The block-adjacent solve restated through the token recurrence, for one (b, h) slice.

    T = (I + A)^-1 is lower triangular, so any contiguous run of its diagonal blocks is the
    inverse of the same run of I + A. Keeping T's blocks (i, i - band) .. (i, i) therefore makes
    the pseudo-values u of block i those of the exact delta rule run over blocks i - band .. i
    alone, started from the chunk-start state decayed to the window's start. Here that run is the
    C oracle's decode step, token by token, and u_r is read back from two successive states
    (S_r - a_r S_{r-1} = k_r u_r^T). The chunk's outputs and next state are then the plain sums
        o_r = e^{g_r} H^T q_r + sum_{s <= r} e^{g_r - g_s} (q_r . k_s) u_s
        H'  = e^{g_C} H + sum_s e^{g_C - g_s} k_s u_s^T.
    """
    L, D = k.shape
    H = np.array(h0, dtype=np.float64)
    o = np.zeros((L, v.shape[1]))
    one = lambda x: np.asarray(x, dtype=np.float64).reshape(1, 1, -1)
    for t0 in range(0, L, chunk):
        n = min(chunk, L - t0)
        g = np.cumsum(la[t0:t0 + n])
        u = np.zeros((n, v.shape[1]))
        for i0 in range(0, n, block):
            w0 = max(0, i0 - band * block)
            S = (np.exp(g[w0 - 1]) if w0 > 0 else 1.0) * H
            for r in range(w0, min(n, i0 + block)):
                t = t0 + r
                _, S1 = oracle.gdn_decode_step(one(q[t]), one(k[t]), one(v[t]), np.full((1, 1), beta[t]),
                                               np.full((1, 1), la[t]), S[None, None])
                S1 = S1[0, 0]
                if r >= i0:
                    u[r] = (S1 - np.exp(la[t]) * S).T @ k[t] / (k[t] @ k[t])
                S = S1
        for r in range(n):
            acc = np.exp(g[r]) * (H.T @ q[t0 + r])
            for s in range(r + 1):
                acc = acc + np.exp(g[r] - g[s]) * (q[t0 + r] @ k[t0 + s]) * u[s]
            o[t0 + r] = acc
        Hn = np.exp(g[-1]) * H
        for s in range(n):
            Hn = Hn + np.exp(g[-1] - g[s]) * np.outer(k[t0 + s], u[s])
        H = Hn
    return o, H


@pytest.mark.parametrize("band", [0, 1, 2, 3])
@pytest.mark.parametrize("L,long_memory", [(64, True), (150, True), (200, False)])
def test_band_equals_windowed_recurrence(band, L, long_memory):
    """Every band on general inputs (unit keys that interact across blocks, h0 != 0, ragged
    tails): the oracle's banded chunked form against the windowed token recurrence above."""
    q, k, v, beta, la, h0 = _inputs(100 + L + band, 1, 2, L, 8, long_memory)
    o, hf = oracle.gdn_prefill_banded(q, k, v, beta, la, h0, band=band)
    for h in range(2):
        ro, rh = _windowed_chunk_form(q[0, h], k[0, h], v[0, h], beta[0, h], la[0, h], h0[0, h], band)
        np.testing.assert_allclose(o[0, h], ro, rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(hf[0, h], rh, rtol=1e-9, atol=1e-11)
    if band == 3:   # the window of the full band is the whole chunk: the plain recurrence
        ro, rh = oracle.gdn_prefill(q, k, v, beta, la, h0)
        np.testing.assert_allclose(o, ro, rtol=1e-10, atol=1e-12)
