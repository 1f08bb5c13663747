"""Pins for the oracle's gated linear attention with a gate per key dimension (CPU only):

    S_t = S_{t-1} diag(a_t) + v_t k_t^T,  o_t = S_t q_t,  a_t[i] = exp(log_alpha_t[i])

(the forpes.ru article's survey of linearised models: GLA, its gating applied over the key
vectors). Each pin uses code written independently of the oracle: the unrolled closed form in
NumPy, exact rational brute force with explicit matrices, and special cases that reduce to other
forms.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _frac_mat(r, c, gen):
    return [[Fraction(int(gen.integers(-4, 5)), 4) for _ in range(c)] for _ in range(r)]


def _f(m):
    return np.array([[float(x) for x in row] for row in m])


@pytest.mark.parametrize("L,Dk,Dv", [(1, 8, 8), (37, 16, 8), (150, 24, 40)])
def test_gla_vec_equals_unrolled_form(L, Dk, Dv):
    """With G_t = sum_{s<=t} log a_s (a vector per token), unrolling the recurrence gives
        o_t = sum_{s<=t} (sum_i q_t[i] k_s[i] exp(G_t[i] - G_s[i])) v_s + sum_i q_t[i] exp(G_t[i]) h0[i, :]
        h_L[i, :] = exp(G_L[i]) h0[i, :] + sum_s exp(G_L[i] - G_s[i]) k_s[i] v_s."""
    r = np.random.default_rng(L + 300)
    q, k = r.standard_normal((L, Dk)), r.standard_normal((L, Dk))
    v, h0 = r.standard_normal((L, Dv)), r.standard_normal((Dk, Dv))
    la = -r.uniform(0.0, 0.4, (L, Dk))
    o, hf = oracle.gla_vec_prefill(q, k, v, la, h0)
    G = np.cumsum(la, axis=0)                                        # [L, Dk]
    decay = np.exp(G[:, None, :] - G[None, :, :])                     # [t, s, i]
    scores = np.einsum("ti,si,tsi->ts", q, k, decay) * np.tril(np.ones((L, L)))
    ref = scores @ v + (q * np.exp(G)) @ h0
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-11, atol=1e-11)
    ref_h = np.exp(G[-1])[:, None] * h0 + (k * np.exp(G[-1][None, :] - G)).T @ v
    np.testing.assert_allclose(hf[0, 0], ref_h, rtol=1e-11, atol=1e-11)


def test_gla_vec_exact_rational_bruteforce():
    """Explicit Dv x Dk matrices in Fractions: S <- S diag(a_t) + v_t k_t^T, Dk != Dv, h0 != 0."""
    gen = np.random.default_rng(23)
    Dk, Dv, L = 3, 2, 5
    q, k, v = _frac_mat(L, Dk, gen), _frac_mat(L, Dk, gen), _frac_mat(L, Dv, gen)
    alpha = [[Fraction(int(gen.integers(1, 8)), 8) for _ in range(Dk)] for _ in range(L)]
    h0 = _frac_mat(Dk, Dv, gen)
    S = [[h0[i][j] for i in range(Dk)] for j in range(Dv)]
    o_exact = []
    for t in range(L):
        S = [[S[rr][c] * alpha[t][c] + v[t][rr] * k[t][c] for c in range(Dk)] for rr in range(Dv)]
        o_exact.append([sum(S[rr][c] * q[t][c] for c in range(Dk)) for rr in range(Dv)])
    la = np.log(_f(alpha))
    o, hf = oracle.gla_vec_prefill(_f(q), _f(k), _f(v), la, _f(h0))
    np.testing.assert_allclose(o[0, 0], _f(o_exact), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hf[0, 0], _f(S).T, rtol=1e-12, atol=1e-12)


def test_gla_vec_equal_gates_is_scalar_gated():
    """The same gate on every key dimension is the per-token decay of decay-only gated linear
    attention."""
    r = np.random.default_rng(5)
    q, k, v = r.standard_normal((2, 2, 90, 12)), r.standard_normal((2, 2, 90, 12)), r.standard_normal((2, 2, 90, 7))
    h0 = r.standard_normal((2, 2, 12, 7))
    la = -r.uniform(0.0, 0.5, (2, 2, 90))
    o1, h1 = oracle.gla_vec_prefill(q, k, v, np.repeat(la[..., None], 12, axis=-1), h0)
    o2, h2 = oracle.gla_prefill(q, k, v, la, h0)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h1, h2, rtol=1e-12, atol=1e-12)


def test_gla_vec_zero_gate_is_plain_linear_attention():
    r = np.random.default_rng(6)
    q, k, v = r.standard_normal((1, 3, 50, 8)), r.standard_normal((1, 3, 50, 8)), r.standard_normal((1, 3, 50, 8))
    o1, h1 = oracle.gla_vec_prefill(q, k, v, np.zeros((1, 3, 50, 8)))
    o2, h2 = oracle.linattn_prefill(q, k, v)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)


def test_gla_vec_closed_dimensions_forget():
    """a_t[i] = 0 on some key dimensions: those rows of the state hold only the latest token,
    h[i, :] = k_t[i] v_t, while the open (a = 1) rows sum every token."""
    r = np.random.default_rng(7)
    L, Dk, Dv = 20, 6, 5
    q, k, v = r.standard_normal((L, Dk)), r.standard_normal((L, Dk)), r.standard_normal((L, Dv))
    la = np.zeros((L, Dk))
    la[:, :3] = -np.inf
    o, hf = oracle.gla_vec_prefill(q, k, v, la)
    np.testing.assert_allclose(hf[0, 0, :3], k[-1, :3, None] * v[-1][None, :], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hf[0, 0, 3:], k[:, 3:].T @ v, rtol=1e-12, atol=1e-12)
    ref_o = (q[:, :3] * k[:, :3]).sum(-1)[:, None] * v + np.stack(
        [q[t, 3:] @ (k[:t + 1, 3:].T @ v[:t + 1]) for t in range(L)])
    np.testing.assert_allclose(o[0, 0], ref_o, rtol=1e-12, atol=1e-12)


def test_gla_vec_chaining():
    """Two calls chained through the state equal one call over the concatenated sequence."""
    r = np.random.default_rng(8)
    q, k, v = r.standard_normal((1, 2, 77, 16)), r.standard_normal((1, 2, 77, 16)), r.standard_normal((1, 2, 77, 9))
    la = -r.uniform(0.0, 0.2, (1, 2, 77, 16))
    h0 = r.standard_normal((1, 2, 16, 9))
    o, h = oracle.gla_vec_prefill(q, k, v, la, h0)
    a, b = slice(0, 30), slice(30, 77)
    o1, h1 = oracle.gla_vec_prefill(q[:, :, a], k[:, :, a], v[:, :, a], la[:, :, a], h0)
    o2, h2 = oracle.gla_vec_prefill(q[:, :, b], k[:, :, b], v[:, :, b], la[:, :, b], h1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h2, h, rtol=1e-12, atol=1e-12)
