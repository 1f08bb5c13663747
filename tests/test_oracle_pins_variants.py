"""Pins for the oracle's two variants of the hot path (CPU only):

- decay-only gated linear attention, S_t = a_t S_{t-1} + v_t k_t^T (linear attention with a
  per-token decay, one of the modifications the forpes.ru article on linear attention lists
  after the recurrent form);
- the gated delta rule with skipped chunk updates: a skipped chunk only decays the carried state,
  every token still gets its output from the chunk-start snapshot (the SparseGDN article,
  fileenergy.com, selector and scan_with_skips illustration).

Each is checked against code written independently of the oracle: closed forms in NumPy and
exact rational brute force with explicit matrices.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _frac_mat(r, c, gen):
    return [[Fraction(int(gen.integers(-4, 5)), 4) for _ in range(c)] for _ in range(r)]


def _mm(A, B):
    return [[sum(A[i][t] * B[t][j] for t in range(len(B))) for j in range(len(B[0]))] for i in range(len(A))]


def _f(m):
    return np.array([[float(x) for x in row] for row in m])


# --------------------------------------------------------------------------------------
# decay-only gated linear attention
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("L,Dk,Dv", [(1, 8, 8), (45, 16, 8), (200, 32, 40)])
def test_gla_equals_decayed_masked_form(L, Dk, Dv):
    """o_t = sum_{s<=t} exp(g_t - g_s) (q_t.k_s) v_s + exp(g_t) h0^T q_t and
    h_L = exp(g_L) h0 + sum_s exp(g_L - g_s) k_s v_s^T, g the inclusive prefix sum of log a."""
    r = np.random.default_rng(L + 100)
    q, k = r.standard_normal((L, Dk)), r.standard_normal((L, Dk))
    v, h0 = r.standard_normal((L, Dv)), r.standard_normal((Dk, Dv))
    la = -r.uniform(0.0, 0.3, L)
    o, hf = oracle.gla_prefill(q, k, v, la, h0)
    g = np.cumsum(la)
    gamma = np.tril(np.exp(g[:, None] - g[None, :]))
    ref = ((q @ k.T) * gamma) @ v + np.exp(g)[:, None] * (q @ h0)
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-11, atol=1e-11)
    ref_h = np.exp(g[-1]) * h0 + (k * np.exp(g[-1] - g)[:, None]).T @ v
    np.testing.assert_allclose(hf[0, 0], ref_h, rtol=1e-11, atol=1e-11)


def test_gla_zero_gate_is_plain_linear_attention():
    """log a = 0 is plain linear attention, bit for bit (a = 1 scales exactly)."""
    r = np.random.default_rng(11)
    q, k, v = r.standard_normal((2, 3, 70, 16)), r.standard_normal((2, 3, 70, 16)), r.standard_normal((2, 3, 70, 12))
    h0 = r.standard_normal((2, 3, 16, 12))
    o1, h1 = oracle.gla_prefill(q, k, v, np.zeros((2, 3, 70)), h0)
    o2, h2 = oracle.linattn_prefill(q, k, v, h0)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)


def test_gla_exact_rational_bruteforce():
    """S_t = a_t S_{t-1} + v_t k_t^T with explicit Dv x Dk matrices in Fractions, Dk != Dv, h0 != 0."""
    gen = np.random.default_rng(17)
    Dk, Dv, L = 3, 2, 6
    q, k, v = _frac_mat(L, Dk, gen), _frac_mat(L, Dk, gen), _frac_mat(L, Dv, gen)
    alpha = [Fraction(int(gen.integers(1, 8)), 8) for _ in range(L)]
    h0 = _frac_mat(Dk, Dv, gen)
    S = [[h0[i][j] for i in range(Dk)] for j in range(Dv)]
    o_exact = []
    for t in range(L):
        S = [[alpha[t] * S[rr][c] + v[t][rr] * k[t][c] for c in range(Dk)] for rr in range(Dv)]
        o_exact.append([sum(S[rr][c] * q[t][c] for c in range(Dk)) for rr in range(Dv)])
    o, hf = oracle.gla_prefill(_f(q), _f(k), _f(v), np.log(np.array([float(a) for a in alpha])), _f(h0))
    np.testing.assert_allclose(o[0, 0], _f(o_exact), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hf[0, 0], _f(S).T, rtol=1e-12, atol=1e-12)


def test_gla_chaining():
    r = np.random.default_rng(5)
    q, k, v = r.standard_normal((1, 2, 80, 8)), r.standard_normal((1, 2, 80, 8)), r.standard_normal((1, 2, 80, 8))
    la = -r.uniform(0, 0.2, (1, 2, 80))
    o, hf = oracle.gla_prefill(q, k, v, la)
    a, b = slice(0, 33), slice(33, 80)
    o1, h1 = oracle.gla_prefill(q[:, :, a], k[:, :, a], v[:, :, a], la[:, :, a])
    o2, h2 = oracle.gla_prefill(q[:, :, b], k[:, :, b], v[:, :, b], la[:, :, b], h1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h2, hf, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------------------
# gated delta rule with skipped chunk updates
# --------------------------------------------------------------------------------------
def _skip_bruteforce(q, k, v, beta, alpha, h0, keep, C):
    """Exact rational evaluation of the skip semantics with explicit (I - beta k k^T) matrices."""
    L, Dk, Dv = len(q), len(q[0]), len(v[0])
    S = [[h0[i][j] for i in range(Dk)] for j in range(Dv)]
    outs = []
    for c in range((L + C - 1) // C):
        snap = [row[:] for row in S]
        decay = Fraction(1)
        for t in range(c * C, min(L, (c + 1) * C)):
            kk = [[k[t][i] * k[t][j] for j in range(Dk)] for i in range(Dk)]
            M = [[(1 if i == j else 0) - beta[t] * kk[i][j] for j in range(Dk)] for i in range(Dk)]
            SM = _mm(S, M)
            S = [[alpha[t] * SM[rr][cc] + beta[t] * v[t][rr] * k[t][cc] for cc in range(Dk)] for rr in range(Dv)]
            outs.append([sum(S[rr][cc] * q[t][cc] for cc in range(Dk)) for rr in range(Dv)])
            decay *= alpha[t]
        if not keep[c]:
            S = [[decay * x for x in row] for row in snap]
    return outs, S


@pytest.mark.parametrize("keep", [[1, 0, 1], [0, 0, 1], [0, 1, 0], [0, 0, 0], [1, 1, 1]])
def test_skip_exact_rational_bruteforce(keep):
    gen = np.random.default_rng(23)
    Dk, Dv, L, C = 3, 2, 7, 3           # three chunks, the last one ragged
    q, k, v = _frac_mat(L, Dk, gen), _frac_mat(L, Dk, gen), _frac_mat(L, Dv, gen)
    beta = [Fraction(int(gen.integers(1, 4)), 4) for _ in range(L)]
    alpha = [Fraction(int(gen.integers(1, 8)), 8) for _ in range(L)]
    h0 = _frac_mat(Dk, Dv, gen)
    o_exact, S = _skip_bruteforce(q, k, v, beta, alpha, h0, keep, C)
    o, hf = oracle.gdn_prefill_skip(_f(q), _f(k), _f(v), np.array([float(b) for b in beta]),
                                    np.log(np.array([float(a) for a in alpha])), np.array(keep), _f(h0), chunk=C)
    np.testing.assert_allclose(o[0, 0], _f(o_exact), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hf[0, 0], _f(S).T, rtol=1e-12, atol=1e-12)


def _gdn_inputs(seed, B, H, L, D):
    r = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q, k = unit(r.standard_normal((B, H, L, D))), unit(r.standard_normal((B, H, L, D)))
    v = r.standard_normal((B, H, L, D))
    beta = 1 / (1 + np.exp(-r.standard_normal((B, H, L))))
    la = -r.uniform(0, 0.05, (B, H, L))
    h0 = 0.1 * r.standard_normal((B, H, D, D))
    return q, k, v, beta, la, h0


def test_skip_all_kept_is_the_dense_rule():
    """keep everywhere: the plain gated delta rule, bit for bit (SparseGDN article, check against
    the native kernel at 100 percent retention)."""
    q, k, v, beta, la, h0 = _gdn_inputs(3, 2, 2, 150, 16)
    keep = np.ones((2, 2, 3), dtype=np.int32)
    o1, h1 = oracle.gdn_prefill_skip(q, k, v, beta, la, keep, h0, chunk=64)
    o2, h2 = oracle.gdn_prefill(q, k, v, beta, la, h0)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)


def test_skip_none_kept_only_decays_the_carried_state():
    """keep nowhere: the final state is exp(sum log a) h0; each chunk's outputs are the delta rule
    run from the decayed snapshot exp(g at the chunk start) h0, so chunk 0 matches the dense rule."""
    q, k, v, beta, la, h0 = _gdn_inputs(8, 1, 2, 130, 8)
    keep = np.zeros((1, 2, 3), dtype=np.int32)
    o, hf = oracle.gdn_prefill_skip(q, k, v, beta, la, keep, h0, chunk=64)
    g = np.cumsum(la, axis=-1)
    np.testing.assert_allclose(hf, np.exp(g[..., -1])[..., None, None] * h0, rtol=1e-12, atol=1e-15)
    od, _ = oracle.gdn_prefill(q, k, v, beta, la, h0)
    np.testing.assert_array_equal(o[:, :, :64], od[:, :, :64])
    assert not np.allclose(o[:, :, 64:], od[:, :, 64:])
