"""Pins for the oracle's bidirectional (non-causal) linear attention (CPU only).

The datadaily.news overview (section "Linear attention") writes the non-causal form with a
kernel feature map: KV = sum_n phi(k_n) v_n^T, o_n = phi(q_n)^T KV, normalised by
Z_n = phi(q_n) . sum_m phi(k_m), phi = elu + 1 by default. Its point is that this equals the
quadratic form (phi(Q) phi(K)^T) V with row sums as normaliser, reordered. The pins check the
oracle against that quadratic form, exact rational arithmetic, the feature map's closed form,
invariances that hold for any inputs, and the causal oracle at the last token.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _inputs(seed, B, H, L, Dk, Dv, positive=False):
    r = np.random.default_rng(seed)
    q, k = r.standard_normal((B, H, L, Dk)), r.standard_normal((B, H, L, Dk))
    if positive:
        q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
    return q, k, r.standard_normal((B, H, L, Dv))


def _elu1(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


@pytest.mark.parametrize("normalize", [False, True])
@pytest.mark.parametrize("elu1", [False, True])
@pytest.mark.parametrize("L,Dk,Dv", [(1, 4, 3), (37, 8, 8), (130, 16, 12)])
def test_equals_quadratic_form(normalize, elu1, L, Dk, Dv):
    """o = (phi(Q) phi(K)^T) V, divided by the row sums of phi(Q) phi(K)^T when normalising."""
    q, k, v = _inputs(L + Dk, 2, 2, L, Dk, Dv, positive=normalize and not elu1)
    o, _ = oracle.linattn_bidir(q, k, v, normalize=normalize, elu1=elu1)
    fq, fk = (_elu1(q), _elu1(k)) if elu1 else (q, k)
    A = fq @ np.swapaxes(fk, -1, -2)                  # [B,H,L,L], every pair of tokens
    ref = A @ v
    if normalize:
        ref = ref / A.sum(-1, keepdims=True)
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-12)


def test_exact_rational():
    """Identity feature map, normalised, in exact rationals: o_n = sum_m (q_n.k_m) v_m / sum_m q_n.k_m."""
    gen = np.random.default_rng(5)
    L, Dk, Dv = 5, 3, 2
    fr = lambda r, c: [[Fraction(int(gen.integers(1, 9)), 4) for _ in range(c)] for _ in range(r)]
    q, k, v = fr(L, Dk), fr(L, Dk), [[Fraction(int(gen.integers(-8, 9)), 4) for _ in range(Dv)] for _ in range(L)]
    exact = []
    for n in range(L):
        w = [sum(q[n][i] * k[m][i] for i in range(Dk)) for m in range(L)]
        exact.append([sum(w[m] * v[m][j] for m in range(L)) / sum(w) for j in range(Dv)])
    f = lambda m: np.array([[float(x) for x in row] for row in m])
    o, kv = oracle.linattn_bidir(f(q), f(k), f(v), normalize=True, elu1=False)
    np.testing.assert_allclose(o[0, 0], f(exact), rtol=1e-13, atol=1e-14)
    kv_exact = [[sum(k[m][i] * v[m][j] for m in range(L)) for j in range(Dv)] for i in range(Dk)]
    np.testing.assert_allclose(kv[0, 0], f(kv_exact), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("x,phi", [(0.0, 1.0), (1.0, 2.0), (2.5, 3.5), (-1.0, np.exp(-1.0)), (-3.0, np.exp(-3.0))])
def test_feature_map_values(x, phi):
    """One token, Dk = Dv = 1, q = 1 (phi(1) = 2), v = 1: unnormalised o = 2 phi(x), kv = phi(x)."""
    o, kv = oracle.linattn_bidir(np.ones((1, 1, 1, 1)), np.full((1, 1, 1, 1), x), np.ones((1, 1, 1, 1)),
                                 normalize=False, elu1=True)
    assert o[0, 0, 0, 0] == pytest.approx(2.0 * phi, rel=1e-15)
    assert kv[0, 0, 0, 0] == pytest.approx(phi, rel=1e-15)


def test_invariances():
    q, k, v = _inputs(9, 1, 3, 50, 8, 6, positive=True)
    o, kv = oracle.linattn_bidir(q, k, v, normalize=True, elu1=False)
    # keys scaled by c > 0: normalised output unchanged; values scaled: output scaled
    o2, _ = oracle.linattn_bidir(q, 3.0 * k, v, normalize=True, elu1=False)
    np.testing.assert_allclose(o2, o, rtol=1e-12)
    o3, _ = oracle.linattn_bidir(q, k, -2.0 * v, normalize=True, elu1=False)
    np.testing.assert_allclose(o3, -2.0 * o, rtol=1e-12)
    # permuting the key/value tokens together changes nothing; permuting queries permutes outputs
    perm = np.random.default_rng(1).permutation(50)
    o4, kv4 = oracle.linattn_bidir(q, k[:, :, perm], v[:, :, perm], normalize=True, elu1=False)
    np.testing.assert_allclose(o4, o, rtol=1e-12)
    np.testing.assert_allclose(kv4, kv, rtol=1e-12, atol=1e-12)
    o5, _ = oracle.linattn_bidir(q[:, :, perm], k, v, normalize=True, elu1=False)
    np.testing.assert_allclose(o5, o[:, :, perm], rtol=1e-12)


def test_equal_keys_give_the_mean_value():
    """All keys equal: every normalised output is the mean of the values, whatever the query."""
    q, _, v = _inputs(3, 2, 2, 40, 8, 5)
    k = np.broadcast_to(np.random.default_rng(4).standard_normal(8), (2, 2, 40, 8)).copy()
    o, _ = oracle.linattn_bidir(q, k, v, normalize=True, elu1=True)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), rtol=1e-11, atol=1e-12)


def test_last_token_matches_causal():
    """Unnormalised, identity feature map: the last token sees every key in both forms, so its
    output equals the causal linear-attention oracle's, and kv equals its final state."""
    q, k, v = _inputs(12, 2, 2, 70, 16, 16)
    o, kv = oracle.linattn_bidir(q, k, v, normalize=False, elu1=False)
    oc, hc = oracle.linattn_prefill(q, k, v)
    np.testing.assert_allclose(o[:, :, -1], oc[:, :, -1], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(kv, hc, rtol=1e-11, atol=1e-12)
    assert not np.allclose(o[:, :, 0], oc[:, :, 0])


def test_empty_sequence():
    z = np.zeros((1, 2, 0, 8))
    o, kv = oracle.linattn_bidir(z, z, z, normalize=True, elu1=True)
    assert o.shape == (1, 2, 0, 8) and np.all(kv == 0)
