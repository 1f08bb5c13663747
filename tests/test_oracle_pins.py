"""Pins for the fp64 oracle: it is checked against things other than itself.

Each test names what it pins. Together they are meant to catch the plausible slips in a
recurrence implementation: a dropped gate, a wrong sign on the delta term, a swapped
k/v role or a transposed state, an off-by-one in causality, a gate applied to the write.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from chunked_form import gdn_chunked, linattn_chunked
from gated_deltanet_chunked_rule_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def gdn_random(seed, B, H, L, Dk, Dv, gate="config", with_h0=True):
    r = np.random.default_rng(seed)
    q = unit_rows(r.standard_normal((B, H, L, Dk)))
    k = unit_rows(r.standard_normal((B, H, L, Dk)))
    v = r.standard_normal((B, H, L, Dv))
    beta = 1 / (1 + np.exp(-r.standard_normal((B, H, L))))
    if gate == "config":
        la = -np.log1p(np.exp(r.standard_normal((B, H, L)) + 2.0))
    else:
        la = -r.uniform(0, 0.01, (B, H, L))
    h0 = 0.1 * r.standard_normal((B, H, Dk, Dv)) if with_h0 else None
    return q, k, v, beta, la, h0


# --------------------------------------------------------------------------------------
# worked examples derived by hand (tests/golden/hand_examples.json)
# --------------------------------------------------------------------------------------
def test_hand_examples():
    g = json.load(open(GOLDEN))
    e = g["prefill_gdn"]
    o, hf = oracle.gdn_prefill(np.array(e["q"]), np.array(e["k"]), np.array(e["v"]),
                               np.array(e["beta"]), np.log(np.array(e["alpha"])))
    np.testing.assert_allclose(o[0, 0], e["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(hf[0, 0], e["h_final"], rtol=0, atol=1e-14)

    e = g["prefill_linattn"]
    o, hf = oracle.linattn_prefill(np.array(e["q"]), np.array(e["k"]), np.array(e["v"]))
    np.testing.assert_allclose(o[0, 0], e["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(hf[0, 0], e["h_final"], rtol=0, atol=1e-14)

    e = g["decode_gdn"]
    o, st = oracle.gdn_decode_step(np.array(e["q"])[None], np.array(e["k"])[None], np.array(e["v"])[None],
                                   np.array([e["beta"]]), np.log(np.array([e["alpha"]])),
                                   np.array(e["state"])[None, None])
    np.testing.assert_allclose(o[0, 0], e["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(st[0, 0], e["new_state"], rtol=0, atol=1e-14)


# --------------------------------------------------------------------------------------
# brute force in exact rational arithmetic, with the full matrix (I - beta k k^T)
# --------------------------------------------------------------------------------------
def _frac_mat(rows, cols, gen):
    return [[Fraction(int(gen.integers(-4, 5)), int(gen.integers(1, 5))) for _ in range(cols)]
            for _ in range(rows)]


def _mm(a, b):
    return [[sum(a[i][t] * b[t][j] for t in range(len(b))) for j in range(len(b[0]))] for i in range(len(a))]


def test_gdn_exact_rational_bruteforce():
    """S_t = a S_{t-1} (I - beta k k^T) + beta v k^T with explicit d x d matrices, in Fractions.

    Keys are not normalised, Dk != Dv, and h0 is non-zero, so every term and the state
    orientation matter."""
    gen = np.random.default_rng(7)
    Dk, Dv, L = 3, 2, 5
    q = _frac_mat(L, Dk, gen)
    k = _frac_mat(L, Dk, gen)
    v = _frac_mat(L, Dv, gen)
    beta = [Fraction(int(gen.integers(1, 4)), 4) for _ in range(L)]
    alpha = [Fraction(int(gen.integers(1, 8)), 8) for _ in range(L)]
    h0 = _frac_mat(Dk, Dv, gen)                       # key-major
    S = [[h0[i][j] for i in range(Dk)] for j in range(Dv)]   # S = h0^T
    o_exact = []
    for t in range(L):
        kk = [[k[t][i] * k[t][j] for j in range(Dk)] for i in range(Dk)]
        M = [[(1 if i == j else 0) - beta[t] * kk[i][j] for j in range(Dk)] for i in range(Dk)]
        SM = _mm(S, M)
        S = [[alpha[t] * SM[r][c] + beta[t] * v[t][r] * k[t][c] for c in range(Dk)] for r in range(Dv)]
        o_exact.append([sum(S[r][c] * q[t][c] for c in range(Dk)) for r in range(Dv)])
    f = lambda m: np.array([[float(x) for x in row] for row in m])
    o, hf = oracle.gdn_prefill(f(q), f(k), f(v), np.array([float(b) for b in beta]),
                               np.log(np.array([float(a) for a in alpha])), f(h0))
    np.testing.assert_allclose(o[0, 0], f(o_exact), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hf[0, 0], f(S).T, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------------------
# plain linear attention against the masked quadratic form and the page's code
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("L,Dk,Dv", [(1, 8, 8), (37, 16, 8), (256, 32, 48)])
def test_linattn_equals_masked_quadratic_form(L, Dk, Dv):
    """alpha = 1, no delta term: o = (Q K^T * M) V + Q h0 with M causal incl. the diagonal
    (the associativity argument of the datadaily.news overview, section 'Linear attention')."""
    r = np.random.default_rng(L)
    q, k = r.standard_normal((L, Dk)), r.standard_normal((L, Dk))
    v, h0 = r.standard_normal((L, Dv)), r.standard_normal((Dk, Dv))
    o, hf = oracle.linattn_prefill(q, k, v, h0)
    ref = np.tril(q @ k.T) @ v + q @ h0
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(hf[0, 0], h0 + k.T @ v, rtol=1e-11, atol=1e-11)


def test_linattn_last_token_equals_page_noncausal_code():
    """At the last token the causal output equals the non-causal KV-then-Q product of the
    datadaily.news code sample (section 'Linear attention'), taken before its normaliser Z
    and applied to feature-mapped q, k = elu(x)+1."""
    r = np.random.default_rng(3)
    x = r.standard_normal((2, 50, 16))
    phi = lambda t: np.where(t > 0, t + 1, np.exp(np.minimum(t, 0)))
    Q, K = phi(x), phi(r.standard_normal((2, 50, 16)))
    V = r.standard_normal((2, 50, 12))
    KV = np.einsum("bnd,bnm->bdm", K, V)
    full = np.einsum("bnd,bdm->bnm", Q, KV)
    o, hf = oracle.linattn_prefill(Q[:, None], K[:, None], V[:, None])
    np.testing.assert_allclose(o[:, 0, -1], full[:, -1], rtol=1e-11)
    np.testing.assert_allclose(hf[:, 0], KV, rtol=1e-11)


# --------------------------------------------------------------------------------------
# the chunked (WY) form reaches the same result
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("gate", ["config", "long"])
@pytest.mark.parametrize("L", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("C", [1, 3, 16, 64])
def test_gdn_chunked_equals_recurrent(L, C, gate):
    q, k, v, beta, la, h0 = gdn_random(100 + L, 1, 1, L, 16, 12, gate=gate)
    o, hf = oracle.gdn_prefill(q, k, v, beta, la, h0)
    oc, hc = gdn_chunked(q[0, 0], k[0, 0], v[0, 0], beta[0, 0], la[0, 0], h0[0, 0], C=C)
    scale_o, scale_h = np.abs(oc).max(), np.abs(hc).max()
    assert np.abs(o[0, 0] - oc).max() <= 1e-11 * scale_o
    assert np.abs(hf[0, 0] - hc).max() <= 1e-11 * scale_h


@pytest.mark.parametrize("L", [1, 65, 130])
def test_linattn_chunked_equals_recurrent(L):
    r = np.random.default_rng(L)
    q, k, v = r.standard_normal((L, 8)), r.standard_normal((L, 8)), r.standard_normal((L, 8))
    o, hf = oracle.linattn_prefill(q, k, v)
    oc, hc = linattn_chunked(q, k, v, C=64)
    np.testing.assert_allclose(o[0, 0], oc, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(hf[0, 0], hc, rtol=1e-10, atol=1e-10)


# --------------------------------------------------------------------------------------
# invariants of the delta rule
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("n,Dk,Dv", [(8, 8, 8), (5, 16, 4), (16, 16, 24)])
def test_retrieval_with_orthonormal_keys(n, Dk, Dv):
    """Orthonormal keys, beta = 1, alpha = 1, zero start: S k_i = v_i for every written i,
    and o_t = v_t when q_t = k_t. Swapping the roles of k and v or transposing the stored
    state fails this when Dk != Dv or the values are random."""
    r = np.random.default_rng(n * Dk)
    basis, _ = np.linalg.qr(r.standard_normal((Dk, Dk)))
    k = basis.T[:n]
    v = r.standard_normal((n, Dv))
    o, hf = oracle.gdn_prefill(k, k, v, np.ones(n), np.zeros(n))
    S = hf[0, 0].T
    np.testing.assert_allclose(S @ k.T, v.T, atol=1e-12)
    np.testing.assert_allclose(o[0, 0], v, atol=1e-12)


def test_delta_overwrite_identity():
    """For any inputs: S_t k = a (1 - beta |k|^2) S_{t-1} k + beta |k|^2 v."""
    r = np.random.default_rng(11)
    N, H, Dk, Dv = 3, 2, 16, 8
    st = r.standard_normal((N, H, Dk, Dv))
    q, k = r.standard_normal((N, H, Dk)), r.standard_normal((N, H, Dk))
    v = r.standard_normal((N, H, Dv))
    beta, la = r.uniform(0, 1, (N, H)), -r.uniform(0, 3, (N, H))
    _, new = oracle.gdn_decode_step(q, k, v, beta, la, st)
    a = np.exp(la)
    kk = np.sum(k * k, -1)
    lhs = np.einsum("nhij,nhi->nhj", new, k)
    old = np.einsum("nhij,nhi->nhj", st, k)
    rhs = (a * (1 - beta * kk))[..., None] * old + (beta * kk)[..., None] * v
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-11)


def test_pure_decay_when_beta_zero():
    """beta = 0 writes nothing: the state only decays by the gate (the SparseGDN article's
    reading of a skipped update, section 'Two-level sparsity'): h_L = exp(sum log a) h0 and
    o_t = exp(g_t) h0^T q_t with g_t the inclusive prefix sum of log a."""
    q, k, v, beta, la, h0 = gdn_random(5, 1, 2, 40, 8, 6, gate="long")
    o, hf = oracle.gdn_prefill(q, k, v, np.zeros_like(beta), la, h0)
    g = np.cumsum(la, axis=-1)
    np.testing.assert_allclose(hf, np.exp(g[..., -1])[..., None, None] * h0, rtol=1e-12)
    ref = np.exp(g)[..., None] * np.einsum("bhtd,bhdm->bhtm", q, h0)
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-13)


def test_one_token_closed_form():
    """S_1 = a h0^T (I - beta k k^T) + beta v k^T: the gate does not scale the new write."""
    r = np.random.default_rng(2)
    Dk, Dv = 6, 4
    q, k, v = r.standard_normal(Dk), r.standard_normal(Dk), r.standard_normal(Dv)
    h0 = r.standard_normal((Dk, Dv))
    beta, a = 0.3, 0.25
    o, hf = oracle.gdn_prefill(q[None], k[None], v[None], np.array([beta]), np.log([a]), h0)
    S1 = a * h0.T @ (np.eye(Dk) - beta * np.outer(k, k)) + beta * np.outer(v, k)
    np.testing.assert_allclose(hf[0, 0], S1.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o[0, 0, 0], S1 @ q, rtol=1e-12, atol=1e-12)


def test_chaining_initial_and_final_state():
    """Running L1 then L2 tokens from the returned state equals running L1 + L2 at once
    (the state after prefill is what generation continues from, SparseGDN article,
    section 'Limitations')."""
    q, k, v, beta, la, h0 = gdn_random(9, 2, 2, 90, 16, 16)
    o, hf = oracle.gdn_prefill(q, k, v, beta, la, h0)
    a = slice(0, 37)
    b = slice(37, 90)
    o1, h1 = oracle.gdn_prefill(q[:, :, a], k[:, :, a], v[:, :, a], beta[:, :, a], la[:, :, a], h0)
    o2, h2 = oracle.gdn_prefill(q[:, :, b], k[:, :, b], v[:, :, b], beta[:, :, b], la[:, :, b], h1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h2, hf, rtol=1e-12, atol=1e-12)


def test_decode_steps_equal_prefill():
    """T single-token decode steps give the prefill's outputs and final state."""
    q, k, v, beta, la, h0 = gdn_random(4, 1, 3, 12, 8, 8)
    o, hf = oracle.gdn_prefill(q, k, v, beta, la, h0)
    st = h0[0]
    for t in range(12):
        ot, st = oracle.gdn_decode_step(q[0, :, t], k[0, :, t], v[0, :, t], beta[0, :, t], la[0, :, t], st)
        np.testing.assert_allclose(ot[0], o[0, :, t], rtol=1e-12, atol=1e-12)
        st = st[0]
    np.testing.assert_allclose(st, hf[0], rtol=1e-12, atol=1e-12)


def test_value_columns_independent_and_linear():
    """The d_v columns of o and of the state evolve independently, and the map is linear in
    (V, h0) jointly for fixed q, k, beta, alpha."""
    q, k, v, beta, la, h0 = gdn_random(21, 1, 1, 70, 8, 10)
    o, hf = oracle.gdn_prefill(q, k, v, beta, la, h0)
    cols = [1, 4, 7]
    oc, hc = oracle.gdn_prefill(q, k, v[..., cols], beta, la, h0[..., cols])
    np.testing.assert_allclose(oc, o[..., cols], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(hc, hf[..., cols], rtol=1e-12, atol=1e-13)
    r = np.random.default_rng(0)
    v2, h2 = r.standard_normal(v.shape), r.standard_normal(h0.shape)
    o2, hf2 = oracle.gdn_prefill(q, k, v2, beta, la, h2)
    o3, hf3 = oracle.gdn_prefill(q, k, 2 * v - 3 * v2, beta, la, 2 * h0 - 3 * h2)
    np.testing.assert_allclose(o3, 2 * o - 3 * o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(hf3, 2 * hf - 3 * hf2, rtol=1e-10, atol=1e-12)


def test_oracle_on_generated_inputs_matches_chunked_form():
    """The seeded generator's small fp32 workload (B=1, H=2, L=512, d=64) through both forms."""
    cfg = inputs.GDN_REF_FP32
    x = inputs.prefill_inputs(cfg)
    o, hf = oracle.gdn_prefill(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], x["h0"])
    for h in range(cfg.H):
        oc, hc = gdn_chunked(x["q"][0, h], x["k"][0, h], x["v"][0, h], x["beta"][0, h],
                             x["log_alpha"][0, h], None, C=64)
        assert np.abs(o[0, h] - oc).max() <= 1e-11 * np.abs(oc).max()
        assert np.abs(hf[0, h] - hc).max() <= 1e-11 * np.abs(hc).max()


def test_generator_rounding_and_prefix():
    """bf16 rounding is to nearest-even and a shorter L is a prefix of a longer one."""
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -9), 3.0])
    np.testing.assert_array_equal(inputs.round_bf16(x), [1.0, 1.0 + 2.0 ** -6, -1.0, 3.0])
    cfg = inputs.GDN_32K
    a = inputs.prefill_slice(cfg, 0, 3, L=100)
    b = inputs.prefill_slice(cfg, 0, 3, L=300)
    for key in ("q", "k", "v", "beta", "log_alpha"):
        np.testing.assert_array_equal(a[key], b[key][:100])
    np.testing.assert_array_equal(a["h0"], b["h0"])
    assert np.all(inputs.round_bf16(a["q"]) == a["q"])
