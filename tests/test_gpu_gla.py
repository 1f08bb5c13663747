"""GPU parity of gated linear attention with a gate per key dimension (gla_prefill_fwd) against
the fp64 oracle (oracle.gla_vec_prefill): bf16 and fp32, d = 64 and 128, ragged lengths, short-
and long-memory gates, blocks of many chunks (small workspaces), in-place state, chaining through
the state, repeat calls bitwise equal, and the full 8K workload on sampled slices.

Same error metric and bounds as test_gpu_parity.py.
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_chunked_rule_amd import inputs
from gpu_util import TOL_BF16, TOL_F32, dev_tensor, host, max_rel_err, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

from gated_deltanet_chunked_rule_amd import ops  # noqa: E402

TD = {"bf16": torch.bfloat16, "f32": torch.float32}


def _cfg(name, B, H, L, D, dtype, seed, gate_dist="config", qk="elu1", h0=0.1):
    return inputs.LINATTN_8K.with_(name=name, B=B, H=H, L=L, Dk=D, Dv=D, dtype=dtype, seed=seed, qk=qk,
                                   gates=False, gate_dist=gate_dist, h0=h0)


def _dev(cfg, x, la):
    dt = TD[cfg.dtype]
    q, k, v = (dev_tensor(x[n], dt) for n in ("q", "k", "v"))
    h0 = dev_tensor(x["h0"], torch.float32)
    return q, k, v, dev_tensor(la, torch.float32), h0


def _check(cfg, o, hf, ro, rh):
    tol = TOL_BF16 if cfg.dtype == "bf16" else TOL_F32
    eo, eh = max_rel_err(host(o), ro), max_rel_err(host(hf), rh)
    say(f"  {cfg.name}: max rel err o {eo:.3e}, h_final {eh:.3e} (bound {tol:g})")
    assert eo <= tol and eh <= tol, (eo, eh)


@pytest.mark.parametrize("gate_dist", ["config", "long"])
@pytest.mark.parametrize("dtype,D,L", [("bf16", 128, 1), ("bf16", 128, 64), ("bf16", 128, 1000), ("bf16", 64, 777),
                                       ("f32", 128, 333), ("f32", 64, 1000), ("f32", 64, 17)])
def test_gla_ragged(gate_dist, dtype, D, L):
    cfg = _cfg(f"gla_{gate_dist}_{dtype}_d{D}_L{L}", 2, 2, L, D, dtype, 7200 + D + L + (gate_dist == "long"),
               gate_dist=gate_dist)
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    la = inputs.gate_vectors(cfg)
    q, k, v, lad, h0 = _dev(cfg, x, la)
    o, hf = ops.gla_prefill_fwd(q, k, v, lad, h0)
    torch.cuda.synchronize()
    ro, rh = oracle.gla_vec_prefill(x["q"], x["k"], x["v"], la, x["h0"])
    _check(cfg, o, hf, ro, rh)


@pytest.mark.parametrize("dtype,D,L", [("bf16", 128, 1500), ("f32", 64, 900), ("f32", 128, 900), ("bf16", 64, 129)])
def test_gla_small_workspace_long_blocks(dtype, D, L):
    """The smallest workspace (one block of all chunks per slice) and one of two blocks; each
    result checked, and a second call with the same workspace bitwise equal."""
    cfg = _cfg(f"gla_blocks_{dtype}_d{D}_L{L}", 1, 3, L, D, dtype, 7300 + D + L, gate_dist="long", qk="l2")
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    la = inputs.gate_vectors(cfg)
    q, k, v, lad, h0 = _dev(cfg, x, la)
    ro, rh = oracle.gla_vec_prefill(x["q"], x["k"], x["v"], la, x["h0"])
    per = D * D * 4 + D * 4
    for nblk in (1, 2):
        ws = torch.empty(nblk * cfg.B * cfg.H * per, dtype=torch.uint8, device="cuda")
        o, hf = ops.gla_prefill_fwd(q, k, v, lad, h0, workspace=ws)
        o2, hf2 = ops.gla_prefill_fwd(q, k, v, lad, h0, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(hf, hf2)
        _check(cfg.with_(name=f"{cfg.name} {nblk} block(s)"), o, hf, ro, rh)


def test_gla_in_place_state_and_chaining():
    """h_final == h0 is read before it is written; two calls chained through the state match one
    call over the whole sequence (to the bound: the block split differs)."""
    cfg = _cfg("gla_in_place", 1, 2, 700, 128, "bf16", 7400, gate_dist="long")
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    la = inputs.gate_vectors(cfg)
    q, k, v, lad, h0 = _dev(cfg, x, la)
    o_ref, h_ref = ops.gla_prefill_fwd(q, k, v, lad, h0.clone())
    state = h0.clone()
    o, hf = ops.gla_prefill_fwd(q, k, v, lad, state, h_final=state)
    torch.cuda.synchronize()
    assert hf.data_ptr() == state.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(hf, h_ref)
    s = 300
    part = lambda t, a, b: t[:, :, a:b].contiguous()
    o1, h1 = ops.gla_prefill_fwd(part(q, 0, s), part(k, 0, s), part(v, 0, s), part(lad, 0, s), h0)
    o2, h2 = ops.gla_prefill_fwd(part(q, s, 700), part(k, s, 700), part(v, s, 700), part(lad, s, 700), h1)
    torch.cuda.synchronize()
    ro, rh = oracle.gla_vec_prefill(x["q"], x["k"], x["v"], la, x["h0"])
    _check(cfg.with_(name="gla_chained"), torch.cat([o1, o2], dim=2), h2, ro, rh)


def test_gla_zero_length_copies_state():
    cfg = _cfg("gla_L0", 1, 2, 5, 64, "f32", 7500)
    x = inputs.prefill_inputs(cfg)
    h0 = dev_tensor(x["h0"], torch.float32)
    e = torch.empty((1, 2, 0, 64), device="cuda")
    o, hf = ops.gla_prefill_fwd(e, e, e, e, h0)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 64) and torch.equal(hf, h0)


def test_gla_full_8k_workload_sampled():
    """The 8K linear-attention workload (B=4, H=16, L=8192, d=128, bf16) with per-dimension
    gates, launched whole with the preferred workspace; two slices against the oracle."""
    cfg = inputs.LINATTN_8K.with_(name="gla_B4H16L8192d128", gate_dist="config", h0=0.1)
    say(f"case {cfg.name}")
    sample = [(0, 3), (3, 15)]
    dt = torch.bfloat16
    shape = (cfg.B, cfg.H, cfg.L, cfg.Dk)
    q, k, v = (torch.empty(shape, dtype=dt, device="cuda") for _ in range(3))
    h0 = torch.empty((cfg.B, cfg.H, cfg.Dk, cfg.Dv), dtype=torch.float32, device="cuda")
    la = torch.from_numpy(inputs.gate_vectors(cfg).astype(np.float32)).to("cuda")
    kept = {}
    for b in range(cfg.B):
        for h in range(cfg.H):
            s = inputs.prefill_slice(cfg, b, h)
            for name, t in (("q", q), ("k", k), ("v", v)):
                t[b, h] = dev_tensor(s[name], dt)
            h0[b, h] = dev_tensor(s["h0"], torch.float32)
            if (b, h) in sample:
                kept[(b, h)] = s
    o, hf = ops.gla_prefill_fwd(q, k, v, la, h0)
    torch.cuda.synchronize()
    lah = host(la)
    for (b, h) in sample:
        s = kept[(b, h)]
        say(f"  oracle on slice {(b, h)}")
        ro, rh = oracle.gla_vec_prefill(s["q"], s["k"], s["v"], lah[b, h], s["h0"])
        _check(cfg.with_(name=f"{cfg.name} slice {(b, h)}"), o[b:b + 1, h:h + 1], hf[b:b + 1, h:h + 1], ro, rh)


@pytest.mark.parametrize("gate_dist", ["strong", "very_strong"])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("f32", 128)])
def test_gla_strong_gates(dtype, D, gate_dist):
    """log a ~ -U(0, 8) and -U(0, 40) per token and dimension: a chunk's cumulative gates reach
    -2,560, far past exp's range in fp32; every factor the kernels form must stay at most 1."""
    cfg = _cfg(f"gla_{gate_dist}_{dtype}_d{D}", 1, 2, 333, D, dtype, 7600 + D + (gate_dist == "very_strong"),
               gate_dist=gate_dist, qk="l2")
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    la = inputs.gate_vectors(cfg)
    q, k, v, lad, h0 = _dev(cfg, x, la)
    o, hf = ops.gla_prefill_fwd(q, k, v, lad, h0)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(hf).all()
    ro, rh = oracle.gla_vec_prefill(x["q"], x["k"], x["v"], la, x["h0"])
    _check(cfg, o, hf, ro, rh)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 128), ("bf16", 64), ("f32", 64)])
def test_gla_closed_dimensions(dtype, D):
    """Zero gates (log a = -inf): a quarter of the key dimensions closed at every token (their
    state rows hold only the latest token), an eighth closed at random tokens (each one clears
    that row), the rest long-memory; two blocks per slice, against the oracle, which computes
    exp(-inf) = 0."""
    cfg = _cfg(f"gla_closed_{dtype}_d{D}", 1, 2, 64 * 9 + 21, D, dtype, 7650 + D, gate_dist="long", qk="l2")
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    la = inputs.gate_vectors(cfg).copy()
    rng = np.random.default_rng(D)
    la[:, :, :, : D // 4] = -np.inf
    sparse = rng.random(la[:, :, :, D // 4: D // 4 + D // 8].shape) < 0.05
    la[:, :, :, D // 4: D // 4 + D // 8][sparse] = -np.inf
    q, k, v, lad, h0 = _dev(cfg, x, la)
    ws = torch.empty(max(1, 2 * 2 * (D * D * 4 + D * 4)), dtype=torch.uint8, device="cuda")
    o, hf = ops.gla_prefill_fwd(q, k, v, lad, h0, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(hf).all()
    ro, rh = oracle.gla_vec_prefill(x["q"], x["k"], x["v"], la, x["h0"])
    assert np.isfinite(ro).all() and np.isfinite(rh).all()
    _check(cfg, o, hf, ro, rh)
    # the always-closed rows of the final state are the last token's k v^T exactly in the oracle
    assert np.allclose(rh[:, :, : D // 4], x["k"][:, :, -1, : D // 4, None] * x["v"][:, :, -1, None, :])


def test_gla_equal_gates_match_per_token_decay():
    """The same gate on every key dimension is the per-token decay: gla_prefill_fwd against the
    separate kernels of linattn_prefill_fwd with log_alpha [B,H,L] (both to the oracle's bound)."""
    cfg = _cfg("gla_equal_gates", 2, 2, 500, 128, "bf16", 7700, gate_dist="config").with_(gates=True)
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    la_vec = np.repeat(x["log_alpha"][..., None], 128, axis=-1)
    q, k, v, lad, h0 = _dev(cfg, x, la_vec)
    o1, h1 = ops.gla_prefill_fwd(q, k, v, lad, h0)
    o2, h2 = ops.linattn_prefill_fwd(q, k, v, h0, log_alpha=dev_tensor(x["log_alpha"], torch.float32))
    torch.cuda.synchronize()
    ro, rh = oracle.gla_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
    _check(cfg.with_(name="gla_equal_gates per-dimension kernels"), o1, h1, ro, rh)
    _check(cfg.with_(name="gla_equal_gates per-token kernels"), o2, h2, ro, rh)
    assert max_rel_err(host(o1), host(o2)) <= TOL_BF16


def test_gla_million_token_sequence_window():
    """A gate per key dimension (long-memory gates) over one slice of 2^20 + 37 tokens: the last W
    tokens' outputs and the final state against the oracle started from a prefix call's final
    state, and the two calls' prefix outputs against each other."""
    L, W = 2 ** 20 + 37, 64 * 64 + 37
    cfg = _cfg("gla_1m", 1, 1, L, 128, "bf16", 71, gate_dist="long")
    say(f"case {cfg.name}: inputs")
    s = inputs.prefill_slice(cfg, 0, 0)
    la_np = inputs.gate_vectors(cfg)[0, 0]
    t = lambda a, d: dev_tensor(a[None, None], d)
    q, k, v = t(s["q"], torch.bfloat16), t(s["k"], torch.bfloat16), t(s["v"], torch.bfloat16)
    la = t(la_np, torch.float32)
    h0 = t(s["h0"], torch.float32)
    say(f"case {cfg.name}: GPU, whole sequence and prefix")
    o, hf = ops.gla_prefill_fwd(q, k, v, la, h0)
    P = L - W
    pre = lambda x: x[:, :, :P].contiguous()
    o_p, h_p = ops.gla_prefill_fwd(pre(q), pre(k), pre(v), pre(la), h0)
    torch.cuda.synchronize()
    win = lambda a: a[P:][None, None]
    say(f"case {cfg.name}: oracle over the last {W} tokens")
    ro, rh = oracle.gla_vec_prefill(win(s["q"]), win(s["k"]), win(s["v"]), win(la_np), host(h_p))
    eo, eh = max_rel_err(host(o[:, :, P:]), ro), max_rel_err(host(hf), rh)
    say(f"  window: max rel err o {eo:.3e}, h_final {eh:.3e}")
    assert eo <= TOL_BF16 and eh <= TOL_BF16
    e = max_rel_err(host(o_p), host(o[:, :, :P]))
    say(f"  prefix outputs of the two calls: max rel diff {e:.3e}")
    assert e <= TOL_BF16
