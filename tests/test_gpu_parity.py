"""Parity of the HIP path (through the C ABI) with the fp64 oracle on identical seeded inputs.

Error metric: max |gpu - oracle| / max |oracle| per (b, h) slice, maximised over slices, for the
outputs and for the final state separately. Bounds: 2e-2 on bf16-input paths, 1e-4 on fp32.
Full-size workloads run the whole GPU launch and compare sampled heads, whose whole sequence
the oracle recomputes.
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


def _run_prefill(cfg, x, gdn=True, h0_dev="auto"):
    dt = TD[cfg.dtype]
    q, k, v = (dev_tensor(x[n], dt) for n in ("q", "k", "v"))
    h0 = dev_tensor(x["h0"], torch.float32) if h0_dev == "auto" else h0_dev
    if gdn:
        beta = dev_tensor(x["beta"], torch.float32)
        la = dev_tensor(x["log_alpha"], torch.float32)
        o, hf = ops.gdn_prefill_fwd(q, k, v, beta, la, h0)
    else:
        o, hf = ops.linattn_prefill_fwd(q, k, v, h0)
    torch.cuda.synchronize()
    return host(o), host(hf)


def _oracle(x, gdn=True, sl=(slice(None), slice(None))):
    g = lambda key: None if x[key] is None else x[key][sl]
    if gdn:
        return oracle.gdn_prefill(g("q"), g("k"), g("v"), g("beta"), g("log_alpha"), g("h0"))
    return oracle.linattn_prefill(g("q"), g("k"), g("v"), g("h0"))


def _check(o, hf, ro, rh, tol, what):
    eo, eh = max_rel_err(o, ro), max_rel_err(hf, rh)
    say(f"  {what}: max rel err o {eo:.3e}, h_final {eh:.3e} (bound {tol:g})")
    assert eo <= tol and eh <= tol, (eo, eh)


# ---------------------------------------------------------------------------------------------
# small and ragged shapes, whole-tensor comparison
# ---------------------------------------------------------------------------------------------
def test_gdn_fp32_reference_workload():
    cfg = inputs.GDN_REF_FP32
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    o, hf = _run_prefill(cfg, x)
    ro, rh = _oracle(x)
    _check(o, hf, ro, rh, TOL_F32, cfg.name)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("L", [1, 63, 64, 65, 200, 1000])
def test_gdn_bf16_ragged(L, D):
    cfg = inputs.GDN_32K.with_(name=f"gdn_bf16_L{L}_d{D}", B=2, H=3, L=L, Dk=D, Dv=D, seed=2000 + L + D)
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    o, hf = _run_prefill(cfg, x)
    ro, rh = _oracle(x)
    _check(o, hf, ro, rh, TOL_BF16, cfg.name)


@pytest.mark.parametrize("gate_dist", ["config", "long"])
@pytest.mark.parametrize("D", [64, 128])
def test_gdn_fp32_paths(D, gate_dist):
    cfg = inputs.GDN_32K.with_(name=f"gdn_f32_d{D}_{gate_dist}", B=1, H=2, L=333, Dk=D, Dv=D, dtype="f32",
                               seed=3000 + D, gate_dist=gate_dist)
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    o, hf = _run_prefill(cfg, x)
    ro, rh = _oracle(x)
    _check(o, hf, ro, rh, TOL_F32, cfg.name)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("L,with_h0", [(1, False), (100, True), (640, False), (1000, True)])
def test_linattn_ragged(L, with_h0, D, dtype):
    cfg = inputs.LINATTN_8K.with_(name=f"la_L{L}_d{D}_{dtype}", B=1, H=2, L=L, Dk=D, Dv=D, dtype=dtype,
                                  seed=4000 + L + D, h0=0.1 if with_h0 else None)
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    o, hf = _run_prefill(cfg, x, gdn=False)
    ro, rh = _oracle(x, gdn=False)
    _check(o, hf, ro, rh, TOL_BF16 if dtype == "bf16" else TOL_F32, cfg.name)


# ---------------------------------------------------------------------------------------------
# exact cases and edge cases
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("D", [64, 128])
def test_standard_basis_keys_retrieve_exactly(D):
    """Keys e_1 .. e_D (exact in bf16), beta = 1, alpha = 1: T = I, every write lands in its own
    key row, so o_t = v_t and the final state's row i is v_i, bit for bit."""
    L = D
    k = np.eye(D)[None, None]
    v = inputs.round_bf16(np.random.default_rng(D).standard_normal((1, 1, L, D)))
    kk = dev_tensor(k, torch.bfloat16)
    vv = dev_tensor(v, torch.bfloat16)
    beta = torch.ones((1, 1, L), device="cuda")
    la = torch.zeros((1, 1, L), device="cuda")
    say(f"case basis_keys_d{D}")
    o, hf = ops.gdn_prefill_fwd(kk, kk, vv, beta, la)
    torch.cuda.synchronize()
    assert torch.equal(o, vv)
    assert torch.equal(hf[0, 0], vv[0, 0].float())


def test_zero_length_copies_state():
    h0 = torch.randn((2, 3, 128, 128), device="cuda")
    q = torch.empty((2, 3, 0, 128), device="cuda", dtype=torch.bfloat16)
    beta = torch.empty((2, 3, 0), device="cuda")
    say("case L=0")
    o, hf = ops.gdn_prefill_fwd(q, q.clone(), q.clone(), beta, beta.clone(), h0)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(hf, h0)
    o, hf = ops.linattn_prefill_fwd(q, q.clone(), q.clone())
    torch.cuda.synchronize()
    assert torch.equal(hf, torch.zeros_like(hf))


def test_in_place_state_and_chaining():
    """h_final may be h0 itself; two calls chained through the state equal one long call."""
    cfg = inputs.GDN_32K.with_(name="chain", B=1, H=2, L=300, seed=77)
    x = inputs.prefill_inputs(cfg)
    dt = torch.bfloat16
    q, k, v = (dev_tensor(x[n], dt) for n in ("q", "k", "v"))
    beta, la = dev_tensor(x["beta"], torch.float32), dev_tensor(x["log_alpha"], torch.float32)
    h = dev_tensor(x["h0"], torch.float32)
    say("case in-place chaining")
    o_full, hf_full = ops.gdn_prefill_fwd(q, k, v, beta, la, h)
    a, b = slice(0, 128), slice(128, 300)
    part = lambda t, s: t[:, :, s].contiguous()
    o1, _ = ops.gdn_prefill_fwd(part(q, a), part(k, a), part(v, a), part(beta, a), part(la, a), h, h_final=h)
    o2, _ = ops.gdn_prefill_fwd(part(q, b), part(k, b), part(v, b), part(beta, b), part(la, b), h, h_final=h)
    torch.cuda.synchronize()
    # chunk boundaries coincide (128 is a multiple of 64), so the arithmetic is identical
    assert torch.equal(torch.cat([o1, o2], dim=2), o_full)
    assert torch.equal(h, hf_full)


def test_segmented_schedule_is_bitwise_identical():
    """A small workspace forces many segments of the gated delta-rule prefill (stages overlapped on
    internal streams); every chunk computes exactly the same arithmetic, so the result equals the
    one-segment run. (Linear attention splits the sequence into blocks by workspace size instead,
    which changes the order of its sums: tests/test_gpu_linattn_blocks.py checks small workspaces
    against the oracle.)"""
    cfg = inputs.GDN_32K.with_(name="seg", B=1, H=3, L=64 * 13 + 5, seed=31)
    x = inputs.prefill_inputs(cfg)
    dt = torch.bfloat16
    q, k, v = (dev_tensor(x[n], dt) for n in ("q", "k", "v"))
    h0 = dev_tensor(x["h0"], torch.float32)
    args = (dev_tensor(x["beta"], torch.float32), dev_tensor(x["log_alpha"], torch.float32))
    fn = ops.gdn_prefill_fwd
    rec = ops.prefill_workspace_size(1, 1, 64, 128, dt) * cfg.H
    say("case segmented gdn")
    o1, h1 = fn(q, k, v, *args, h0)
    for seg in (1, 2, 5):   # segment length in chunks: two buffers of seg records and the counters
        ws = torch.empty(2 * seg * rec + 256, dtype=torch.uint8, device="cuda")
        o2, h2 = fn(q, k, v, *args, h0, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(h1, h2), seg


def test_deterministic():
    cfg = inputs.GDN_32K.with_(name="det", B=1, H=4, L=777, seed=5)
    x = inputs.prefill_inputs(cfg)
    say("case determinism")
    o1, h1 = _run_prefill(cfg, x)
    o2, h2 = _run_prefill(cfg, x)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)


# ---------------------------------------------------------------------------------------------
# full-size workloads (launch as timed), sampled slices against the oracle
# ---------------------------------------------------------------------------------------------
def _full_size(cfg, sample, gdn=True):
    """Run the whole [B,H,L] launch; return GPU results for the sampled (b, h) slices and the
    oracle's for the same slices."""
    dt = TD[cfg.dtype]
    shp = (cfg.B, cfg.H, cfg.L)
    q = torch.empty(shp + (cfg.Dk,), dtype=dt, device="cuda")
    k, v = torch.empty_like(q), torch.empty_like(q)
    beta = torch.empty(shp, device="cuda") if gdn else None
    la = torch.empty(shp, device="cuda") if gdn else None
    h0 = torch.empty((cfg.B, cfg.H, cfg.Dk, cfg.Dv), device="cuda") if cfg.h0 is not None else None
    kept = {}
    for b in range(cfg.B):
        for h in range(cfg.H):
            s = inputs.prefill_slice(cfg, b, h)
            for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("log_alpha", la), ("h0", h0)):
                if t is not None:
                    t[b, h] = dev_tensor(s[name], t.dtype)
            if (b, h) in sample:
                kept[(b, h)] = s
    say(f"case {cfg.name}: GPU launch")
    if gdn:
        o, hf = ops.gdn_prefill_fwd(q, k, v, beta, la, h0)
    else:
        o, hf = ops.linattn_prefill_fwd(q, k, v, h0)
    torch.cuda.synchronize()
    got_o = np.stack([host(o[b, h]) for (b, h) in sample])[None]
    got_h = np.stack([host(hf[b, h]) for (b, h) in sample])[None]
    st = lambda key: None if kept[sample[0]][key] is None else np.stack([kept[s][key] for s in sample])[None]
    say(f"case {cfg.name}: oracle on {len(sample)} slices")
    if gdn:
        ro, rh = oracle.gdn_prefill(st("q"), st("k"), st("v"), st("beta"), st("log_alpha"), st("h0"))
    else:
        ro, rh = oracle.linattn_prefill(st("q"), st("k"), st("v"), st("h0"))
    return got_o, got_h, ro, rh


def test_linattn_full_workload_sampled():
    cfg = inputs.LINATTN_8K
    o, hf, ro, rh = _full_size(cfg, [(0, 0), (1, 7), (3, 15)], gdn=False)
    _check(o, hf, ro, rh, TOL_BF16, cfg.name)


def test_gdn_32k_full_workload_sampled():
    cfg = inputs.GDN_32K
    o, hf, ro, rh = _full_size(cfg, [(0, 0), (0, 31)])
    _check(o, hf, ro, rh, TOL_BF16, cfg.name)


def test_gdn_32k_long_memory_gates_sampled():
    """log a ~ -U(0, 0.01): the state carries information across the whole 512-chunk chain."""
    cfg = inputs.GDN_32K.with_(name="gdn_32k_long_memory", gate_dist="long")
    o, hf, ro, rh = _full_size(cfg, [(0, 3)])
    _check(o, hf, ro, rh, TOL_BF16, cfg.name)


def test_gdn_128k_full_workload_sampled():
    cfg = inputs.GDN_128K
    o, hf, ro, rh = _full_size(cfg, [(0, 0), (0, 15)])
    _check(o, hf, ro, rh, TOL_BF16, cfg.name)


def test_gdn_128k_long_memory_gates_sampled():
    """log a ~ -U(0, 0.01) at 128K: the state carries information across the whole 2048-chunk
    chain (and 33 segments of the pipelined launch), so rounding errors can accumulate."""
    cfg = inputs.GDN_128K.with_(name="gdn_128k_long_memory", gate_dist="long")
    o, hf, ro, rh = _full_size(cfg, [(0, 9)])
    _check(o, hf, ro, rh, TOL_BF16, cfg.name)


# ---------------------------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------------------------
def _decode_run(cfg, steps, sample_n):
    dt = TD[cfg.dtype]
    st0 = inputs.decode_state(cfg)
    state = dev_tensor(st0, torch.float32)
    ref_state = st0[:sample_n].copy()
    errs_o = []
    for step in range(steps):
        x = inputs.decode_token(cfg, step)
        args = [dev_tensor(x[n], dt) for n in ("q", "k", "v")]
        args += [dev_tensor(x[n], torch.float32) for n in ("beta", "log_alpha")]
        o = ops.gdn_decode_step(*args, state)
        ro, ref_state = oracle.gdn_decode_step(x["q"][:sample_n], x["k"][:sample_n], x["v"][:sample_n],
                                               x["beta"][:sample_n], x["log_alpha"][:sample_n], ref_state)
        errs_o.append(max_rel_err(host(o[:sample_n]), ro, axes=(2,)))
    torch.cuda.synchronize()
    eh = max_rel_err(host(state[:sample_n]), ref_state)
    return max(errs_o), eh


def test_decode_full_workload_100_steps_sampled():
    cfg = inputs.DECODE_256x32
    say(f"case {cfg.name}: 100 in-place steps, oracle on 4 sequences x 32 heads")
    eo, eh = _decode_run(cfg, cfg.steps, 4)
    say(f"  max rel err o {eo:.3e}, state {eh:.3e}")
    assert eo <= TOL_BF16 and eh <= TOL_BF16


@pytest.mark.parametrize("D", [64, 128])
def test_decode_fp32(D):
    cfg = inputs.DECODE_256x32.with_(name=f"decode_f32_d{D}", N=8, H=4, Dk=D, Dv=D, dtype="f32", seed=6000 + D)
    say(f"case {cfg.name}")
    eo, eh = _decode_run(cfg, 20, 8)
    say(f"  max rel err o {eo:.3e}, state {eh:.3e}")
    assert eo <= TOL_F32 and eh <= TOL_F32


def test_decode_equals_prefill_of_one_token():
    cfg = inputs.GDN_32K.with_(name="one_token", B=1, H=4, L=1, seed=9)
    x = inputs.prefill_inputs(cfg)
    dt = torch.bfloat16
    # one sequence (N = B = 1) with H heads
    q, k, v = (dev_tensor(x[n][:, :, 0], dt) for n in ("q", "k", "v"))
    beta, la = (dev_tensor(x[n][:, :, 0], torch.float32) for n in ("beta", "log_alpha"))
    state = dev_tensor(x["h0"], torch.float32)
    say("case decode == prefill(L=1)")
    o_dec = ops.gdn_decode_step(q, k, v, beta, la, state)
    o_pf, hf = _run_prefill(cfg, x)
    torch.cuda.synchronize()
    assert max_rel_err(host(o_dec), o_pf[:, :, 0], axes=(2,)) < 1e-2
    assert max_rel_err(host(state), hf) < 1e-2


def test_preferred_workspace_whole_sequence_when_chain_fills_device():
    """With more (batch, head) slices than the sequential stage leaves CUs free for (32 heads at
    d = 128 on 256 CUs), the preferred workspace holds the whole sequence's records; with 16 heads
    it is two segment buffers."""
    rec = ops.prefill_workspace_size(1, 1, 64, 128, torch.bfloat16)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    full = ops.prefill_workspace_size(1, 32, 32768, 128, torch.bfloat16)
    if 8 * 4 * 8 >= cus:
        assert full == 512 * 32 * rec
    seg = ops.prefill_workspace_size(1, 16, 131072, 128, torch.bfloat16)
    assert seg < 2048 * 16 * rec and (seg - 256) % (2 * 16 * rec) == 0
