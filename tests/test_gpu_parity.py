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
from gpu_util import TOL_BF16, TOL_F32, dev_tensor, host, max_rel_err, prefill_workspace, say

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
    """h_final may be h0 itself; two calls chained through the state reproduce one long call
    (to rounding: the calls split their sequences into blocks differently) and the oracle."""
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
    ro, rh = _oracle(x)
    o_chain = host(torch.cat([o1, o2], dim=2))
    _check(o_chain, host(h), ro, rh, TOL_BF16, "chained, in place")
    assert max_rel_err(o_chain, host(o_full)) < 1e-2 and max_rel_err(host(h), host(hf_full)) < 1e-2


@pytest.mark.parametrize("D", [64, 128])
def test_block_counts_match_the_oracle(D):
    """The sequence split into 1 (no workspace), 2, 3, 5 and 14 blocks (one per chunk) with a ragged
    tail; every split agrees with the oracle, and a repeated call is bitwise identical."""
    cfg = inputs.GDN_32K.with_(name=f"blocks_d{D}", B=1, H=3, L=64 * 13 + 5, Dk=D, Dv=D, seed=31, gate_dist="long")
    x = inputs.prefill_inputs(cfg)
    dt = torch.bfloat16
    q, k, v = (dev_tensor(x[n], dt) for n in ("q", "k", "v"))
    h0 = dev_tensor(x["h0"], torch.float32)
    args = (dev_tensor(x["beta"], torch.float32), dev_tensor(x["log_alpha"], torch.float32))
    ro, rh = _oracle(x)
    for nb in (1, 2, 3, 5, 14):
        say(f"case {cfg.name}: {nb} blocks per slice")
        ws = prefill_workspace(torch, 1, 3, D, nb) if nb > 1 else None
        o1, h1 = ops.gdn_prefill_fwd(q, k, v, *args, h0, workspace=ws)
        o2, h2 = ops.gdn_prefill_fwd(q, k, v, *args, h0, workspace=ws)
        torch.cuda.synchronize()
        _check(host(o1), host(h1), ro, rh, TOL_BF16, f"{nb} blocks")
        assert torch.equal(o1, o2) and torch.equal(h1, h2), nb


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_blocks_that_forget_partway(dtype):
    """Long-memory gates except one chunk of strong decay (log a = -3 per token, a chunk product
    of e^-192, which is 0 in fp32) at a different place in each block: a block's map is complete
    once its composed transition is exactly zero, which here happens after 1, 2, 3 or 4 of its
    chunk pairs (or never, in the block without such a chunk). Every split matches the oracle and
    the one-block sequential pass, which composes no maps."""
    cfg = inputs.GDN_32K.with_(name=f"forget_{dtype}", B=1, H=2, L=64 * 47 + 9, dtype=dtype, seed=43,
                               gate_dist="long")
    x = inputs.prefill_inputs(cfg)
    la = x["log_alpha"].copy()
    # 48 chunks, 6 blocks of 8 (the last chunk ragged), each block's chunks taken in pairs from its
    # end: the decaying chunk sits at offset 7, 5, 3, 1 and 6 of blocks 0..4; block 5 has none
    for blk, off in zip(range(5), (7, 5, 3, 1, 6)):
        c = 8 * blk + off
        la[:, :, 64 * c:64 * c + 64] = -3.0
    x["log_alpha"] = la
    dt = TD[dtype]
    q, k, v = (dev_tensor(x[n], dt) for n in ("q", "k", "v"))
    h0 = dev_tensor(x["h0"], torch.float32)
    beta, lad = dev_tensor(x["beta"], torch.float32), dev_tensor(la, torch.float32)
    ro, rh = _oracle(x)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for nb in (1, 6, 7):
        say(f"case {cfg.name}: {nb} blocks")
        ws = prefill_workspace(torch, 1, 2, 128, nb) if nb > 1 else None
        o, hf = ops.gdn_prefill_fwd(q, k, v, beta, lad, h0, workspace=ws)
        torch.cuda.synchronize()
        _check(host(o), host(hf), ro, rh, tol, f"{nb} blocks")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_very_negative_gates(dtype):
    """Finite log gates far below the others at single tokens (-1e6, -1e3 and -200, below the
    -110 floor; -60, above it) and a run of -30 whose sum passes -110 inside a chunk, among
    long-memory gates, in one and several blocks: factors over an interval holding such a gate
    are exactly zero and the later cumulative sums keep their precision. Against the oracle, which
    forms exp(-1e6) = 0 in fp64."""
    cfg = inputs.GDN_32K.with_(name=f"neg_gates_{dtype}", B=1, H=2, L=64 * 9 + 17, dtype=dtype, seed=49,
                               gate_dist="long")
    x = inputs.prefill_inputs(cfg)
    la = x["log_alpha"].copy()
    la[0, 0, [5, 130, 300]] = [-1e6, -1e3, -200.0]
    la[0, 1, [64, 200]] = [-60.0, -1e6]
    la[0, 1, 450:460] = -30.0
    x["log_alpha"] = la
    dt = TD[dtype]
    q, k, v = (dev_tensor(x[n], dt) for n in ("q", "k", "v"))
    h0 = dev_tensor(x["h0"], torch.float32)
    beta, lad = dev_tensor(x["beta"], torch.float32), dev_tensor(la, torch.float32)
    ro, rh = _oracle(x)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for nb in (1, 4):
        say(f"case {cfg.name}: {nb} blocks")
        ws = prefill_workspace(torch, 1, 2, 128, nb) if nb > 1 else None
        o, hf = ops.gdn_prefill_fwd(q, k, v, beta, lad, h0, workspace=ws)
        torch.cuda.synchronize()
        _check(host(o), host(hf), ro, rh, tol, f"{nb} blocks")


@pytest.mark.parametrize("B,H,L,D,seed,h0", [(1, 2, 118, 64, 9026, None), (2, 1, 104, 128, 9784, 0.1),
                                               (2, 2, 64 * 12 + 31, 64, 10023, 0.1)])
def test_strong_decay_fp32(B, H, L, D, seed, h0):
    """Per-token gates of -U(0, 40), fp32 inputs: a chunk's cumulative log gates reach about
    -1,300, where one fp32 ulp is about 1e-4, so plain differences of them carried the final state
    or the outputs past the 1e-4 bound (1.1e-4 to 1.5e-4 on these inputs, found by a random
    sweep); the kernels keep each sum as an exact hi + lo pair for fp32 inputs. Dense in one and
    several blocks, and the block-adjacent solve at bands 1 and 2."""
    cfg = inputs.GDN_32K.with_(name=f"strong_f32_B{B}H{H}L{L}d{D}", B=B, H=H, L=L, Dk=D, Dv=D, dtype="f32",
                               seed=seed, gate_dist="very_strong", h0=h0)
    x = inputs.prefill_inputs(cfg)
    q, k, v = (dev_tensor(x[n], torch.float32) for n in ("q", "k", "v"))
    hd = dev_tensor(x["h0"], torch.float32) if h0 is not None else None
    beta, la = dev_tensor(x["beta"], torch.float32), dev_tensor(x["log_alpha"], torch.float32)
    ro, rh = _oracle(x)
    for nb in (1, 3):
        say(f"case {cfg.name}: {nb} blocks")
        ws = prefill_workspace(torch, B, H, D, nb) if nb > 1 else None
        o, hf = ops.gdn_prefill_fwd(q, k, v, beta, la, hd, workspace=ws)
        torch.cuda.synchronize()
        _check(host(o), host(hf), ro, rh, TOL_F32, f"{nb} blocks")
    for band in (1, 2):
        say(f"case {cfg.name}: band {band}")
        o, hf = ops.gdn_prefill_banded_fwd(q, k, v, beta, la, hd, band=band)
        torch.cuda.synchronize()
        bo, bh = oracle.gdn_prefill_banded(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], x["h0"], band=band)
        _check(host(o), host(hf), bo, bh, TOL_F32, f"band {band}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_gates_reset_the_state(dtype):
    """log a = -inf (a zero gate) clears the state before the token's write; the cumulative gate
    sums cannot be differenced across it. Zero gates at chunk starts, ends and inside chunks, in
    several blocks, with h0, against the oracle (which computes a = exp(-inf) = 0 exactly)."""
    cfg = inputs.GDN_32K.with_(name=f"reset_{dtype}", B=1, H=2, L=64 * 9 + 17, dtype=dtype, seed=41, gate_dist="long")
    x = inputs.prefill_inputs(cfg)
    la = x["log_alpha"].copy()
    for t in (0, 5, 63, 64, 100, 101, 250, 383, 511, 590):
        la[:, 0, t] = -np.inf
    la[:, 1, 300] = -np.inf
    x["log_alpha"] = la
    dt = TD[dtype]
    q, k, v = (dev_tensor(x[n], dt) for n in ("q", "k", "v"))
    h0 = dev_tensor(x["h0"], torch.float32)
    beta, lad = dev_tensor(x["beta"], torch.float32), dev_tensor(la, torch.float32)
    ro, rh = _oracle(x)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for nb in (1, 4):
        say(f"case {cfg.name}: {nb} blocks")
        ws = prefill_workspace(torch, 1, 2, 128, nb) if nb > 1 else None
        o, hf = ops.gdn_prefill_fwd(q, k, v, beta, lad, h0, workspace=ws)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all() and torch.isfinite(hf).all()
        _check(host(o), host(hf), ro, rh, tol, f"{nb} blocks")


def test_map_waves_with_zero_columns():
    """A zero gate on a block's last token with that token's key zero in key dimensions 0-15 (the
    columns of Z that the map's first wave holds, at d = 128 in bf16): after the block's last
    chunk only that wave's columns of Z are exactly zero, so it alone skips the second chunk of
    the pair while the other waves apply it. Head 1 zeroes dimensions 16-47 instead (two waves).
    Three blocks of four chunks against the oracle and against the one-block sequential pass."""
    cfg = inputs.GDN_32K.with_(name="map_zero_columns", B=1, H=2, L=64 * 12, seed=47, gate_dist="long")
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    la, kk = x["log_alpha"].copy(), x["k"].copy()
    for c in (3, 7, 11):   # the last chunk of each block of four
        t = 64 * c + 63
        la[0, :, t] = -np.inf
        kk[0, 0, t, 0:16] = 0.0
        kk[0, 1, t, 16:48] = 0.0
    x["log_alpha"], x["k"] = la, kk
    q, k, v = (dev_tensor(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    h0 = dev_tensor(x["h0"], torch.float32)
    beta, lad = dev_tensor(x["beta"], torch.float32), dev_tensor(la, torch.float32)
    ro, rh = _oracle(x)
    res = {}
    for nb in (1, 3):
        ws = prefill_workspace(torch, 1, 2, 128, nb) if nb > 1 else None
        o, hf = ops.gdn_prefill_fwd(q, k, v, beta, lad, h0, workspace=ws)
        torch.cuda.synchronize()
        res[nb] = (host(o), host(hf))
        _check(res[nb][0], res[nb][1], ro, rh, TOL_BF16, f"{nb} blocks")
    # the split changes only the order of fp32 sums
    assert max_rel_err(res[3][0], res[1][0]) <= 1e-2 and max_rel_err(res[3][1], res[1][1]) <= 1e-2


def test_many_blocks_mixed_maps():
    """70 blocks of two chunks in one slice, every third block with long-memory gates (its map is
    not zero) and the others with the configured strong decay (map exactly zero after one
    chunk): the pass over blocks reads the zero flags in groups of 64, and the mix of skipped and
    applied maps crosses the group boundary. Against the oracle and the one-block pass."""
    cfg = inputs.GDN_32K.with_(name="many_blocks", B=1, H=1, L=64 * 140, seed=53)
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    la = x["log_alpha"].copy()
    rng = np.random.default_rng(54)
    for blk in range(0, 70, 3):
        t0 = 128 * blk
        la[0, 0, t0:t0 + 128] = (-rng.uniform(0.0, 0.01, 128)).astype(np.float32)
    x["log_alpha"] = la
    q, k, v = (dev_tensor(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    h0 = dev_tensor(x["h0"], torch.float32)
    beta, lad = dev_tensor(x["beta"], torch.float32), dev_tensor(la, torch.float32)
    ro, rh = _oracle(x)
    res = {}
    for nb in (1, 70):
        ws = prefill_workspace(torch, 1, 1, 128, nb) if nb > 1 else None
        o, hf = ops.gdn_prefill_fwd(q, k, v, beta, lad, h0, workspace=ws)
        torch.cuda.synchronize()
        res[nb] = (host(o), host(hf))
        _check(res[nb][0], res[nb][1], ro, rh, TOL_BF16, f"{nb} blocks")
    assert max_rel_err(res[70][0], res[1][0]) <= 1e-2 and max_rel_err(res[70][1], res[1][1]) <= 1e-2



def test_many_blocks_mixed_maps_eight_slices():
    """Eight slices (B=2, H=4: the pass over blocks then runs each slice's value tiles together on
    one XCD and loads the next live block's map during the current product) of 70 blocks of two
    chunks, each slice with its own pattern of long-memory blocks (maps not zero) among strongly
    decaying ones (maps exactly zero): every block live in one slice, none in another, every
    k-th block in the rest, so live blocks follow live, skipped and reloaded blocks and cross the
    64-flag group boundary. Against the oracle and the one-block pass."""
    cfg = inputs.GDN_32K.with_(name="many_blocks_8", B=2, H=4, L=64 * 140, seed=57)
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    la = x["log_alpha"].copy()
    rng = np.random.default_rng(58)
    for sl, every in enumerate((1, 0, 2, 3, 5, 7, 11, 64)):
        b, h = divmod(sl, 4)
        for blk in range(70):
            if every and blk % every == 0:
                la[b, h, 128 * blk:128 * blk + 128] = (-rng.uniform(0.0, 0.01, 128)).astype(np.float32)
    x["log_alpha"] = la
    q, k, v = (dev_tensor(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    h0 = dev_tensor(x["h0"], torch.float32)
    beta, lad = dev_tensor(x["beta"], torch.float32), dev_tensor(la, torch.float32)
    ro, rh = _oracle(x)
    res = {}
    for nb in (1, 70):
        ws = prefill_workspace(torch, 2, 4, 128, nb) if nb > 1 else None
        o, hf = ops.gdn_prefill_fwd(q, k, v, beta, lad, h0, workspace=ws)
        torch.cuda.synchronize()
        res[nb] = (host(o), host(hf))
        _check(res[nb][0], res[nb][1], ro, rh, TOL_BF16, f"{nb} blocks")
    assert max_rel_err(res[70][0], res[1][0]) <= 1e-2 and max_rel_err(res[70][1], res[1][1]) <= 1e-2

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


def test_gdn_32k_full_workload_all_heads():
    cfg = inputs.GDN_32K
    o, hf, ro, rh = _full_size(cfg, [(0, h) for h in range(cfg.H)])
    _check(o, hf, ro, rh, TOL_BF16, cfg.name)


def test_gdn_32k_long_memory_gates_sampled():
    """log a ~ -U(0, 0.01): the state carries information across the whole 512-chunk chain."""
    cfg = inputs.GDN_32K.with_(name="gdn_32k_long_memory", gate_dist="long")
    o, hf, ro, rh = _full_size(cfg, [(0, 3)])
    _check(o, hf, ro, rh, TOL_BF16, cfg.name)


def test_gdn_128k_full_workload_all_heads():
    """The headline workload in the launch bench.py times (the preferred workspace: 32 blocks per
    head), every head's outputs and final state against the oracle's whole sequence."""
    cfg = inputs.GDN_128K
    o, hf, ro, rh = _full_size(cfg, [(0, h) for h in range(cfg.H)])
    _check(o, hf, ro, rh, TOL_BF16, cfg.name)


def test_gdn_128k_long_memory_gates_all_heads():
    """log a ~ -U(0, 0.01) at 128K: the state carries information across the whole 2048-chunk
    sequence, each block's map composes all 64 of its chunks and the pass over blocks multiplies
    31 of them, so rounding errors can accumulate."""
    cfg = inputs.GDN_128K.with_(name="gdn_128k_long_memory", gate_dist="long")
    o, hf, ro, rh = _full_size(cfg, [(0, h) for h in range(cfg.H)])
    _check(o, hf, ro, rh, TOL_BF16, cfg.name)



@pytest.mark.parametrize("gate_dist", ["config", "long"])
def test_gdn_million_token_sequence_window(gate_dist):
    """One slice of 2^20 + 37 tokens (16,385 chunks, the last ragged; about 500 blocks and a pass
    over blocks spanning eight 64-flag groups): token offsets and block indices far beyond the
    other workloads'. The whole sequence runs once and its first L - W tokens once more; the
    oracle, started from the second call's final state, recomputes the last W tokens, which must
    match the first call's outputs there and its final state, and the two calls' outputs agree on
    the shared prefix (their blocks split it differently)."""
    L, W = 2 ** 20 + 37, 64 * 64 + 37
    cfg = inputs.GDN_128K.with_(name=f"gdn_1m_{gate_dist}", H=1, L=L, seed=61, gate_dist=gate_dist)
    say(f"case {cfg.name}: inputs")
    s = inputs.prefill_slice(cfg, 0, 0)
    dt = TD[cfg.dtype]
    t = lambda a, d: dev_tensor(a[None, None], d)
    q, k, v = t(s["q"], dt), t(s["k"], dt), t(s["v"], dt)
    beta, la, h0 = t(s["beta"], torch.float32), t(s["log_alpha"], torch.float32), t(s["h0"], torch.float32)
    say(f"case {cfg.name}: GPU, whole sequence and prefix")
    o, hf = ops.gdn_prefill_fwd(q, k, v, beta, la, h0)
    P = L - W
    pre = lambda x: x[:, :, :P].contiguous()
    o_p, h_p = ops.gdn_prefill_fwd(pre(q), pre(k), pre(v), pre(beta), pre(la), h0)
    torch.cuda.synchronize()
    win = lambda a: a[P:][None, None]
    say(f"case {cfg.name}: oracle over the last {W} tokens")
    ro, rh = oracle.gdn_prefill(win(s["q"]), win(s["k"]), win(s["v"]), win(s["beta"]), win(s["log_alpha"]),
                                host(h_p))
    _check(host(o[:, :, P:]), host(hf), ro, rh, TOL_BF16, f"{cfg.name} window")
    e = max_rel_err(host(o_p), host(o[:, :, :P]))
    say(f"  prefix outputs of the two calls: max rel diff {e:.3e}")
    assert e <= TOL_BF16


@pytest.mark.parametrize("gated", [False, True])
def test_linattn_million_token_sequence_window(gated):
    """Linear attention, plain and with a per-token decay (long-memory gates), over one slice of
    2^20 + 37 tokens: the last W tokens' outputs and the final state against the oracle started
    from a prefix call's final state, and the two calls' prefix outputs against each other."""
    L, W = 2 ** 20 + 37, 64 * 64 + 37
    cfg = inputs.LINATTN_8K.with_(name=f"la_1m_{'gated' if gated else 'plain'}", B=1, H=1, L=L, seed=67,
                                  gates=gated, gate_dist="long")
    say(f"case {cfg.name}: inputs")
    s = inputs.prefill_slice(cfg, 0, 0)
    dt = TD[cfg.dtype]
    t = lambda a, d: None if a is None else dev_tensor(a[None, None], d)
    q, k, v = t(s["q"], dt), t(s["k"], dt), t(s["v"], dt)
    la = t(s["log_alpha"], torch.float32)
    say(f"case {cfg.name}: GPU, whole sequence and prefix")
    o, hf = ops.linattn_prefill_fwd(q, k, v, None, log_alpha=la)
    P = L - W
    pre = lambda x: None if x is None else x[:, :, :P].contiguous()
    o_p, h_p = ops.linattn_prefill_fwd(pre(q), pre(k), pre(v), None, log_alpha=pre(la))
    torch.cuda.synchronize()
    win = lambda a: a[P:][None, None]
    say(f"case {cfg.name}: oracle over the last {W} tokens")
    if gated:
        ro, rh = oracle.gla_prefill(win(s["q"]), win(s["k"]), win(s["v"]), win(s["log_alpha"]), host(h_p))
    else:
        ro, rh = oracle.linattn_prefill(win(s["q"]), win(s["k"]), win(s["v"]), host(h_p))
    _check(host(o[:, :, P:]), host(hf), ro, rh, TOL_BF16, f"{cfg.name} window")
    e = max_rel_err(host(o_p), host(o[:, :, :P]))
    say(f"  prefix outputs of the two calls: max rel diff {e:.3e}")
    assert e <= TOL_BF16

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


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_extreme_gates(dtype):
    """Decode steps where some (sequence, head) pairs take a zero gate (log a = -inf), a gate of
    -1e6 or a gate of 0 (a = 1), beta of 0 or 1, against the oracle step by step."""
    cfg = inputs.DECODE_256x32.with_(name=f"decode_gates_{dtype}", N=4, H=4, Dk=128, Dv=128, dtype=dtype, seed=6100)
    dt = TD[dtype]
    st = inputs.decode_state(cfg)
    state = dev_tensor(st, torch.float32)
    ref = st.copy()
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    say(f"case {cfg.name}")
    for step in range(6):
        x = inputs.decode_token(cfg, step)
        la, beta = x["log_alpha"].copy(), x["beta"].copy()
        la[step % 4, 0] = -np.inf
        la[(step + 1) % 4, 1] = -1e6
        la[(step + 2) % 4, 2] = 0.0
        beta[(step + 3) % 4, 3] = 0.0
        beta[step % 4, 3] = 1.0
        args = [dev_tensor(x[n], dt) for n in ("q", "k", "v")] + [dev_tensor(beta, torch.float32),
                                                                 dev_tensor(la, torch.float32)]
        o = ops.gdn_decode_step(*args, state)
        ro, ref = oracle.gdn_decode_step(x["q"], x["k"], x["v"], beta, la, ref)
        torch.cuda.synchronize()
        eo = max_rel_err(host(o)[:, :, None], ro[:, :, None])
        assert eo <= tol, (step, eo)
    eh = max_rel_err(host(state), ref)
    say(f"  state after 6 steps: max rel err {eh:.3e}")
    assert eh <= tol

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


def test_many_slices_one_block_each():
    """B=8, H=40: 320 (batch, head) slices, more than the device has CUs, so the call takes no
    workspace and runs one output workgroup per slice over its whole sequence (no maps, no pass
    over blocks); sampled slices in every batch against the oracle."""
    cfg = inputs.GDN_32K.with_(name="many_slices", B=8, H=40, L=64 * 3 + 11, seed=59)
    say(f"case {cfg.name}")
    o, hf, ro, rh = _full_size(cfg, [(b, (7 * b) % 40) for b in range(8)] + [(7, 39)])
    _check(o, hf, ro, rh, TOL_BF16, cfg.name)

def test_preferred_workspace_follows_the_device():
    """The preferred workspace gives about two output workgroups per CU of this device, and none
    once the (batch, head) slices alone give every CU one."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nb = -(-2 * cus // 16)
    flags = ((nb - 1) * 4 + 255) // 256 * 256
    assert ops.prefill_workspace_size(1, 16, 131072, 128, torch.bfloat16) == 16 * ((2 * nb - 1) * 4 * 128 * 128 + flags)
    assert ops.prefill_workspace_size(1, cus, 4096, 128, torch.bfloat16) == 0


def test_fp32_gate_factors_exact_under_strong_decay():
    """One chunk of 64 tokens with log a ~ -U(0, 40) and beta zero before the last token: the final
    state is then beta_C k_C v_C^T (key-major) and every gate factor that reaches it is e^0 = 1.
    fp32 inputs must give it to rounding (bound 1e-5, ten times under the fp32 path's 1e-4):
    cumulative gate sums of ~10^3 kept as exact hi + lo pairs leave that factor exactly 1, but one
    unrounded product inside the pair's bookkeeping (floating-point contraction) made it
    e^{+-half an ulp of the sums}, 7.5e-5 off."""
    cfg = inputs.GDN_32K.with_(name="fp32_last_token_factor", B=1, H=3, L=64, dtype="f32", seed=9354,
                               gate_dist="very_strong", h0=None)
    x = inputs.prefill_inputs(cfg)
    beta = x["beta"].copy()
    beta[..., :-1] = 0.0
    say(f"case {cfg.name}")
    d = {n: dev_tensor(x[n], torch.float32) for n in ("q", "k", "v", "log_alpha")}
    o, hf = ops.gdn_prefill_fwd(d["q"], d["k"], d["v"], dev_tensor(beta, torch.float32), d["log_alpha"], None)
    torch.cuda.synchronize()
    ro, rh = oracle.gdn_prefill(x["q"], x["k"], x["v"], beta, x["log_alpha"], None)
    _check(host(o), host(hf), ro, rh, 1e-5, cfg.name)
