"""Seeded random shapes across every prefill entry point against the oracle.

Each case draws its entry point (gated delta rule dense, with skipped chunk updates or with the
block-adjacent solve; linear attention plain or with a per-token decay; a gate per key dimension;
bidirectional), dtype, d, B, H, L (short and up to 2,500 tokens), gate distribution, h0 and, for
the gated delta rule, a workspace of a random number of blocks. Error metric as elsewhere:
max |gpu - oracle| / max |oracle| per tensor, with the denominator at least 1e-30: a reference
wholly below fp32's range (a skipped last chunk after a decay of e^-256 leaves a final state
near 1e-112) is zero in fp32.

A second group draws from a wider distribution: also the no-allocation prefill and decode steps
(some heads with a zero gate, a gate of -1e6 or a gate of 1), gates down to log a ~ -U(0, 40) per
token or key dimension (where fp32 sums of the gates lose precision), and many slices (B H up to
240) with short sequences.
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_chunked_rule_amd import _lib, inputs
from gpu_util import TOL_BF16, TOL_F32, dev_tensor, host, prefill_workspace, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

from gated_deltanet_chunked_rule_amd import ops  # noqa: E402

TD = {"bf16": torch.bfloat16, "f32": torch.float32}


def _rel(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.abs(np.asarray(got, dtype=np.float64) - ref).max() / max(np.abs(ref).max(), 1e-30))


def _case(i):
    r = np.random.default_rng(31000 + i)
    kind = r.choice(["gdn", "gdn", "gdn", "skip", "band", "la", "lag", "gla", "bidir"])
    dtype = str(r.choice(["bf16", "bf16", "f32"]))
    D = int(r.choice([64, 128]))
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    L = int(r.choice([int(r.integers(1, 130)), int(r.integers(1, 2500))]))
    gate = str(r.choice(["config", "long", "strong"]))
    h0 = None if r.random() < 0.3 else 0.1
    name = f"{kind}_{dtype}_B{B}H{H}L{L}d{D}_{gate}_h0{h0 is not None}"
    base = inputs.LINATTN_8K if kind in ("la", "gla", "bidir") else inputs.GDN_32K
    cfg = base.with_(name=name, B=B, H=H, L=L, Dk=D, Dv=D, dtype=dtype, seed=32000 + i, gate_dist=gate, h0=h0,
                     gates=kind not in ("la", "gla", "bidir"))
    return r, kind, cfg


@pytest.mark.parametrize("i", range(120))
def test_random_case(i):
    r, kind, cfg = _case(i)
    say(f"case {i}: {cfg.name}")
    _check(r, kind, cfg)


def _case_wide(i):
    r = np.random.default_rng(33000 + i)
    kind = str(r.choice(["gdn", "gdn", "noalloc", "skip", "band", "la", "lag", "gla", "bidir", "decode"]))
    dtype = str(r.choice(["bf16", "bf16", "f32"]))
    D = int(r.choice([64, 128]))
    if r.random() < 0.7:
        B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
        L = int(r.choice([int(r.integers(1, 130)), int(r.integers(1, 4000)),
                          64 * int(r.integers(1, 20)) + int(r.integers(-1, 2))]))
    else:
        B, H = int(r.integers(1, 7)), int(r.integers(1, 41))
        L = int(r.integers(1, 300))
    L = max(L, 1)
    gate = str(r.choice(["config", "long", "strong", "very_strong"]))
    h0 = None if r.random() < 0.3 else 0.1
    name = f"{kind}_{dtype}_B{B}H{H}L{L}d{D}_{gate}_h0{h0 is not None}"
    base = inputs.LINATTN_8K if kind in ("la", "gla", "bidir") else inputs.GDN_32K
    cfg = base.with_(name=name, B=B, H=H, L=L, Dk=D, Dv=D, dtype=dtype, seed=34000 + i, gate_dist=gate, h0=h0,
                     gates=kind not in ("la", "gla", "bidir"))
    return r, kind, cfg


@pytest.mark.parametrize("i", range(80))
def test_random_case_wide(i):
    r, kind, cfg = _case_wide(i)
    say(f"case wide {i}: {cfg.name}")
    if kind == "decode":
        _check_decode(r, cfg)
    else:
        _check(r, kind, cfg)


def _check_decode(r, cfg):
    """A few decode steps on N sequences x H heads; in each step about a tenth of the (sequence,
    head) pairs take a zero gate, a tenth a gate of -1e6 and a tenth a gate of 1."""
    dc = inputs.DECODE_256x32.with_(name=cfg.name, N=int(r.integers(1, 40)), H=int(r.integers(1, 9)), Dk=cfg.Dk,
                                    Dv=cfg.Dv, dtype=cfg.dtype, seed=cfg.seed)
    dt = TD[cfg.dtype]
    st0 = inputs.decode_state(dc)
    state = dev_tensor(st0, torch.float32)
    ref = st0.copy()
    eo = 0.0
    for step in range(int(r.integers(1, 6))):
        xt = inputs.decode_token(dc, step)
        la = xt["log_alpha"].copy()
        u = r.random(la.shape)
        la[u < 0.1] = -np.inf
        la[(u >= 0.1) & (u < 0.2)] = -1e6
        la[(u >= 0.2) & (u < 0.3)] = 0.0
        args = [dev_tensor(xt[n], dt) for n in ("q", "k", "v")] + [dev_tensor(xt["beta"], torch.float32),
                                                                  dev_tensor(la, torch.float32)]
        o = ops.gdn_decode_step(*args, state)
        ro, ref = oracle.gdn_decode_step(xt["q"], xt["k"], xt["v"], xt["beta"], la, ref)
        torch.cuda.synchronize()
        eo = max(eo, _rel(host(o), ro))
    tol = TOL_BF16 if cfg.dtype == "bf16" else TOL_F32
    eh = _rel(host(state), ref)
    say(f"  max rel err o {eo:.3e}, state {eh:.3e} (bound {tol:g})")
    assert eo <= tol and eh <= tol, (eo, eh)


def _check(r, kind, cfg):
    x = inputs.prefill_inputs(cfg)
    dt = TD[cfg.dtype]
    q, k, v = (dev_tensor(x[n], dt) for n in ("q", "k", "v"))
    hd = dev_tensor(x["h0"], torch.float32)
    B, H, L, D = cfg.B, cfg.H, cfg.L, cfg.Dk
    if kind in ("gdn", "skip", "band", "noalloc"):
        beta, la = dev_tensor(x["beta"], torch.float32), dev_tensor(x["log_alpha"], torch.float32)
        nch = (L + 63) // 64
        nb = int(r.integers(1, max(2, min(nch, 40))))
        ws = prefill_workspace(torch, B, H, D, nb) if (nb > 1 and r.random() < 0.6) else None
        if kind == "noalloc":   # a random share of the static scratch, or the default
            o, hf = torch.empty_like(v), torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
            sb = int(r.integers(0, ops.prefill_workspace_size(B, H, L, D, dt) + 2)) if r.random() < 0.5 else None
            if sb is not None:
                sb = min(sb, _lib.GDN_PREFILL_NOALLOC_MAX_BYTES)
            ops.gdn_prefill_fwd_noalloc(q, k, v, beta, la, hd, o, hf, sb)
            ro, rh = oracle.gdn_prefill(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], x["h0"])
        elif kind == "gdn":
            o, hf = ops.gdn_prefill_fwd(q, k, v, beta, la, hd, workspace=ws)
            ro, rh = oracle.gdn_prefill(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], x["h0"])
        elif kind == "skip":
            keep = (r.random((B, H, nch)) < r.random()).astype(np.uint8)
            o, hf = ops.gdn_prefill_skip_fwd(q, k, v, beta, la, torch.from_numpy(keep).cuda(), hd, workspace=ws)
            ro, rh = oracle.gdn_prefill_skip(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], keep, x["h0"])
        else:
            band = int(r.integers(0, 4))
            o, hf = ops.gdn_prefill_banded_fwd(q, k, v, beta, la, hd, band=band, workspace=ws)
            ro, rh = oracle.gdn_prefill_banded(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], x["h0"], band=band)
    elif kind in ("la", "lag"):
        la_np = x["log_alpha"] if kind == "lag" else None
        o, hf = ops.linattn_prefill_fwd(q, k, v, hd, log_alpha=dev_tensor(la_np, torch.float32))
        if kind == "lag":
            ro, rh = oracle.gla_prefill(x["q"], x["k"], x["v"], la_np, x["h0"])
        else:
            ro, rh = oracle.linattn_prefill(x["q"], x["k"], x["v"], x["h0"])
    elif kind == "gla":
        la_np = inputs.gate_vectors(cfg)
        o, hf = ops.gla_prefill_fwd(q, k, v, dev_tensor(la_np, torch.float32), hd)
        ro, rh = oracle.gla_vec_prefill(x["q"], x["k"], x["v"], la_np, x["h0"])
    else:
        norm, elu = bool(r.integers(0, 2)), bool(r.integers(0, 2))
        o, hf = ops.linattn_bidir_fwd(q, k, v, normalize=norm, elu1=elu, kv_out=True)
        ro, rh = oracle.linattn_bidir(x["q"], x["k"], x["v"], normalize=norm, elu1=elu)
    torch.cuda.synchronize()
    tol = TOL_BF16 if cfg.dtype == "bf16" else TOL_F32
    eo, eh = _rel(host(o), ro), _rel(host(hf), rh)
    say(f"  max rel err o {eo:.3e}, state {eh:.3e} (bound {tol:g})")
    assert eo <= tol and eh <= tol, (eo, eh)
