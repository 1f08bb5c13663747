"""GPU parity of the block-parallel causal linear attention (linattn_prefill_fwd) where its block
structure matters: blocks of many chunks (a small workspace holds few blocks), ragged tails inside
a block, plain and decay-gated, bf16 and fp32, against the fp64 oracle; repeat calls bitwise equal.

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


def _min_workspace(B, H, D, dt):
    """The smallest workspace linattn_prefill_fwd accepts: one block (a D x D fp32 state and
    4 bytes) per slice, so each slice is a single block of all its chunks."""
    return torch.empty(B * H * (D * D * 4 + 4), dtype=torch.uint8, device="cuda")


def _two_blocks_workspace(B, H, D, dt):
    return torch.empty(2 * B * H * (D * D * 4 + 4), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dtype,D,L", [("bf16", 128, 1000), ("bf16", 64, 1500), ("f32", 128, 777),
                                       ("f32", 64, 640), ("bf16", 128, 129)])
def test_linattn_small_workspace_long_blocks(gated, dtype, D, L):
    cfg = inputs.GDN_32K.with_(name=f"la_blocks_{'gated' if gated else 'plain'}_{dtype}_d{D}_L{L}", B=1, H=3, L=L,
                               Dk=D, Dv=D, dtype=dtype, seed=7000 + D + L + gated, gate_dist="long")
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    dt = TD[dtype]
    q, k, v = (dev_tensor(x[n], dt) for n in ("q", "k", "v"))
    h0 = dev_tensor(x["h0"], torch.float32)
    la = dev_tensor(x["log_alpha"], torch.float32) if gated else None
    if gated:
        ro, rh = oracle.gla_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
    else:
        ro, rh = oracle.linattn_prefill(x["q"], x["k"], x["v"], x["h0"])
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for mk in (_min_workspace, _two_blocks_workspace):
        ws = mk(cfg.B, cfg.H, D, dt)
        o, hf = ops.linattn_prefill_fwd(q, k, v, h0, log_alpha=la, workspace=ws)
        o2, hf2 = ops.linattn_prefill_fwd(q, k, v, h0, log_alpha=la, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(hf, hf2)
        eo, eh = max_rel_err(host(o), ro), max_rel_err(host(hf), rh)
        say(f"  {cfg.name} {mk.__name__}: max rel err o {eo:.3e}, h_final {eh:.3e} (bound {tol:g})")
        assert eo <= tol and eh <= tol, (eo, eh)


def test_linattn_in_place_state():
    """h_final == h0: the state is read before it is overwritten."""
    cfg = inputs.LINATTN_8K.with_(name="la_in_place", B=2, H=2, L=300, seed=7100, h0=0.1)
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    q, k, v = (dev_tensor(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    h0 = dev_tensor(x["h0"], torch.float32)
    o_ref, h_ref = ops.linattn_prefill_fwd(q, k, v, h0.clone())
    o, hf = ops.linattn_prefill_fwd(q, k, v, h0, h_final=h0)
    torch.cuda.synchronize()
    assert hf.data_ptr() == h0.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(hf, h_ref)
