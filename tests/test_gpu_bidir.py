"""GPU parity of bidirectional linear attention (linattn_bidir_fwd) through the C ABI against the
fp64 oracle: KV = sum_n phi(k_n) v_n^T, o_n = phi(q_n)^T KV, divided by phi(q_n) . sum_m phi(k_m)
when normalising (datadaily.news overview, section "Linear attention").

Inputs are the linear-attention workload's recipe: q, k either elu(x)+1 features (identity
feature map in the kernel) or raw N(0,1) values with the kernel's elu+1; v N(0,1). Same error
metric and bounds as the other parity tests.
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


def _case(dtype, D, L, B=2, H=3, elu1=True, seed=0):
    cfg = inputs.LINATTN_8K.with_(name=f"bidir_{dtype}_d{D}_L{L}", B=B, H=H, L=L, Dk=D, Dv=D, dtype=dtype,
                                  seed=8000 + seed + D + L, qk="raw" if elu1 else "elu1")
    return cfg, inputs.prefill_inputs(cfg)


def _run(cfg, x, normalize, elu1):
    dt = TD[cfg.dtype]
    q, k, v = (dev_tensor(x[n], dt) for n in ("q", "k", "v"))
    o, kv = ops.linattn_bidir_fwd(q, k, v, normalize=normalize, elu1=elu1, kv_out=True)
    torch.cuda.synchronize()
    return host(o), host(kv)


@pytest.mark.parametrize("normalize,elu1", [(True, True), (False, True), (True, False), (False, False)])
@pytest.mark.parametrize("dtype,D,L", [("bf16", 128, 1), ("bf16", 128, 65), ("bf16", 64, 1000), ("bf16", 128, 777),
                                       ("f32", 128, 333), ("f32", 64, 130)])
def test_bidir_parity(dtype, D, L, normalize, elu1):
    cfg, x = _case(dtype, D, L, elu1=elu1)
    say(f"case {cfg.name} normalize={normalize} elu1={elu1}")
    o, kv = _run(cfg, x, normalize, elu1)
    ro, rkv = oracle.linattn_bidir(x["q"], x["k"], x["v"], normalize=normalize, elu1=elu1)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    eo, ek = max_rel_err(o, ro), max_rel_err(kv, rkv)
    say(f"  max rel err o {eo:.3e}, kv {ek:.3e} (bound {tol:g})")
    assert eo <= tol and ek <= tol, (eo, ek)


def test_bidir_many_blocks_and_deterministic():
    """Long enough that stage 1 splits each head over many blocks; two calls agree bit for bit."""
    cfg, x = _case("bf16", 128, 64 * 300 + 17, B=1, H=2, seed=1)
    say(f"case {cfg.name}")
    dt = TD[cfg.dtype]
    q, k, v = (dev_tensor(x[n], dt) for n in ("q", "k", "v"))
    o1, kv1 = ops.linattn_bidir_fwd(q, k, v, kv_out=True)
    o2, kv2 = ops.linattn_bidir_fwd(q, k, v, kv_out=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(kv1, kv2)
    ro, rkv = oracle.linattn_bidir(x["q"], x["k"], x["v"])
    eo, ek = max_rel_err(host(o1), ro), max_rel_err(host(kv1), rkv)
    say(f"  max rel err o {eo:.3e}, kv {ek:.3e}")
    assert eo <= TOL_BF16 and ek <= TOL_BF16


def test_bidir_empty_sequence():
    q = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    o, kv = ops.linattn_bidir_fwd(q, q, q, kv_out=True)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 128) and torch.count_nonzero(kv).item() == 0


def test_bidir_full_size_sampled_heads():
    """The linear-attention workload's shape (B=4, H=16, L=8192, d=128), raw N(0,1) q and k with
    the elu+1 feature map and the normaliser; three heads checked against the oracle."""
    cfg = inputs.LINATTN_8K.with_(qk="raw")
    say(f"case {cfg.name} bidirectional")
    x = inputs.prefill_inputs(cfg)
    dt = TD[cfg.dtype]
    q, k, v = (dev_tensor(x[n], dt) for n in ("q", "k", "v"))
    o, kv = ops.linattn_bidir_fwd(q, k, v, kv_out=True)
    torch.cuda.synchronize()
    o, kv = host(o), host(kv)
    for b, h in ((0, 0), (3, 15), (1, 9)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ro, rkv = oracle.linattn_bidir(x["q"][sl], x["k"][sl], x["v"][sl])
        eo, ek = max_rel_err(o[sl], ro), max_rel_err(kv[sl], rkv)
        say(f"  b{b} h{h}: max rel err o {eo:.3e}, kv {ek:.3e}")
        assert eo <= TOL_BF16 and ek <= TOL_BF16
