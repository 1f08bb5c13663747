"""GPU parity of the gated delta rule with the block-adjacent intra-chunk solve
(gdn_prefill_banded_fwd) through the C ABI, against the oracle's chunked form with the same band
(oracle/banded.py). Same error metric and bounds as test_gpu_parity.py. band = 3 must equal
gdn_prefill_fwd bit for bit."""
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


def _dev(cfg, x):
    dt = TD[cfg.dtype]
    return ([dev_tensor(x[n], dt) for n in ("q", "k", "v")]
            + [dev_tensor(x[n], torch.float32) for n in ("beta", "log_alpha", "h0")])


@pytest.mark.parametrize("band", [0, 1, 2])
@pytest.mark.parametrize("dtype,D,L,gates", [("bf16", 128, 200, "long"), ("bf16", 64, 1000, "long"),
                                             ("bf16", 128, 333, "config"), ("f32", 128, 150, "long"),
                                             ("f32", 64, 97, "long")])
def test_banded_parity(dtype, D, L, gates, band):
    cfg = inputs.GDN_32K.with_(name=f"banded_{dtype}_d{D}_L{L}_{gates}", B=2, H=2, L=L, Dk=D, Dv=D, dtype=dtype,
                               seed=9000 + D + L, gate_dist=gates)
    say(f"case {cfg.name} band {band}")
    x = inputs.prefill_inputs(cfg)
    q, k, v, beta, la, h0 = _dev(cfg, x)
    o, hf = ops.gdn_prefill_banded_fwd(q, k, v, beta, la, h0, band=band)
    torch.cuda.synchronize()
    ro, rh = oracle.gdn_prefill_banded(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], x["h0"], band=band)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    eo, eh = max_rel_err(host(o), ro), max_rel_err(host(hf), rh)
    say(f"  max rel err o {eo:.3e}, h_final {eh:.3e} (bound {tol:g})")
    assert eo <= tol and eh <= tol, (eo, eh)


def test_full_band_is_the_dense_path_bitwise():
    cfg = inputs.GDN_32K.with_(name="banded_full", B=1, H=3, L=700, seed=9100)
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    q, k, v, beta, la, h0 = _dev(cfg, x)
    o1, h1 = ops.gdn_prefill_banded_fwd(q, k, v, beta, la, h0, band=3)
    o2, h2 = ops.gdn_prefill_fwd(q, k, v, beta, la, h0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_banded_full_size_sampled_heads():
    """The 32K GDN workload (B=1, H=32, L=32768) with band 1, long-memory gates, its sequences in 7
    blocks (of 74 chunks, the last one shorter)."""
    cfg = inputs.GDN_32K.with_(gate_dist="long")
    say(f"case {cfg.name} band 1, 7 blocks")
    x = inputs.prefill_inputs(cfg)
    q, k, v, beta, la, h0 = _dev(cfg, x)
    ws = prefill_workspace(torch, cfg.B, cfg.H, 128, 7)
    o, hf = ops.gdn_prefill_banded_fwd(q, k, v, beta, la, h0, band=1, workspace=ws)
    torch.cuda.synchronize()
    o, hf = host(o), host(hf)
    for h in (0, 21):
        sl = (slice(0, 1), slice(h, h + 1))
        ro, rh = oracle.gdn_prefill_banded(x["q"][sl], x["k"][sl], x["v"][sl], x["beta"][sl], x["log_alpha"][sl],
                                           x["h0"][sl], band=1)
        eo, eh = max_rel_err(o[sl], ro), max_rel_err(hf[sl], rh)
        say(f"  head {h}: max rel err o {eo:.3e}, h_final {eh:.3e}")
        assert eo <= TOL_BF16 and eh <= TOL_BF16
