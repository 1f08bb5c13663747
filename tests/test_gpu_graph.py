"""The entry points under HIP graph capture: one call each of gdn_prefill_fwd, gdn_prefill_fwd_noalloc,
linattn_prefill_fwd (plain and gated) and gdn_decode_step is captured into one graph with caller-owned
outputs and workspaces (nothing is allocated inside the capture), and the graph is replayed several
times with eager work and synchronisations between the replays. Every replay must reproduce the
eager results bit for bit (the kernels are deterministic), and the eager results are checked against
the fp64 oracle, so that a replay cannot match a wrong result. The library makes no memset, copy,
allocation or synchronisation call, so nothing but its kernel launches enters the graph."""
import numpy as np
import pytest

import oracle
from gated_deltanet_chunked_rule_amd import inputs
from gpu_util import TOL_BF16, dev_tensor, host, max_rel_err, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gated_deltanet_chunked_rule_amd import ops  # noqa: E402

BF = torch.bfloat16


def _prefill_case(name, seed, L, gates=True, gate_dist="config"):
    base = inputs.GDN_32K if gates else inputs.LINATTN_8K
    cfg = base.with_(name=name, B=1, H=3, L=L, seed=seed, h0=0.1, gates=gates, gate_dist=gate_dist)
    x = inputs.prefill_inputs(cfg)
    d = {n: dev_tensor(x[n], BF) for n in ("q", "k", "v")}
    d.update({n: dev_tensor(x[n], torch.float32) for n in ("beta", "log_alpha", "h0") if x.get(n) is not None})
    return x, d


def test_graph_replays_equal_eager_calls():
    say("case graph: gdn prefill, noalloc prefill, linear attention plain and gated, decode step")
    xg, dg = _prefill_case("graph_gdn", 7101, 64 * 12 + 29)
    xn, dn = _prefill_case("graph_noalloc", 7102, 64 * 5 + 3, gate_dist="long")
    xl, dl = _prefill_case("graph_la", 7103, 64 * 9 + 40, gates=False)
    xa, da = _prefill_case("graph_la_gated", 7104, 64 * 7 + 1, gates=True)
    dcfg = inputs.DECODE_256x32.with_(name="graph_decode", N=6, H=4, seed=7105)
    st0 = inputs.decode_state(dcfg)
    xd = inputs.decode_token(dcfg, 0)
    dd = {n: dev_tensor(xd[n], BF) for n in ("q", "k", "v")}
    dd.update({n: dev_tensor(xd[n], torch.float32) for n in ("beta", "log_alpha")})
    state0 = dev_tensor(st0, torch.float32)

    # caller-owned outputs and workspaces
    B, H, D = 1, 3, 128
    ws_g = torch.empty(ops.prefill_workspace_size(B, H, xg["q"].shape[2], D, BF), dtype=torch.uint8, device="cuda")
    ws_l = torch.empty(ops.linattn_prefill_workspace_size(B, H, xl["q"].shape[2], D, BF), dtype=torch.uint8,
                       device="cuda")
    ws_a = torch.empty(ops.linattn_prefill_workspace_size(B, H, xa["q"].shape[2], D, BF), dtype=torch.uint8,
                       device="cuda")
    outs = {
        "gdn": (torch.empty_like(dg["v"]), torch.empty_like(dg["h0"])),
        "noalloc": (torch.empty_like(dn["v"]), torch.empty_like(dn["h0"])),
        "la": (torch.empty_like(dl["v"]), torch.empty_like(dl["h0"])),
        "la_gated": (torch.empty_like(da["v"]), torch.empty_like(da["h0"])),
    }
    o_dec = torch.empty_like(dd["v"])
    state = torch.empty_like(state0)

    def calls():
        ops.gdn_prefill_fwd(dg["q"], dg["k"], dg["v"], dg["beta"], dg["log_alpha"], dg["h0"],
                            o=outs["gdn"][0], h_final=outs["gdn"][1], workspace=ws_g)
        ops.gdn_prefill_fwd_noalloc(dn["q"], dn["k"], dn["v"], dn["beta"], dn["log_alpha"], dn["h0"],
                                    outs["noalloc"][0], outs["noalloc"][1])
        ops.linattn_prefill_fwd(dl["q"], dl["k"], dl["v"], dl["h0"], o=outs["la"][0], h_final=outs["la"][1],
                                workspace=ws_l)
        ops.linattn_prefill_fwd(da["q"], da["k"], da["v"], da["h0"], log_alpha=da["log_alpha"],
                                o=outs["la_gated"][0], h_final=outs["la_gated"][1], workspace=ws_a)
        ops.gdn_decode_step(dd["q"], dd["k"], dd["v"], dd["beta"], dd["log_alpha"], state, o=o_dec)

    def clear():   # eager, between replays: every output poisoned, the decode state reset
        for o, h in outs.values():
            o.fill_(float("nan"))
            h.fill_(float("nan"))
        o_dec.fill_(float("nan"))
        state.copy_(state0)

    # eager results (also the warm-up: one-time set-up of the library happens outside the capture)
    clear()
    calls()
    torch.cuda.synchronize()
    eager = {k: (o.clone(), h.clone()) for k, (o, h) in outs.items()}
    eager_dec = (o_dec.clone(), state.clone())

    # the eager results against the oracle
    ro, rh = oracle.gdn_prefill(*(xg[n] for n in ("q", "k", "v", "beta", "log_alpha", "h0")))
    assert max_rel_err(host(eager["gdn"][0]), ro) <= TOL_BF16 and max_rel_err(host(eager["gdn"][1]), rh) <= TOL_BF16
    ro, rh = oracle.gdn_prefill(*(xn[n] for n in ("q", "k", "v", "beta", "log_alpha", "h0")))
    assert max_rel_err(host(eager["noalloc"][0]), ro) <= TOL_BF16
    assert max_rel_err(host(eager["noalloc"][1]), rh) <= TOL_BF16
    ro, rh = oracle.linattn_prefill(xl["q"], xl["k"], xl["v"], xl["h0"])
    assert max_rel_err(host(eager["la"][0]), ro) <= TOL_BF16 and max_rel_err(host(eager["la"][1]), rh) <= TOL_BF16
    ro, rh = oracle.gla_prefill(xa["q"], xa["k"], xa["v"], xa["log_alpha"], xa["h0"])
    assert max_rel_err(host(eager["la_gated"][0]), ro) <= TOL_BF16
    assert max_rel_err(host(eager["la_gated"][1]), rh) <= TOL_BF16
    ro, rs = oracle.gdn_decode_step(xd["q"], xd["k"], xd["v"], xd["beta"], xd["log_alpha"], st0)
    assert max_rel_err(host(eager_dec[0]), ro) <= TOL_BF16 and max_rel_err(host(eager_dec[1]), rs) <= TOL_BF16

    g = torch.cuda.CUDAGraph()
    clear()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (o, h) in outs.items():
            assert torch.equal(o, eager[k][0]), f"replay {rep}: {k} outputs differ from the eager call"
            assert torch.equal(h, eager[k][1]), f"replay {rep}: {k} final state differs from the eager call"
        assert torch.equal(o_dec, eager_dec[0]), f"replay {rep}: decode outputs differ"
        assert torch.equal(state, eager_dec[1]), f"replay {rep}: decode state differs"
        say(f"  replay {rep}: bitwise equal to the eager calls")
