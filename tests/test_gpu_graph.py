"""The entry points under HIP graph capture. One call each of gdn_prefill_fwd, gdn_prefill_fwd_noalloc,
gdn_prefill_skip_fwd, gdn_prefill_banded_fwd, linattn_prefill_fwd (plain and gated), gla_prefill_fwd
and gdn_decode_step is captured into one graph, linattn_bidir_fwd into a graph of its own, all with
caller-owned outputs and workspaces (nothing is allocated inside the capture), and each graph is
replayed several times with eager work and synchronisations between the replays. Every replay must
reproduce the eager results bit for bit (the kernels are deterministic), and the eager results are
checked against the fp64 oracle, so that a replay cannot match a wrong result. The library makes no
memset, copy, allocation or synchronisation call, so nothing but its kernel launches enters a graph."""
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
B, H, D = 1, 3, 128


def _case(name, seed, L, base, **kw):
    cfg = base.with_(name=name, B=B, H=H, L=L, seed=seed, **kw)
    x = inputs.prefill_inputs(cfg)
    d = {n: dev_tensor(x[n], BF) for n in ("q", "k", "v")}
    d.update({n: dev_tensor(x[n], torch.float32) for n in ("beta", "log_alpha", "h0") if x.get(n) is not None})
    return cfg, x, d


def _ws(size_fn, L):
    return torch.empty(max(size_fn(B, H, L, D, BF), 1), dtype=torch.uint8, device="cuda")


def _gdn_case(name, seed, L, gate_dist="config"):
    return _case(name, seed, L, inputs.GDN_32K, h0=0.1, gate_dist=gate_dist)


def test_graph_replays_equal_eager_calls():
    say("case graph: every entry point, one call each, in one captured graph")
    cases = []   # (name, call, outputs, oracle results)

    # gated delta rule: dense, no-allocation, skipped updates, block-adjacent solve
    _, xg, dg = _gdn_case("graph_gdn", 7101, 64 * 12 + 29)
    outg = [torch.empty_like(dg["v"]), torch.empty_like(dg["h0"])]
    wsg = _ws(ops.prefill_workspace_size, xg["q"].shape[2])
    cases.append(("gdn", lambda: ops.gdn_prefill_fwd(dg["q"], dg["k"], dg["v"], dg["beta"], dg["log_alpha"], dg["h0"],
                                                     o=outg[0], h_final=outg[1], workspace=wsg),
                  outg, oracle.gdn_prefill(*(xg[n] for n in ("q", "k", "v", "beta", "log_alpha", "h0")))))

    _, xn, dn = _gdn_case("graph_noalloc", 7102, 64 * 5 + 3, "long")
    outn = [torch.empty_like(dn["v"]), torch.empty_like(dn["h0"])]
    cases.append(("noalloc", lambda: ops.gdn_prefill_fwd_noalloc(dn["q"], dn["k"], dn["v"], dn["beta"], dn["log_alpha"],
                                                                 dn["h0"], outn[0], outn[1]),
                  outn, oracle.gdn_prefill(*(xn[n] for n in ("q", "k", "v", "beta", "log_alpha", "h0")))))

    Ls = 64 * 10 + 7
    _, xs, ds = _gdn_case("graph_skip", 7103, Ls, "long")
    keep_np = (np.random.default_rng(7103).random((B, H, (Ls + 63) // 64)) < 0.4).astype(np.uint8)
    keep = torch.from_numpy(keep_np).cuda()
    outs_ = [torch.empty_like(ds["v"]), torch.empty_like(ds["h0"])]
    wss = _ws(ops.prefill_workspace_size, Ls)
    cases.append(("skip", lambda: ops.gdn_prefill_skip_fwd(ds["q"], ds["k"], ds["v"], ds["beta"], ds["log_alpha"], keep,
                                                           ds["h0"], o=outs_[0], h_final=outs_[1], workspace=wss),
                  outs_, oracle.gdn_prefill_skip(*(xs[n] for n in ("q", "k", "v", "beta", "log_alpha")), keep_np,
                                                 xs["h0"])))

    _, xb, db = _gdn_case("graph_band1", 7104, 64 * 8 + 50)
    outb = [torch.empty_like(db["v"]), torch.empty_like(db["h0"])]
    wsb = _ws(ops.prefill_workspace_size, xb["q"].shape[2])
    cases.append(("band1", lambda: ops.gdn_prefill_banded_fwd(db["q"], db["k"], db["v"], db["beta"], db["log_alpha"],
                                                              db["h0"], band=1, o=outb[0], h_final=outb[1],
                                                              workspace=wsb),
                  outb, oracle.gdn_prefill_banded(*(xb[n] for n in ("q", "k", "v", "beta", "log_alpha", "h0")),
                                                  band=1)))

    # linear attention: plain, a decay per token, a gate per key dimension (the bidirectional
    # form, whose binding allocates its KV output, is captured through the C ABI below)
    _, xl, dl = _case("graph_la", 7105, 64 * 9 + 40, inputs.LINATTN_8K, h0=0.1)
    outl = [torch.empty_like(dl["v"]), torch.empty_like(dl["h0"])]
    wsl = _ws(ops.linattn_prefill_workspace_size, xl["q"].shape[2])
    cases.append(("la", lambda: ops.linattn_prefill_fwd(dl["q"], dl["k"], dl["v"], dl["h0"], o=outl[0],
                                                        h_final=outl[1], workspace=wsl),
                  outl, oracle.linattn_prefill(xl["q"], xl["k"], xl["v"], xl["h0"])))

    _, xa, da = _case("graph_la_gated", 7106, 64 * 7 + 1, inputs.LINATTN_8K, h0=0.1, gates=True, gate_dist="long")
    outa = [torch.empty_like(da["v"]), torch.empty_like(da["h0"])]
    wsa = _ws(ops.linattn_prefill_workspace_size, xa["q"].shape[2])
    cases.append(("la_gated", lambda: ops.linattn_prefill_fwd(da["q"], da["k"], da["v"], da["h0"],
                                                              log_alpha=da["log_alpha"], o=outa[0], h_final=outa[1],
                                                              workspace=wsa),
                  outa, oracle.gla_prefill(xa["q"], xa["k"], xa["v"], xa["log_alpha"], xa["h0"])))

    cv, xv, dv = _case("graph_gla_vec", 7107, 64 * 6 + 33, inputs.LINATTN_8K, h0=0.1)
    la_vec = inputs.gate_vectors(cv)
    la_vec_d = dev_tensor(la_vec, torch.float32)
    outv = [torch.empty_like(dv["v"]), torch.empty_like(dv["h0"])]
    wsv = _ws(ops.gla_prefill_workspace_size, xv["q"].shape[2])
    cases.append(("gla_vec", lambda: ops.gla_prefill_fwd(dv["q"], dv["k"], dv["v"], la_vec_d, dv["h0"], o=outv[0],
                                                         h_final=outv[1], workspace=wsv),
                  outv, oracle.gla_vec_prefill(xv["q"], xv["k"], xv["v"], la_vec, xv["h0"])))

    # decode: the state is updated in place, so it is reset before every run
    dcfg = inputs.DECODE_256x32.with_(name="graph_decode", N=6, H=4, seed=7109)
    st0 = inputs.decode_state(dcfg)
    xd = inputs.decode_token(dcfg, 0)
    dd = {n: dev_tensor(xd[n], BF) for n in ("q", "k", "v")}
    dd.update({n: dev_tensor(xd[n], torch.float32) for n in ("beta", "log_alpha")})
    state0 = dev_tensor(st0, torch.float32)
    outd = [torch.empty_like(dd["v"]), torch.empty_like(state0)]
    cases.append(("decode", lambda: ops.gdn_decode_step(dd["q"], dd["k"], dd["v"], dd["beta"], dd["log_alpha"], outd[1],
                                                        o=outd[0]),
                  outd, oracle.gdn_decode_step(xd["q"], xd["k"], xd["v"], xd["beta"], xd["log_alpha"], st0)))

    def calls():
        for _, call, _, _ in cases:
            call()

    def clear():   # eager, between replays: every output poisoned, the decode state reset
        for _, _, outs, _ in cases:
            for t in outs:
                t.fill_(float("nan"))
        outd[1].copy_(state0)

    # eager results (also the warm-up: the library's one-time set-up happens outside the capture)
    clear()
    calls()
    torch.cuda.synchronize()
    eager = {name: [t.clone() for t in outs] for name, _, outs, _ in cases}
    for name, _, outs, ref in cases:
        for got, r, what in zip(eager[name], ref, ("outputs", "final state")):
            e = max_rel_err(host(got), r)
            assert e <= TOL_BF16, f"{name} eager {what}: {e:.3e}"

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
        for name, _, outs, _ in cases:
            for got, want, what in zip(outs, eager[name], ("outputs", "final state")):
                assert torch.equal(got, want), f"replay {rep}: {name} {what} differ from the eager call"
        say(f"  replay {rep}: {len(cases)} calls bitwise equal to the eager calls")


def test_graph_bidirectional():
    """linattn_bidir_fwd through the C ABI with caller-owned o, KV and workspace, captured and replayed."""
    from gated_deltanet_chunked_rule_amd import _lib
    say("case graph_bidir")
    _, x, d = _case("graph_bidir", 7108, 64 * 5 + 9, inputs.LINATTN_8K, qk="raw")
    L = x["q"].shape[2]
    o = torch.empty_like(d["v"])
    kv = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    wsb = ops.linattn_bidir_workspace_size(B, H, L, D, BF)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    flags = _lib.GDN_BIDIR_NORMALIZE | _lib.GDN_BIDIR_ELU1

    def call():
        rc = _lib.load().linattn_bidir_fwd(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), o.data_ptr(),
                                           kv.data_ptr(), B, H, L, D, D, _lib.GDN_BF16, flags, ws.data_ptr(), wsb,
                                           torch.cuda.current_stream().cuda_stream)
        _lib.check(rc, "linattn_bidir_fwd")

    call()
    torch.cuda.synchronize()
    eo, ekv = o.clone(), kv.clone()
    ro, rkv = oracle.linattn_bidir(x["q"], x["k"], x["v"], normalize=True, elu1=True)
    assert max_rel_err(host(eo), ro) <= TOL_BF16 and max_rel_err(host(ekv), rkv) <= TOL_BF16
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        o.fill_(float("nan"))
        kv.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eo) and torch.equal(kv, ekv), f"replay {rep}: bidirectional results differ"
    say("  3 replays bitwise equal to the eager call")
