"""Tensors of more than 2^31 elements: B=1, H=17 slices of 2^20 + 37 tokens at d = 128, so the last
slice's rows start 2,147,559,424 elements into q, k, v and o (past 2^31) and only 64-bit offsets
reach them. Every slice holds the same inputs (one slice from the seeded generator, repeated on the
device), so every slice's outputs and final state must equal the first slice's bit for bit (one call
splits every slice into the same blocks). The last slice's last W tokens and its final state are
checked against the oracle, started from the final state of a one-slice call over the first L - W
tokens (which the million-token tests check on their own).
"""
import pytest

import oracle
from gated_deltanet_chunked_rule_amd import inputs
from gpu_util import TOL_BF16, dev_tensor, host, max_rel_err, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gated_deltanet_chunked_rule_amd import ops  # noqa: E402

H, L, W, D = 17, 2 ** 20 + 37, 64 * 64 + 37, 128
BF = torch.bfloat16


def test_shape_passes_two_to_the_31():
    assert (H - 1) * L * D > 2 ** 31 and H * L * D < 2 ** 32


@pytest.mark.parametrize("kind", ["gdn", "la", "la_gated", "gla_vec"])
def test_slices_beyond_two_to_the_31_elements(kind):
    base = inputs.GDN_128K if kind == "gdn" else inputs.LINATTN_8K
    cfg = base.with_(name=f"large_offsets_{kind}", B=1, H=1, L=L, seed=81, h0=0.1,
                     gates=kind in ("gdn", "la_gated"), gate_dist="long")
    say(f"case {cfg.name}: inputs (one slice, repeated {H} times on the device)")
    s = inputs.prefill_slice(cfg, 0, 0)
    one = lambda a, d: dev_tensor(a[None, None], d)
    rep = lambda t: t.expand(1, H, *t.shape[2:]).contiguous()
    q1, k1, v1 = one(s["q"], BF), one(s["k"], BF), one(s["v"], BF)
    h01 = one(s["h0"], torch.float32)
    if kind == "gla_vec":
        la_np = inputs.gate_vectors(cfg)[0, 0]
    else:
        la_np = s.get("log_alpha")
    la1 = one(la_np, torch.float32) if la_np is not None else None
    b1 = one(s["beta"], torch.float32) if kind == "gdn" else None

    def run(n_slices, P):
        cut = lambda t: None if t is None else (rep(t) if n_slices == H else t)[:, :, :P].contiguous()
        args = (cut(q1), cut(k1), cut(v1))
        h0 = h01.expand(1, n_slices, D, D).contiguous()
        if kind == "gdn":
            return ops.gdn_prefill_fwd(*args, cut(b1), cut(la1), h0)
        if kind == "gla_vec":
            return ops.gla_prefill_fwd(*args, cut(la1), h0)
        return ops.linattn_prefill_fwd(*args, h0, log_alpha=cut(la1))

    say(f"case {cfg.name}: GPU, {H} slices of {L} tokens")
    o, hf = run(H, L)
    torch.cuda.synchronize()
    for h in range(1, H):
        assert torch.equal(o[0, h], o[0, 0]), f"slice {h} outputs differ from slice 0"
        assert torch.equal(hf[0, h], hf[0, 0]), f"slice {h} final state differs from slice 0"
    o_last = host(o[:, H - 1:, L - W:])
    h_last = host(hf[:, H - 1:])
    del o, hf
    P = L - W
    _, h_p = run(1, P)
    torch.cuda.synchronize()
    win = lambda a: None if a is None else a[P:][None, None]
    say(f"case {cfg.name}: oracle over the last {W} tokens of the last slice")
    x = {n: win(s.get(n)) for n in ("q", "k", "v", "beta")}
    if kind == "gdn":
        ro, rh = oracle.gdn_prefill(x["q"], x["k"], x["v"], x["beta"], win(la_np), host(h_p))
    elif kind == "gla_vec":
        ro, rh = oracle.gla_vec_prefill(x["q"], x["k"], x["v"], win(la_np), host(h_p))
    elif kind == "la_gated":
        ro, rh = oracle.gla_prefill(x["q"], x["k"], x["v"], win(la_np), host(h_p))
    else:
        ro, rh = oracle.linattn_prefill(x["q"], x["k"], x["v"], host(h_p))
    eo, eh = max_rel_err(o_last, ro), max_rel_err(h_last, rh)
    say(f"  last slice window: max rel err o {eo:.3e}, h_final {eh:.3e} (bound {TOL_BF16:g})")
    assert eo <= TOL_BF16 and eh <= TOL_BF16
    torch.cuda.empty_cache()


def test_bidirectional_slices_beyond_two_to_the_31_elements():
    """Bidirectional linear attention (elu + 1, normalised) on the same 17 identical slices: every
    slice's outputs and KV equal the first slice's bit for bit, and the last slice's outputs and KV
    match the oracle over the whole slice."""
    cfg = inputs.LINATTN_8K.with_(name="large_offsets_bidir", B=1, H=1, L=L, seed=83, qk="raw")
    say(f"case {cfg.name}: inputs (one slice, repeated {H} times on the device)")
    s = inputs.prefill_slice(cfg, 0, 0)
    rep = lambda a: dev_tensor(a[None, None], BF).expand(1, H, L, D).contiguous()
    q, k, v = rep(s["q"]), rep(s["k"]), rep(s["v"])
    say(f"case {cfg.name}: GPU, {H} slices of {L} tokens")
    o, kv = ops.linattn_bidir_fwd(q, k, v, normalize=True, elu1=True, kv_out=True)
    torch.cuda.synchronize()
    del q, k, v
    for h in range(1, H):
        assert torch.equal(o[0, h], o[0, 0]), f"slice {h} outputs differ from slice 0"
        assert torch.equal(kv[0, h], kv[0, 0]), f"slice {h} KV differs from slice 0"
    say(f"case {cfg.name}: oracle over the last slice ({L} tokens)")
    ro, rkv = oracle.linattn_bidir(s["q"][None, None], s["k"][None, None], s["v"][None, None], normalize=True,
                                   elu1=True)
    eo, ekv = max_rel_err(host(o[:, H - 1:]), ro), max_rel_err(host(kv[:, H - 1:]), rkv)
    say(f"  last slice: max rel err o {eo:.3e}, KV {ekv:.3e} (bound {TOL_BF16:g})")
    assert eo <= TOL_BF16 and ekv <= TOL_BF16
    del o, kv
    torch.cuda.empty_cache()
