"""Guard bands around every buffer a call writes: outputs, final states, workspaces, the decode
state and the bidirectional KV output are carved out of larger allocations whose margins (4 KiB
on each side) hold a byte pattern; after the call the margins must be unchanged, the inputs
bitwise unchanged, and the results still within the oracle's bounds. An out-of-bounds store that
happens to leave the results right is caught here."""

import numpy as np
import pytest

import oracle
from gated_deltanet_chunked_rule_amd import _lib, inputs
from gpu_util import TOL_BF16, TOL_F32, dev_tensor, host, max_rel_err, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

from gated_deltanet_chunked_rule_amd import ops  # noqa: E402

PAD = 4096
PATTERN = 0xA5
TD = {"bf16": torch.bfloat16, "f32": torch.float32}


class Guarded:
    """A tensor of `shape` and `dtype` inside a byte buffer with PAD guard bytes on each side."""

    def __init__(self, shape, dtype, fill=None):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.buf = torch.full((PAD + max(n, 1) + PAD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.buf[PAD:PAD + n].view(dtype).view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def intact(self):
        head, tail = self.buf[:PAD], self.buf[PAD + self.n:]
        return bool((head == PATTERN).all()) and bool((tail == PATTERN).all())


def _check(o, hf, ro, rh, tol, what):
    eo, eh = max_rel_err(host(o), ro), max_rel_err(host(hf), rh)
    say(f"  {what}: max rel err o {eo:.3e}, h_final {eh:.3e} (bound {tol:g})")
    assert eo <= tol and eh <= tol, (eo, eh)


def _gdn_inputs(dtype, D, L, seed, gate_dist="config"):
    cfg = inputs.GDN_32K.with_(name=f"canary_{dtype}_d{D}_L{L}", B=1, H=3, L=L, Dk=D, Dv=D, dtype=dtype, seed=seed,
                               gate_dist=gate_dist)
    x = inputs.prefill_inputs(cfg)
    dt = TD[dtype]
    d = {n: dev_tensor(x[n], dt) for n in ("q", "k", "v")}
    d.update({n: dev_tensor(x[n], torch.float32) for n in ("beta", "log_alpha", "h0")})
    return cfg, x, d


@pytest.mark.parametrize("variant", ["dense", "skip", "band1", "noalloc"])
@pytest.mark.parametrize("dtype,D,gates", [("bf16", 128, "config"), ("bf16", 128, "long"), ("f32", 64, "long")])
def test_gdn_prefill_guard_bands(variant, dtype, D, gates):
    L = 64 * 11 + 13
    cfg, x, d = _gdn_inputs(dtype, D, L, 9100 + D, gates)
    say(f"case {cfg.name} {gates} {variant}")
    before = {n: t.clone() for n, t in d.items()}
    o = Guarded(d["v"].shape, TD[dtype])
    hf = Guarded(d["h0"].shape, torch.float32)
    nb = 4   # four blocks per slice: map, scan and output kernels all run
    wsb = 3 * ((2 * nb - 1) * 4 * D * D + 256)
    ws = Guarded((wsb,), torch.uint8)
    args = (d["q"], d["k"], d["v"], d["beta"], d["log_alpha"])
    keep = None
    if variant == "dense":
        ops.gdn_prefill_fwd(*args, d["h0"], o=o.t, h_final=hf.t, workspace=ws.t)
    elif variant == "skip":
        keep_np = (np.random.default_rng(9101).random((1, 3, (L + 63) // 64)) < 0.29).astype(np.uint8)
        # the last chunk kept: skipped under the configured gates, it would leave a final state of
        # about e^-136 times the previous one, below fp32's range (the oracle's is not zero)
        keep_np[..., -1] = 1
        keep = torch.from_numpy(keep_np).cuda()
        ops.gdn_prefill_skip_fwd(*args, keep, d["h0"], o=o.t, h_final=hf.t, workspace=ws.t)
    elif variant == "band1":
        ops.gdn_prefill_banded_fwd(*args, d["h0"], band=1, o=o.t, h_final=hf.t, workspace=ws.t)
    else:
        ops.gdn_prefill_fwd_noalloc(*args, d["h0"], o.t, hf.t, scratch_bytes=wsb)
    torch.cuda.synchronize()
    assert o.intact() and hf.intact() and ws.intact()
    for n, t in d.items():
        assert torch.equal(t, before[n]), n
    if variant == "dense" or variant == "noalloc":
        ro, rh = oracle.gdn_prefill(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], x["h0"])
    elif variant == "skip":
        ro, rh = oracle.gdn_prefill_skip(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], keep.cpu().numpy(),
                                         x["h0"])
    else:
        ro, rh = oracle.gdn_prefill_banded(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], x["h0"], band=1)
    _check(o.t, hf.t, ro, rh, TOL_BF16 if dtype == "bf16" else TOL_F32, f"{cfg.name} {variant}")


@pytest.mark.parametrize("kind", ["plain", "gated", "gla_vec"])
def test_linattn_guard_bands(kind):
    D, L = 128, 64 * 9 + 5
    cfg = inputs.LINATTN_8K.with_(name=f"canary_la_{kind}", B=1, H=2, L=L, seed=9200, h0=0.1,
                                  gates=kind == "gated", gate_dist="long")
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    q, k, v = (dev_tensor(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    h0 = dev_tensor(x["h0"], torch.float32)
    o = Guarded(v.shape, torch.bfloat16)
    hf = Guarded(h0.shape, torch.float32)
    if kind == "gla_vec":
        la_np = inputs.gate_vectors(cfg)
        wsb = 2 * 3 * (D * D * 4 + D * 4)     # three blocks per slice
        ws = Guarded((wsb,), torch.uint8)
        ops.gla_prefill_fwd(q, k, v, dev_tensor(la_np, torch.float32), h0, o=o.t, h_final=hf.t, workspace=ws.t)
        ro, rh = oracle.gla_vec_prefill(x["q"], x["k"], x["v"], la_np, x["h0"])
    else:
        wsb = 2 * 3 * (D * D * 4 + 4)
        ws = Guarded((wsb,), torch.uint8)
        la = dev_tensor(x["log_alpha"], torch.float32) if kind == "gated" else None
        ops.linattn_prefill_fwd(q, k, v, h0, log_alpha=la, o=o.t, h_final=hf.t, workspace=ws.t)
        if kind == "gated":
            ro, rh = oracle.gla_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
        else:
            ro, rh = oracle.linattn_prefill(x["q"], x["k"], x["v"], x["h0"])
    torch.cuda.synchronize()
    assert o.intact() and hf.intact() and ws.intact()
    _check(o.t, hf.t, ro, rh, TOL_BF16, cfg.name)


def test_bidir_guard_bands():
    B, H, L, D = 1, 2, 64 * 7 + 9, 128
    cfg = inputs.LINATTN_8K.with_(name="canary_bidir", B=B, H=H, L=L, seed=9300, qk="raw")
    say(f"case {cfg.name}")
    x = inputs.prefill_inputs(cfg)
    q, k, v = (dev_tensor(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    o = Guarded(v.shape, torch.bfloat16)
    kv = Guarded((B, H, D, D), torch.float32)
    wsb = ops.linattn_bidir_workspace_size(B, H, L, D, torch.bfloat16)
    ws = Guarded((wsb,), torch.uint8)
    flags = _lib.GDN_BIDIR_NORMALIZE | _lib.GDN_BIDIR_ELU1
    rc = _lib.load().linattn_bidir_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.t.data_ptr(), kv.t.data_ptr(),
                                       B, H, L, D, D, _lib.GDN_BF16, flags, ws.t.data_ptr(), wsb,
                                       torch.cuda.current_stream().cuda_stream)
    _lib.check(rc, "linattn_bidir_fwd")
    torch.cuda.synchronize()
    assert o.intact() and kv.intact() and ws.intact()
    ro, rkv = oracle.linattn_bidir(x["q"], x["k"], x["v"], normalize=True, elu1=True)
    assert max_rel_err(host(o.t), ro) <= TOL_BF16 and max_rel_err(host(kv.t), rkv) <= TOL_BF16


def test_decode_guard_bands():
    cfg = inputs.DECODE_256x32.with_(name="canary_decode", N=8, H=4)
    say(f"case {cfg.name}")
    st_np = inputs.decode_state(cfg)
    tok = inputs.decode_token(cfg, 0)
    st = Guarded(st_np.shape, torch.float32, fill=dev_tensor(st_np, torch.float32))
    o = Guarded(tok["v"].shape, torch.bfloat16)
    args = [dev_tensor(tok[n], torch.bfloat16) for n in ("q", "k", "v")] + \
           [dev_tensor(tok[n], torch.float32) for n in ("beta", "log_alpha")]
    ops.gdn_decode_step(*args, st.t, o=o.t)
    torch.cuda.synchronize()
    assert st.intact() and o.intact()
    ro, rst = oracle.gdn_decode_step(tok["q"], tok["k"], tok["v"], tok["beta"], tok["log_alpha"], st_np)
    assert max_rel_err(host(o.t), ro, axes=(2,)) <= TOL_BF16
    assert max_rel_err(host(st.t), rst) <= TOL_BF16
