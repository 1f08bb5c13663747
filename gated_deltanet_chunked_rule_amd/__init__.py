"""MI355X (gfx950) gated delta rule / causal linear attention: chunked prefill and decode.

The compute lives in libgdn.so (hand-written HIP, C ABI in include/gdn.h); `ops` wraps it for
PyTorch tensors, `inputs` draws the seeded synthetic workloads.
"""
__all__ = ["ops", "inputs", "build"]


def __getattr__(name):
    if name in ("gdn_prefill_fwd", "linattn_prefill_fwd", "gdn_decode_step", "prefill_workspace_size"):
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
