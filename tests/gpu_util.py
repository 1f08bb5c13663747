"""Helpers for the GPU parity tests: move generator arrays to the device, compare with the oracle."""
import sys

import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None


def say(msg):
    """Name the case before each GPU step, flushed, so a failing run says where it was."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensor(x, dtype):
    """Exact fp64 values of the storage dtype -> device tensor of that dtype."""
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to("cuda").to(dtype).contiguous()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_rel_err(got, ref, axes=None):
    """max |got - ref| / max |ref| per leading slice, maximised over slices (fp64).

    `axes` are the trailing axes that form one slice (default: all but the first two)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if axes is None:
        axes = tuple(range(2, ref.ndim))
    num = np.abs(got - ref).max(axis=axes)
    den = np.abs(ref).max(axis=axes)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


TOL_BF16 = 2e-2   # bf16 inputs: max relative error bound per (b, h) slice, o and final state
TOL_F32 = 1e-4    # fp32 inputs


def prefill_workspace(torch, B, H, D, nblocks):
    """A gated delta-rule prefill workspace that holds `nblocks` blocks per (batch, head): the call
    then uses that many blocks (at most its preferred count and one per chunk)."""
    flags = 0 if nblocks <= 1 else ((nblocks - 1) * 4 + 255) // 256 * 256
    n = B * H * ((2 * nblocks - 1) * 4 * D * D + flags)
    return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
