"""PyTorch-facing wrappers of the C ABI (include/gdn.h).

PyTorch supplies device memory and the current stream; every step of the computation runs in
libgdn's HIP kernels. These functions only check tensors and pass pointers. There is no CPU or
PyTorch fallback: if libgdn.so is missing or the device is not gfx950 they raise.

Layouts (row-major, contiguous):
    q, k [B,H,L,D]; v, o [B,H,L,D]; beta, log_alpha [B,H,L] fp32; h0, h_final [B,H,D,D] fp32,
    key-major (element [i][j] is S[j][i]). Decode: q, k, v, o [N,H,D]; beta, log_alpha [N,H];
    state [N,H,D,D] fp32 updated in place.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib

_DT = {torch.bfloat16: _lib.GDN_BF16, torch.float32: _lib.GDN_F32}


def _code(dtype: torch.dtype) -> int:
    if dtype not in _DT:
        raise TypeError(f"q/k/v must be bfloat16 or float32, got {dtype}")
    return _DT[dtype]


def _req(name, t, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _p(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device, stream) -> int:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def prefill_workspace_size(B: int, H: int, L: int, D: int, dtype: torch.dtype) -> int:
    return int(_lib.load().gdn_prefill_workspace_size(B, H, L, D, D, _code(dtype)))


def gdn_prefill_timing(enable: bool) -> None:
    """Turn per-kernel HIP-event timing of the gated delta-rule prefill calls on or off."""
    _lib.check(_lib.load().gdn_prefill_timing(1 if enable else 0), "gdn_prefill_timing")


def gdn_prefill_kernel_times() -> dict:
    """Summed ms and launch counts of the block-map, block-pass and output kernels since the last
    query (waits for the recorded events, then clears them)."""
    import ctypes
    ms = (ctypes.c_float * 3)()
    n = (ctypes.c_int * 3)()
    _lib.check(_lib.load().gdn_prefill_kernel_times(ctypes.addressof(ms), ctypes.addressof(n)),
               "gdn_prefill_kernel_times")
    return {name: {"ms": float(ms[i]), "launches": int(n[i])} for i, name in enumerate(("map", "scan", "out"))}


def linattn_prefill_workspace_size(B: int, H: int, L: int, D: int, dtype: torch.dtype) -> int:
    return int(_lib.load().linattn_prefill_workspace_size(B, H, L, D, D, _code(dtype)))


def _prefill(entry, q, k, v, beta, log_alpha, h0, o, h_final, workspace, stream, delta, keep=None, band=None):
    B, H, L, D = q.shape
    dev, dt = q.device, q.dtype
    _req("q", q, (B, H, L, D), dt, dev)
    _req("k", k, (B, H, L, D), dt, dev)
    _req("v", v, (B, H, L, D), dt, dev)
    if delta:
        _req("beta", beta, (B, H, L), torch.float32, dev)
    if delta or log_alpha is not None:
        _req("log_alpha", log_alpha, (B, H, L), torch.float32, dev)
    if entry == "gdn_prefill_skip_fwd":
        _req("keep", keep, (B, H, (L + 63) // 64), torch.uint8, dev)
    if h0 is not None:
        _req("h0", h0, (B, H, D, D), torch.float32, dev)
    o = torch.empty_like(v) if o is None else _req("o", o, (B, H, L, D), dt, dev)
    if h_final is None:
        h_final = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    _req("h_final", h_final, (B, H, D, D), torch.float32, dev)
    if workspace is None:   # the preferred size; any size the C ABI accepts works (it checks)
        size = prefill_workspace_size if delta else linattn_prefill_workspace_size
        workspace = torch.empty(max(size(B, H, L, D, dt), 1), dtype=torch.uint8, device=dev)
    elif not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    lib = _lib.load()
    gates = (_p(q), _p(k), _p(v), _p(beta), _p(log_alpha))
    if entry == "gdn_prefill_skip_fwd":
        gates = gates + (_p(keep),)
    dims = (B, H, L, D, D, _code(dt)) + ((band,) if entry == "gdn_prefill_banded_fwd" else ())
    rc = getattr(lib, entry)(*gates, _p(h0), _p(o), _p(h_final), *dims, _p(workspace),
                             workspace.numel() * workspace.element_size(), _stream(dev, stream))
    _lib.check(rc, entry)
    return o, h_final


def gdn_prefill_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                    log_alpha: torch.Tensor, h0: Optional[torch.Tensor] = None, *,
                    o: Optional[torch.Tensor] = None, h_final: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunked gated delta-rule prefill. Returns (o, h_final)."""
    return _prefill("gdn_prefill_fwd", q, k, v, beta, log_alpha, h0, o, h_final, workspace, stream, True)


def gdn_prefill_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                            log_alpha: torch.Tensor, h0: Optional[torch.Tensor], o: torch.Tensor,
                            h_final: torch.Tensor, scratch_bytes: Optional[int] = None, *,
                            stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """gdn_prefill_fwd with the library's static per-device scratch as its workspace; allocates
    nothing (o and h_final are required). scratch_bytes: how much of the scratch to use, default
    the preferred workspace size capped at GDN_PREFILL_NOALLOC_MAX_BYTES. Returns (o, h_final)."""
    B, H, L, D = q.shape
    dev, dt = q.device, q.dtype
    for name, t in (("q", q), ("k", k), ("v", v)):
        _req(name, t, (B, H, L, D), dt, dev)
    _req("beta", beta, (B, H, L), torch.float32, dev)
    _req("log_alpha", log_alpha, (B, H, L), torch.float32, dev)
    if h0 is not None:
        _req("h0", h0, (B, H, D, D), torch.float32, dev)
    _req("o", o, (B, H, L, D), dt, dev)
    _req("h_final", h_final, (B, H, D, D), torch.float32, dev)
    if scratch_bytes is None:
        scratch_bytes = min(prefill_workspace_size(B, H, L, D, dt), _lib.GDN_PREFILL_NOALLOC_MAX_BYTES)
    rc = _lib.load().gdn_prefill_fwd_noalloc(_p(q), _p(k), _p(v), _p(beta), _p(log_alpha), _p(h0), _p(o),
                                             _p(h_final), B, H, L, D, D, _code(dt), int(scratch_bytes),
                                             _stream(dev, stream))
    _lib.check(rc, "gdn_prefill_fwd_noalloc")
    return o, h_final


def gdn_prefill_skip_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                         log_alpha: torch.Tensor, keep: torch.Tensor, h0: Optional[torch.Tensor] = None, *,
                         o: Optional[torch.Tensor] = None, h_final: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Gated delta rule whose chunks (64 tokens) with keep == 0 only decay the carried state; every
    token still gets its output. keep: uint8 [B,H,ceil(L/64)]. Returns (o, h_final)."""
    return _prefill("gdn_prefill_skip_fwd", q, k, v, beta, log_alpha, h0, o, h_final, workspace, stream, True,
                    keep=keep)


def gdn_prefill_banded_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                           log_alpha: torch.Tensor, h0: Optional[torch.Tensor] = None, *, band: int = 1,
                           o: Optional[torch.Tensor] = None, h_final: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Gated delta rule with the block-adjacent intra-chunk solve: the blocks of each chunk's
    (I + A)^-1 more than `band` 16 x 16 block rows below the diagonal are zero (band 3: exact).
    Returns (o, h_final)."""
    return _prefill("gdn_prefill_banded_fwd", q, k, v, beta, log_alpha, h0, o, h_final, workspace, stream, True,
                    band=band)


def linattn_prefill_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, h0: Optional[torch.Tensor] = None, *,
                        log_alpha: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                        h_final: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunked causal linear attention S_t = a_t S_{t-1} + v_t k_t^T (a_t = exp(log_alpha), 1 when
    log_alpha is None). Returns (o, h_final)."""
    return _prefill("linattn_prefill_fwd", q, k, v, None, log_alpha, h0, o, h_final, workspace, stream, False)


def gla_prefill_workspace_size(B: int, H: int, L: int, D: int, dtype: torch.dtype) -> int:
    return int(_lib.load().gla_prefill_workspace_size(B, H, L, D, D, _code(dtype)))


def gla_prefill_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
                    h0: Optional[torch.Tensor] = None, *, o: Optional[torch.Tensor] = None,
                    h_final: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Gated linear attention with a gate per key dimension: S_t = S_{t-1} diag(exp(log_alpha_t))
    + v_t k_t^T, o_t = S_t q_t; log_alpha fp32 [B,H,L,D]. Returns (o, h_final)."""
    B, H, L, D = q.shape
    dev, dt = q.device, q.dtype
    _req("q", q, (B, H, L, D), dt, dev)
    _req("k", k, (B, H, L, D), dt, dev)
    _req("v", v, (B, H, L, D), dt, dev)
    _req("log_alpha", log_alpha, (B, H, L, D), torch.float32, dev)
    if h0 is not None:
        _req("h0", h0, (B, H, D, D), torch.float32, dev)
    o = torch.empty_like(v) if o is None else _req("o", o, (B, H, L, D), dt, dev)
    if h_final is None:
        h_final = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    _req("h_final", h_final, (B, H, D, D), torch.float32, dev)
    if workspace is None:
        workspace = torch.empty(max(gla_prefill_workspace_size(B, H, L, D, dt), 1), dtype=torch.uint8, device=dev)
    elif not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    rc = _lib.load().gla_prefill_fwd(_p(q), _p(k), _p(v), _p(log_alpha), _p(h0), _p(o), _p(h_final), B, H, L, D, D,
                                     _code(dt), _p(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(dev, stream))
    _lib.check(rc, "gla_prefill_fwd")
    return o, h_final


def gdn_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                    log_alpha: torch.Tensor, state: torch.Tensor, *, o: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """One decode token per (sequence, head); `state` is updated in place. Returns o."""
    N, H, D = q.shape
    dev, dt = q.device, q.dtype
    _req("q", q, (N, H, D), dt, dev)
    _req("k", k, (N, H, D), dt, dev)
    _req("v", v, (N, H, D), dt, dev)
    _req("beta", beta, (N, H), torch.float32, dev)
    _req("log_alpha", log_alpha, (N, H), torch.float32, dev)
    _req("state", state, (N, H, D, D), torch.float32, dev)
    o = torch.empty_like(v) if o is None else _req("o", o, (N, H, D), dt, dev)
    rc = _lib.load().gdn_decode_step(_p(q), _p(k), _p(v), _p(beta), _p(log_alpha), _p(state), _p(o),
                                     N, H, D, D, _code(dt), _stream(dev, stream))
    _lib.check(rc, "gdn_decode_step")
    return o


def linattn_bidir_workspace_size(B: int, H: int, L: int, D: int, dtype: torch.dtype) -> int:
    return int(_lib.load().linattn_bidir_workspace_size(B, H, L, D, D, _code(dtype)))


def linattn_bidir_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, normalize: bool = True,
                      elu1: bool = True, kv_out: bool = False, o: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None):
    """Bidirectional (non-causal) linear attention: KV = sum_n phi(k_n) v_n^T, o_n = phi(q_n)^T KV,
    divided by phi(q_n) . sum_m phi(k_m) when normalize; phi = elu + 1 when elu1, else identity.
    Returns o, or (o, kv) with kv [B,H,D,D] fp32 when kv_out."""
    B, H, L, D = q.shape
    dev, dt = q.device, q.dtype
    _req("q", q, (B, H, L, D), dt, dev)
    _req("k", k, (B, H, L, D), dt, dev)
    _req("v", v, (B, H, L, D), dt, dev)
    o = torch.empty_like(v) if o is None else _req("o", o, (B, H, L, D), dt, dev)
    kv = torch.empty((B, H, D, D), dtype=torch.float32, device=dev) if kv_out else None
    if workspace is None:
        workspace = torch.empty(max(linattn_bidir_workspace_size(B, H, L, D, dt), 1), dtype=torch.uint8, device=dev)
    elif not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    flags = (_lib.GDN_BIDIR_NORMALIZE if normalize else 0) | (_lib.GDN_BIDIR_ELU1 if elu1 else 0)
    rc = _lib.load().linattn_bidir_fwd(_p(q), _p(k), _p(v), _p(o), _p(kv), B, H, L, D, D, _code(dt), flags,
                                       _p(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(dev, stream))
    _lib.check(rc, "linattn_bidir_fwd")
    return (o, kv) if kv_out else o
