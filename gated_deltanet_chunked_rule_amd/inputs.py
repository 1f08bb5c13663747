"""Seeded synthetic inputs for the gated delta rule and plain causal linear attention.

This module only draws random numbers and rounds them to the storage dtype. It holds
none of the method's arithmetic, and both the fp64 oracle and the HIP path consume
exactly the arrays it returns (the GPU gets the rounded values, the oracle their exact
fp64 upcast), so a paired comparison on identical inputs is always possible (SparseGDN
article, fileenergy.com, section on checking the selector against the native kernel).

Recipe (one independent NumPy stream per tensor and per (batch, head) slice):
    rng = numpy.random.default_rng(SeedSequence([seed, tensor_id, stream_index]))
    tensor_id: q=0, k=1, v=2, beta=3, log_alpha=4, h0/state=5, log_alpha per key dimension=6
    stream_index: b*H + h for prefill; the decode step index for per-step decode inputs
    (0 for the decode state).
Values are drawn in fp64, transformed in fp64 and rounded once to the storage dtype
(bf16 by round-to-nearest-even straight from fp64, or fp32). Because each slice is its
own stream and rows are filled in order, a shorter L yields a prefix of a longer one.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

TID_Q, TID_K, TID_V, TID_BETA, TID_LOGA, TID_H0, TID_LOGA_VEC = range(7)


# ---------------------------------------------------------------------------
# rounding
# ---------------------------------------------------------------------------
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 (ties to even), returned as fp64.

    bf16 keeps 8 significant bits, i.e. the top 7 of fp64's 52 stored mantissa bits,
    so the rounding point is bit 45. Inputs here are finite and well inside bf16's
    normal range, where this bit trick is exact.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    return r.view(np.float64)


def round_fp32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of values that are already exactly bf16-representable."""
    f = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# distributions
# ---------------------------------------------------------------------------
def _rng(seed: int, tid: int, idx: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tid, idx]))


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, 1e-300)


def _elu_plus_one(x: np.ndarray) -> np.ndarray:
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.log1p(np.exp(-np.abs(x))) + np.maximum(x, 0.0)


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    H: int
    L: int
    Dk: int
    Dv: int
    dtype: str            # "bf16" or "f32": dtype of q, k, v and o
    seed: int
    qk: str = "l2"        # "l2": N(0,1) then L2-normalised per token; "elu1": elu(x)+1; "raw": N(0,1)
    gates: bool = True    # beta and log_alpha present (gated delta rule)
    gate_dist: str = "config"   # "config": log a = -softplus(N(0,1)+2); "long": -U(0, 0.01); "strong": -U(0, 8);
                                # "very_strong": -U(0, 40)
    h0: Optional[float] = 0.1   # std of the N(0, 0.01) initial state; None: no h0 (zeros)
    chunk: int = 64

    def with_(self, **kw) -> "PrefillConfig":
        return replace(self, **kw)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    N: int
    H: int
    Dk: int
    Dv: int
    dtype: str
    seed: int
    steps: int
    state_std: float = 0.1

    def with_(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)


# The five workloads (shapes, dtypes, value distributions). Seeds are 1000 + index.
GDN_REF_FP32 = PrefillConfig("gdn_ref_fp32_B1H2L512d64", 1, 2, 512, 64, 64, "f32", 1001, h0=None)
LINATTN_8K = PrefillConfig("linattn_B4H16L8192d128", 4, 16, 8192, 128, 128, "bf16", 1002,
                           qk="elu1", gates=False, h0=None)
GDN_32K = PrefillConfig("gdn_B1H32L32768d128", 1, 32, 32768, 128, 128, "bf16", 1003)
GDN_128K = PrefillConfig("gdn_B1H16L131072d128", 1, 16, 131072, 128, 128, "bf16", 1004)
DECODE_256x32 = DecodeConfig("decode_N256H32d128", 256, 32, 128, 128, "bf16", 1005, steps=100)

CONFIGS = {c.name: c for c in (GDN_REF_FP32, LINATTN_8K, GDN_32K, GDN_128K, DECODE_256x32)}


def _round(x, dtype):
    return round_bf16(x) if dtype == "bf16" else round_fp32(x)


def prefill_slice(cfg: PrefillConfig, b: int, h: int, L: Optional[int] = None) -> dict:
    """Inputs of one (b, h) slice as exact fp64 values of the stored dtype.

    Returns q [L,Dk], k [L,Dk], v [L,Dv], beta [L], log_alpha [L] (None when the config
    has no gates) and h0 [Dk,Dv] (None when absent). beta, log_alpha and h0 are fp32.
    """
    L = cfg.L if L is None else L
    idx = b * cfg.H + h
    out = {}
    for name, tid, d in (("q", TID_Q, cfg.Dk), ("k", TID_K, cfg.Dk)):
        x = _rng(cfg.seed, tid, idx).standard_normal((L, d))
        if cfg.qk == "l2":
            x = _l2_normalise(x)
        elif cfg.qk == "elu1":
            x = _elu_plus_one(x)
        elif cfg.qk != "raw":
            raise ValueError(cfg.qk)
        out[name] = _round(x, cfg.dtype)
    out["v"] = _round(_rng(cfg.seed, TID_V, idx).standard_normal((L, cfg.Dv)), cfg.dtype)
    if cfg.gates:
        out["beta"] = round_fp32(_sigmoid(_rng(cfg.seed, TID_BETA, idx).standard_normal(L)))
        r = _rng(cfg.seed, TID_LOGA, idx)
        if cfg.gate_dist == "config":
            la = -_softplus(r.standard_normal(L) + 2.0)
        elif cfg.gate_dist == "long":
            la = -r.uniform(0.0, 0.01, L)
        elif cfg.gate_dist == "strong":
            la = -r.uniform(0.0, 8.0, L)
        elif cfg.gate_dist == "very_strong":
            la = -r.uniform(0.0, 40.0, L)
        else:
            raise ValueError(cfg.gate_dist)
        out["log_alpha"] = round_fp32(la)
    else:
        out["beta"] = None
        out["log_alpha"] = None
    if cfg.h0 is not None:
        out["h0"] = round_fp32(cfg.h0 * _rng(cfg.seed, TID_H0, idx).standard_normal((cfg.Dk, cfg.Dv)))
    else:
        out["h0"] = None
    return out


def prefill_inputs(cfg: PrefillConfig, L: Optional[int] = None) -> dict:
    """Full [B,H,...] inputs (fp64 exact values), stacked from per-slice streams."""
    L = cfg.L if L is None else L
    sl = [[prefill_slice(cfg, b, h, L) for h in range(cfg.H)] for b in range(cfg.B)]
    out = {}
    for key in ("q", "k", "v", "beta", "log_alpha", "h0"):
        if sl[0][0][key] is None:
            out[key] = None
        else:
            out[key] = np.stack([np.stack([s[key] for s in row]) for row in sl])
    return out


def gate_vectors(cfg: PrefillConfig, L: Optional[int] = None) -> np.ndarray:
    """Log gates with one value per token and key dimension, [B,H,L,Dk] fp32 (exact fp64
    values): the config's gate distribution drawn independently for every key dimension, one
    stream per (b, h) slice (tensor_id 6), rows filled in token order."""
    L = cfg.L if L is None else L
    out = np.empty((cfg.B, cfg.H, L, cfg.Dk))
    for b in range(cfg.B):
        for h in range(cfg.H):
            r = _rng(cfg.seed, TID_LOGA_VEC, b * cfg.H + h)
            if cfg.gate_dist == "config":
                la = -_softplus(r.standard_normal((L, cfg.Dk)) + 2.0)
            elif cfg.gate_dist == "long":
                la = -r.uniform(0.0, 0.01, (L, cfg.Dk))
            elif cfg.gate_dist == "strong":
                la = -r.uniform(0.0, 8.0, (L, cfg.Dk))
            elif cfg.gate_dist == "very_strong":
                la = -r.uniform(0.0, 40.0, (L, cfg.Dk))
            else:
                raise ValueError(cfg.gate_dist)
            out[b, h] = round_fp32(la)
    return out


def decode_state(cfg: DecodeConfig) -> np.ndarray:
    """Initial decode state [N,H,Dk,Dv] fp32 values, N(0, 0.01)."""
    x = _rng(cfg.seed, TID_H0, 0).standard_normal((cfg.N, cfg.H, cfg.Dk, cfg.Dv))
    return round_fp32(cfg.state_std * x)


def decode_token(cfg: DecodeConfig, step: int) -> dict:
    """One new token per (sequence, head): q,k [N,H,Dk] L2-normalised, v [N,H,Dv],
    beta, log_alpha [N,H]."""
    shp = (cfg.N, cfg.H)
    q = _l2_normalise(_rng(cfg.seed, TID_Q, step).standard_normal(shp + (cfg.Dk,)))
    k = _l2_normalise(_rng(cfg.seed, TID_K, step).standard_normal(shp + (cfg.Dk,)))
    v = _rng(cfg.seed, TID_V, step).standard_normal(shp + (cfg.Dv,))
    beta = _sigmoid(_rng(cfg.seed, TID_BETA, step).standard_normal(shp))
    la = -_softplus(_rng(cfg.seed, TID_LOGA, step).standard_normal(shp) + 2.0)
    return {"q": _round(q, cfg.dtype), "k": _round(k, cfg.dtype), "v": _round(v, cfg.dtype),
            "beta": round_fp32(beta), "log_alpha": round_fp32(la)}
