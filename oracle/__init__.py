"""fp64 CPU oracle (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. The product path (``gated_deltanet_chunked_rule_amd``) never imports
it, and it never imports the product path: the two share no code.

The token-by-token arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, OpenMP over
independent slices); this module compiles it with gcc on first use and marshals NumPy arrays.
The chunked form with the block-adjacent intra-chunk solve is NumPy fp64 in ``banded.py``.

    gdn_prefill(q, k, v, beta, log_alpha, h0)  -> (o, h_final)   gated delta rule
    linattn_prefill(q, k, v, h0)               -> (o, h_final)   S_t = S_{t-1} + v_t k_t^T
    gla_prefill(q, k, v, log_alpha, h0)        -> (o, h_final)   S_t = a_t S_{t-1} + v_t k_t^T
    gla_vec_prefill(q, k, v, log_alpha, h0)    -> (o, h_final)   S_t = S_{t-1} diag(a_t) + v_t k_t^T,
                                                                 a gate per key dimension
    gdn_prefill_skip(q, k, v, beta, log_alpha, keep, h0, chunk)  gated delta rule, skipped chunks
                                                                 only decay the carried state
    gdn_decode_step(q, k, v, beta, log_alpha, state) -> (o, new_state)
    linattn_bidir(q, k, v, normalize, elu1)    -> (o, kv)        non-causal: KV = sum phi(k) v^T,
                                                                 o = phi(q) KV [/ phi(q).sum phi(k)]
    gdn_prefill_banded(q, k, v, beta, log_alpha, h0, band)       chunked form with the intra-chunk
                                                                 inverse cut to `band` blocks below
                                                                 its diagonal (oracle/banded.py, NumPy)

Shapes: q,k [B,H,L,Dk]; v [B,H,L,Dv]; beta, log_alpha [B,H,L]; h0/h_final [B,H,Dk,Dv]
(key-major, element [i][j] = S[j][i]); gla_vec_prefill's log_alpha [B,H,L,Dk]; decode: q,k [N,H,Dk], v [N,H,Dv], beta/log_alpha
[N,H], state [N,H,Dk,Dv]. All results are fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

last_threads = 0  # threads the last call used


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                               "-std=c99", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB)
            P = ctypes.POINTER(ctypes.c_double)
            i = ctypes.c_int
            lib.oracle_gdn_prefill.argtypes = [P, P, P, P, P, P, P, P, i, i, i, i, i, i]
            lib.oracle_linattn_prefill.argtypes = [P, P, P, P, P, P, i, i, i, i, i, i]
            lib.oracle_gdn_decode_step.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i]
            lib.oracle_gla_prefill.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, i]
            lib.oracle_gla_vec_prefill.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, i]
            lib.oracle_linattn_bidir.argtypes = [P, P, P, P, P, i, i, i, i, i, i, i]
            IP = ctypes.POINTER(ctypes.c_int)
            lib.oracle_gdn_prefill_skip.argtypes = [P, P, P, P, P, P, IP, i, P, P, i, i, i, i, i, i]
            for f in (lib.oracle_gdn_prefill, lib.oracle_linattn_prefill, lib.oracle_gdn_decode_step,
                      lib.oracle_gla_prefill, lib.oracle_gla_vec_prefill, lib.oracle_gdn_prefill_skip,
                      lib.oracle_linattn_bidir):
                f.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _as4(x, n):
    """Accept [L,D] / [H,L,D] / [B,H,L,D] style inputs by adding leading axes."""
    while x.ndim < n:
        x = x[None]
    return x


def gdn_prefill(q, k, v, beta, log_alpha, h0=None, nthreads: int = 0):
    global last_threads
    q, k, v = (_as4(_f64(t), 4) for t in (q, k, v))
    beta, log_alpha = (_as4(_f64(t), 3) for t in (beta, log_alpha))
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, L)
    assert beta.shape == (B, H, L) and log_alpha.shape == (B, H, L)
    if h0 is not None:
        h0 = _as4(_f64(h0), 4)
        assert h0.shape == (B, H, Dk, Dv)
    o = np.empty((B, H, L, Dv))
    hf = np.empty((B, H, Dk, Dv))
    last_threads = _load().oracle_gdn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
                                              _ptr(h0), _ptr(o), _ptr(hf), B, H, L, Dk, Dv, nthreads)
    return o, hf


def linattn_prefill(q, k, v, h0=None, nthreads: int = 0):
    global last_threads
    q, k, v = (_as4(_f64(t), 4) for t in (q, k, v))
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, L)
    if h0 is not None:
        h0 = _as4(_f64(h0), 4)
        assert h0.shape == (B, H, Dk, Dv)
    o = np.empty((B, H, L, Dv))
    hf = np.empty((B, H, Dk, Dv))
    last_threads = _load().oracle_linattn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(h0), _ptr(o), _ptr(hf),
                                                  B, H, L, Dk, Dv, nthreads)
    return o, hf


def gla_prefill(q, k, v, log_alpha, h0=None, nthreads: int = 0):
    """Decay-only gated linear attention: S_t = exp(log_alpha_t) S_{t-1} + v_t k_t^T, o_t = S_t q_t."""
    global last_threads
    q, k, v = (_as4(_f64(t), 4) for t in (q, k, v))
    log_alpha = _as4(_f64(log_alpha), 3)
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, L) and log_alpha.shape == (B, H, L)
    if h0 is not None:
        h0 = _as4(_f64(h0), 4)
        assert h0.shape == (B, H, Dk, Dv)
    o = np.empty((B, H, L, Dv))
    hf = np.empty((B, H, Dk, Dv))
    last_threads = _load().oracle_gla_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(h0), _ptr(o),
                                              _ptr(hf), B, H, L, Dk, Dv, nthreads)
    return o, hf


def gla_vec_prefill(q, k, v, log_alpha, h0=None, nthreads: int = 0):
    """Gated linear attention with a gate per key dimension: S_t = S_{t-1} diag(exp(log_alpha_t))
    + v_t k_t^T, o_t = S_t q_t; log_alpha [B,H,L,Dk]."""
    global last_threads
    q, k, v, log_alpha = (_as4(_f64(t), 4) for t in (q, k, v, log_alpha))
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, L) and log_alpha.shape == q.shape
    if h0 is not None:
        h0 = _as4(_f64(h0), 4)
        assert h0.shape == (B, H, Dk, Dv)
    o = np.empty((B, H, L, Dv))
    hf = np.empty((B, H, Dk, Dv))
    last_threads = _load().oracle_gla_vec_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(h0), _ptr(o),
                                                  _ptr(hf), B, H, L, Dk, Dv, nthreads)
    return o, hf


def gdn_prefill_skip(q, k, v, beta, log_alpha, keep, h0=None, chunk: int = 64, nthreads: int = 0):
    """Gated delta rule with skipped chunk updates; keep [B,H,ceil(L/chunk)] (nonzero = keep)."""
    global last_threads
    q, k, v = (_as4(_f64(t), 4) for t in (q, k, v))
    beta, log_alpha = (_as4(_f64(t), 3) for t in (beta, log_alpha))
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    nch = (L + chunk - 1) // chunk
    keep = np.ascontiguousarray(_as4(np.asarray(keep), 3), dtype=np.int32)
    assert keep.shape == (B, H, nch)
    if h0 is not None:
        h0 = _as4(_f64(h0), 4)
        assert h0.shape == (B, H, Dk, Dv)
    o = np.empty((B, H, L, Dv))
    hf = np.empty((B, H, Dk, Dv))
    last_threads = _load().oracle_gdn_prefill_skip(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha), _ptr(h0),
        keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), chunk, _ptr(o), _ptr(hf), B, H, L, Dk, Dv, nthreads)
    return o, hf


def gdn_decode_step(q, k, v, beta, log_alpha, state, nthreads: int = 0):
    """Returns (o [N,H,Dv], new_state [N,H,Dk,Dv]); the input state is not modified."""
    global last_threads
    q, k, v = (_as4(_f64(t), 3) for t in (q, k, v))
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    beta = _as4(_f64(beta), 2)
    log_alpha = _as4(_f64(log_alpha), 2)
    st = np.array(_as4(_f64(state), 4), dtype=np.float64, copy=True)
    assert st.shape == (N, H, Dk, Dv) and beta.shape == (N, H) and log_alpha.shape == (N, H)
    o = np.empty((N, H, Dv))
    last_threads = _load().oracle_gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
                                                  _ptr(st), _ptr(o), N, H, Dk, Dv, nthreads)
    return o, st


def linattn_bidir(q, k, v, normalize: bool = True, elu1: bool = True, nthreads: int = 0):
    """Bidirectional linear attention (datadaily.news overview, section "Linear attention"):
    KV = sum_n phi(k_n) v_n^T, o_n = phi(q_n)^T KV, divided by Z_n = phi(q_n) . sum_m phi(k_m)
    when normalize; phi = elu + 1 when elu1, else the identity. Returns (o, kv), kv [B,H,Dk,Dv]."""
    global last_threads
    q, k, v = (_as4(_f64(t), 4) for t in (q, k, v))
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, L)
    o = np.empty((B, H, L, Dv))
    kv = np.empty((B, H, Dk, Dv))
    flags = (1 if normalize else 0) | (2 if elu1 else 0)
    last_threads = _load().oracle_linattn_bidir(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(kv), B, H, L, Dk, Dv,
                                                flags, nthreads)
    return o, kv


from .banded import gdn_prefill_banded  # noqa: E402,F401
