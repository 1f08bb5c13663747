#!/usr/bin/env python3
"""Benchmark of the gated delta-rule hot path on one MI355X.

A step is one chunked GDN prefill of the long-context workload (B=1, H=16, L=131072, d=128,
chunk 64: bf16 q/k/v, fp32 gates and state) through the C ABI, inputs resident in HBM. The call
runs three kernels in order on one stream (block maps, the pass over blocks, outputs); the
roofline is that of the output kernel, which does every step of the chunked algorithm for every
chunk and dominates the call, timed live with the library's per-kernel HIP events. The JSON line
also carries the decode step (256 sequences x 32 heads, 100 in-place steps, state GB/s), plain
causal linear attention (B=4, H=16, L=8192), the 32K GDN workload, the 128K workload with
long-memory gates, the skip and banded variants as components, hardware-counter figures taken
with rocprofv3 on the same kernel sources, and the fp64 oracle timed on this host's cores on a
bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
    python bench.py --counters DIR   # per-kernel bytes and MFMA work from rocprofv3 counter CSVs
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from gated_deltanet_chunked_rule_amd import inputs  # noqa: E402

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
METRIC = "GDN prefill tokens/s at L=128K + % bf16 MFMA peak; decode state GB/s"

# Hardware counters of one 128K prefill call per kernel (rocprofv3 --pmc runs of
# `bench.py --profile-steps 2 --warmup 1`, one counter set per run, read with
# `bench.py --counters DIR`): HBM bytes = FETCH_SIZE and WRITE_SIZE, each divided by what the
# counter reads per byte of a plain device copy of 1 GiB; MFMA flops = 512 x the MOPS counters.
# The commands and raw figures are in profiles/gdn_prefill_B1H16L131072_counters.md. Valid only
# for the kernel sources they were taken on: bench.py reports them only while
# kernel_source_hash() still matches.
COUNTERS_128K = {
    "source_hash": "d92168036b3ea98d",
    "fetch_factor": 0.5000172654787699,
    "write_factor": 1.0,
    "map": {
        "fetch_kib": 32373.5,
        "write_kib": 31759.5,
        "hbm_bytes": 98820366.64452402,
        "mfma_bf16_flops": 6891241472.0,
        "mfma_f32_flops": 154402816.0,
        "mfma_busy_frac": 0.10039755458073331
    },
    "scan": {
        "fetch_kib": 544.5,
        "write_kib": 1024.0,
        "hbm_bytes": 2163673.4946157606,
        "mfma_bf16_flops": 0.0,
        "mfma_f32_flops": 0.0,
        "mfma_busy_frac": 0.0
    },
    "out": {
        "fetch_kib": 811200.859375,
        "write_kib": 525312.8515625,
        "hbm_bytes": 2199202354.3419914,
        "mfma_bf16_flops": 343597383680.0,
        "mfma_f32_flops": 5100273664.0,
        "mfma_busy_frac": 0.32052897430085
    }
}


# the sources the gated delta-rule prefill's kernels and their launcher are built from (the host-side
# argument checks and declarations do not change what the kernels read and write)
PREFILL_SOURCES = ("gdn_device.h", "gdn_mfma.h", "gdn_prefill.hip", "gdn_rows.h")
KERNELS = {"map": "map_kernel", "scan": "scan_kernel", "out": "out_kernel"}


def kernel_source_hash():
    """sha256 over the sources of the gated delta-rule prefill (sorted by name)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_deltanet_chunked_rule_amd", "csrc")
    for name in sorted(PREFILL_SOURCES):
        h.update(name.encode())
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------------------------
# algorithmic work (what the method must compute / move), per workload
# ---------------------------------------------------------------------------------------------
def gdn_flops_per_chunk(C=64, d=128):
    """Triangles counted exactly: 3 state GEMMs (W H, e^g Q H, Khat^T U), K K^T strictly lower,
    Q K^T lower, T (beta e^g K), T (beta V), P U, and the triangular inverse."""
    return (6 * C * d * d + C * (C - 1) * d + C * (C + 1) * d + C * (C - 1) * d + C * (C - 1) * d
            + C * (C + 1) * d + C ** 3 / 3)


def gdn_dense_tile_flops_per_chunk(C=64, d=128):
    """The same products on whole 64 x 64 tiles (what MFMA tiles execute at the least)."""
    return 6 * C * d * d + 10 * C * C * d + C ** 3 / 3


def linattn_flops_per_chunk(C=64, d=128):
    return 4 * C * d * d + 2 * C * (C + 1) * d


def prefill_bytes(cfg, gates=True):
    tok = cfg.B * cfg.H * cfg.L
    e = 2 if cfg.dtype == "bf16" else 4
    b = 3 * tok * cfg.Dk * e + tok * cfg.Dv * e          # q, k, v in; o out
    if gates:
        b += 2 * tok * 4                                   # beta, log_alpha
    st = cfg.B * cfg.H * cfg.Dk * cfg.Dv * 4
    b += st + (st if cfg.h0 is not None else 0)            # h_final out, h0 in
    return b


def out_kernel_bytes(cfg):
    """Algorithmic bytes of the output kernel when the call uses several blocks per slice: every
    token's q, k, v, beta and log_alpha read and o written once, and the final state written (the
    initial state is read by the pass over blocks)."""
    st = cfg.B * cfg.H * cfg.Dk * cfg.Dv * 4
    return prefill_bytes(cfg) - (st if cfg.h0 is not None else 0)


def decode_bytes(cfg):
    S = cfg.N * cfg.H
    e = 2 if cfg.dtype == "bf16" else 4
    state = S * cfg.Dk * cfg.Dv * 4
    return 2 * state + S * (2 * cfg.Dk + 2 * cfg.Dv) * e + 2 * S * 4, 2 * state


# ---------------------------------------------------------------------------------------------
# hardware counters (rocprofv3 CSVs)
# ---------------------------------------------------------------------------------------------
def _counter_rows(path):
    import csv
    rows = {}
    for r in csv.DictReader(open(path)):
        rows.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    return rows


def _find_csv(d, sub):
    for root, _, files in os.walk(os.path.join(d, sub)):
        for f in files:
            if f.endswith("counter_collection.csv"):
                return os.path.join(root, f)
    raise FileNotFoundError(os.path.join(d, sub))


def counters_from(d):
    """Per-launch counter figures of the prefill kernels from rocprofv3 runs under directory d:
    fetch/ (FETCH_SIZE), write/ (WRITE_SIZE), cfetch/ and cwrite/ (the same counters on a 1 GiB
    device copy, `bench.py --copy-calibrate 1073741824`), mfma/ (SQ_INSTS_VALU_MFMA_MOPS_BF16,
    SQ_INSTS_VALU_MFMA_MOPS_F32, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE), and source_hash.txt
    (`bench.py --source-hash` run with them). The first call of each kernel (warm-up) is dropped
    and the others averaged."""
    gib_kib = float(1 << 20)

    def calib(sub, counter):
        rows = _counter_rows(_find_csv(d, sub))
        vals = [v for (k, c), vs in rows.items() if "copyBuffer" in k and c == counter for v in vs if v > 0.4 * gib_kib]
        return sum(vals) / len(vals) / gib_kib     # counter KiB per KiB copied

    f_fetch, f_write = calib("cfetch", "FETCH_SIZE"), calib("cwrite", "WRITE_SIZE")
    runs = {"fetch": _counter_rows(_find_csv(d, "fetch")), "write": _counter_rows(_find_csv(d, "write"))}
    try:
        runs["mfma"] = _counter_rows(_find_csv(d, "mfma"))
    except FileNotFoundError:
        runs["mfma"] = {}
    # the kernel sources the runs were taken on (written next to them by `bench.py --source-hash`)
    hp = os.path.join(d, "source_hash.txt")
    out = {"source_hash": open(hp).read().strip() if os.path.exists(hp) else None,
           "fetch_factor": f_fetch, "write_factor": f_write}
    for short, kname in KERNELS.items():
        def avg(run, counter):
            vals = [vs for (k, c), vs in runs[run].items() if f"gdn::{kname}<128, gdn::BF16" in k and c == counter]
            if not vals:
                return None
            v = vals[0][1:] if len(vals[0]) > 1 else vals[0]
            return sum(v) / len(v)
        fk, wk = avg("fetch", "FETCH_SIZE"), avg("write", "WRITE_SIZE")
        if fk is None:
            continue
        rec = {"fetch_kib": fk, "write_kib": wk, "hbm_bytes": (fk / f_fetch + wk / f_write) * 1024}
        mb, mf = avg("mfma", "SQ_INSTS_VALU_MFMA_MOPS_BF16"), avg("mfma", "SQ_INSTS_VALU_MFMA_MOPS_F32")
        if mb is not None:
            rec["mfma_bf16_flops"] = 512 * mb
            rec["mfma_f32_flops"] = 512 * (mf or 0.0)
            busy, active = avg("mfma", "SQ_VALU_MFMA_BUSY_CYCLES"), avg("mfma", "GRBM_GUI_ACTIVE")
            if busy is not None and active:
                # GRBM_GUI_ACTIVE comes summed over the 8 XCDs; busy cycles summed over all 1024 SIMDs
                rec["mfma_busy_frac"] = busy / (active / 8 * 4 * 256)
        out[short] = rec
    return out


# ---------------------------------------------------------------------------------------------
# device inputs
# ---------------------------------------------------------------------------------------------
def to_dev(torch, x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(dtype)


def prefill_device_inputs(torch, cfg, gates=True, verbose=False):
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shp = (cfg.B, cfg.H, cfg.L)
    q = torch.empty(shp + (cfg.Dk,), dtype=dt, device="cuda")
    k, v = torch.empty_like(q), torch.empty_like(q)
    beta = torch.empty(shp, device="cuda") if gates else None
    la = torch.empty(shp, device="cuda") if gates else None
    h0 = torch.empty((cfg.B, cfg.H, cfg.Dk, cfg.Dv), device="cuda") if cfg.h0 is not None else None
    for b in range(cfg.B):
        for h in range(cfg.H):
            if verbose:
                print(f"inputs: slice {b * cfg.H + h + 1} of {cfg.B * cfg.H}", file=sys.stderr, flush=True)
            s = inputs.prefill_slice(cfg, b, h)
            for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("log_alpha", la), ("h0", h0)):
                if t is not None:
                    t[b, h] = to_dev(torch, s[name], t.dtype)
    return q, k, v, beta, la, h0


def time_loop(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


# ---------------------------------------------------------------------------------------------
# components
# ---------------------------------------------------------------------------------------------
def bench_prefill(torch, ops, cfg, steps, warmup, gdn=True, verbose=False, variant=None, keep_rate=0.29,
                  kernel_times=False):
    """variant None: gdn_prefill_fwd (gdn) or plain linattn_prefill_fwd; "gla": linattn_prefill_fwd with
    per-token gates; "gla_vec": gla_prefill_fwd with a gate per token and key dimension; "skip":
    gdn_prefill_skip_fwd with a seeded keep mask at keep_rate; "band1":
    gdn_prefill_banded_fwd with band 1 (flops counted as for the exact rule). kernel_times (gated
    delta rule only): after the timed loop, time `steps` more calls with the library's per-kernel HIP
    events (recorded on the call's stream around each of its kernels) and report each kernel's
    average launch duration."""
    gates = gdn or variant == "gla"
    q, k, v, beta, la, h0 = prefill_device_inputs(torch, cfg, gates=gates, verbose=verbose)
    if variant == "gla_vec":
        la = torch.from_numpy(inputs.gate_vectors(cfg).astype(np.float32)).cuda()
    o = torch.empty_like(v)
    hf = torch.empty((cfg.B, cfg.H, cfg.Dk, cfg.Dv), device="cuda")
    nchk = (cfg.L + 63) // 64
    if variant == "gla_vec":
        wsb = ops.gla_prefill_workspace_size(cfg.B, cfg.H, cfg.L, cfg.Dk, q.dtype)
    elif not gates or variant == "gla":   # linear attention: blocks of chunks
        wsb = ops.linattn_prefill_workspace_size(cfg.B, cfg.H, cfg.L, cfg.Dk, q.dtype)
    else:
        wsb = ops.prefill_workspace_size(cfg.B, cfg.H, cfg.L, cfg.Dk, q.dtype)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    nchunk = cfg.B * cfg.H * nchk
    kept = nchunk
    if variant == "skip":
        keep_np = (np.random.default_rng(cfg.seed).random((cfg.B, cfg.H, nchk)) < keep_rate).astype(np.uint8)
        kept = int(keep_np.sum())
        keep = torch.from_numpy(keep_np).cuda()
        fn = lambda: ops.gdn_prefill_skip_fwd(q, k, v, beta, la, keep, h0, o=o, h_final=hf, workspace=ws)
    elif variant == "band1":
        fn = lambda: ops.gdn_prefill_banded_fwd(q, k, v, beta, la, h0, band=1, o=o, h_final=hf, workspace=ws)
    elif gdn:
        fn = lambda: ops.gdn_prefill_fwd(q, k, v, beta, la, h0, o=o, h_final=hf, workspace=ws)
    elif variant == "gla":
        fn = lambda: ops.linattn_prefill_fwd(q, k, v, h0, log_alpha=la, o=o, h_final=hf, workspace=ws)
    elif variant == "gla_vec":
        fn = lambda: ops.gla_prefill_fwd(q, k, v, la, h0, o=o, h_final=hf, workspace=ws)
    else:
        fn = lambda: ops.linattn_prefill_fwd(q, k, v, h0, o=o, h_final=hf, workspace=ws)
    ms, wall = time_loop(torch, fn, steps, warmup)
    kern = None
    if kernel_times and gdn:
        ops.gdn_prefill_kernel_times()            # clear
        ops.gdn_prefill_timing(True)
        try:
            for _ in range(steps):
                fn()
            torch.cuda.synchronize()
        finally:
            ops.gdn_prefill_timing(False)
        kt = ops.gdn_prefill_kernel_times()
        kern = {n: {"launches": x["launches"], "ms_avg": x["ms"] / x["launches"]} for n, x in kt.items() if x["launches"]}
    if gdn:
        # a skipped chunk saves its state write, Khat^T U (2 C d_k d_v flop)
        flops = nchunk * gdn_flops_per_chunk(64, cfg.Dk) - (nchunk - kept) * 2 * 64 * cfg.Dk * cfg.Dv
    else:
        flops = nchunk * linattn_flops_per_chunk(64, cfg.Dk)
    nbytes = prefill_bytes(cfg, gates=gdn) + cfg.B * cfg.H * cfg.L * 4 * {"gla": 1, "gla_vec": cfg.Dk}.get(variant, 0)
    nbytes += nchunk if variant == "skip" else 0
    res = {
        "workload": cfg.name + ("_long_memory_gates" if gdn and cfg.gate_dist == "long" else "")
        + ({"gla": "_gated", "gla_vec": "_gated_per_dim", "skip": f"_skip_keep{keep_rate}",
                                 "band1": "_banded1"}.get(variant, "")),
        "ms": ms, "tokens_per_s": cfg.B * cfg.L / (ms * 1e-3),
        "alg_tflops": flops / (ms * 1e-3) / 1e12, "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "alg_bytes": nbytes, "hbm_GBps": nbytes / (ms * 1e-3) / 1e9,
        "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, "wall_s": wall,
    }
    if gdn:
        res["dense_tile_tflops"] = nchunk * gdn_dense_tile_flops_per_chunk(64, cfg.Dk) / (ms * 1e-3) / 1e12
    if kern is not None:
        res["kernels"] = kern
    if variant == "skip":
        res["kept_fraction"] = kept / nchunk
    return res, (q, k, v, beta, la, h0, o, hf)


def bench_bidir(torch, ops, cfg, steps, warmup):
    """Bidirectional linear attention with the elu+1 feature map and the normaliser on raw N(0,1)
    q and k of the linear-attention workload's shape."""
    cfg = cfg.with_(qk="raw")
    q, k, v, _, _, _ = prefill_device_inputs(torch, cfg, gates=False)
    o = torch.empty_like(v)
    ws = torch.empty(max(1, ops.linattn_bidir_workspace_size(cfg.B, cfg.H, cfg.L, cfg.Dk, q.dtype)),
                     dtype=torch.uint8, device="cuda")
    ms, wall = time_loop(torch, lambda: ops.linattn_bidir_fwd(q, k, v, o=o, workspace=ws), steps, warmup)
    tok = cfg.B * cfg.H * cfg.L
    flops = 2 * 2 * tok * cfg.Dk * cfg.Dv + 2 * 2 * tok * cfg.Dk      # phi(K)^T V and KV^T phi(q); key sums, Z
    e = 2 if cfg.dtype == "bf16" else 4
    nbytes = 3 * tok * cfg.Dk * e + tok * cfg.Dv * e
    return {"workload": cfg.name + "_bidirectional_elu1_normalized", "ms": ms, "tokens_per_s": cfg.B * cfg.L / (ms * 1e-3),
            "alg_tflops": flops / (ms * 1e-3) / 1e12, "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "alg_bytes": nbytes, "hbm_GBps": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, "wall_s": wall}


def bench_decode(torch, ops, cfg, steps):
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    state = to_dev(torch, inputs.decode_state(cfg), torch.float32)
    toks = []
    for s in range(steps):
        x = inputs.decode_token(cfg, s)
        toks.append([to_dev(torch, x[n], dt) for n in ("q", "k", "v")]
                    + [to_dev(torch, x[n], torch.float32) for n in ("beta", "log_alpha")])
    o = torch.empty_like(toks[0][2])
    ops.gdn_decode_step(*toks[0], state, o=o)        # warm-up (the state keeps evolving in place)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(steps):
        ops.gdn_decode_step(*toks[s], state, o=o)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    total, st_bytes = decode_bytes(cfg)
    return {"workload": cfg.name, "steps": steps, "ms_per_step": ms,
            "tokens_per_s": cfg.N / (ms * 1e-3), "state_GBps": st_bytes / (ms * 1e-3) / 1e9,
            "hbm_GBps": total / (ms * 1e-3) / 1e9, "hbm_frac": total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, target_s, gpu_out=None, gpu_hf=None):
    """The fp64 oracle on this host: all heads of the workload over its first L_s tokens on up to
    16 OpenMP threads (one per head), L_s calibrated so the run takes about `target_s` seconds;
    then one head of the same sample on one thread (its rate per head, times the heads, is the
    one-thread figure)."""
    import oracle
    threads = min(os.cpu_count() or 1, 16, cfg.B * cfg.H)

    def sample(L, heads):
        sl = [inputs.prefill_slice(cfg, 0, h, L) for h in heads]
        st = lambda key: np.stack([s[key] for s in sl])[None]
        return st("q"), st("k"), st("v"), st("beta"), st("log_alpha"), st("h0")

    L = 1024
    x = sample(L, range(cfg.H))
    t0 = time.perf_counter()
    oracle.gdn_prefill(*x, nthreads=threads)
    t = time.perf_counter() - t0
    L = int(min(cfg.L, max(1024, (target_s / max(t, 1e-3)) * L)) // 1024 * 1024)
    x = sample(L, range(cfg.H))
    t0 = time.perf_counter()
    ro, rh = oracle.gdn_prefill(*x, nthreads=threads)
    t = time.perf_counter() - t0
    used = oracle.last_threads
    # one thread, one head, a quarter of the sample's tokens
    L1 = max(1024, L // 4 // 1024 * 1024)
    x1 = sample(L1, [0])
    t1s = time.perf_counter()
    oracle.gdn_prefill(*x1, nthreads=1)
    t1 = time.perf_counter() - t1s
    out = {"value": cfg.B * L / t, "unit": "tokens/s", "cores": used, "kind": "oracle",
           "sample": f"{cfg.name}: all {cfg.H} heads, first {L} of {cfg.L} tokens, fp64 token recurrence, "
                     f"{used} OpenMP threads (one per head), {t:.1f} s",
           "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
           "one_thread": {"value": L1 / t1 / cfg.H, "unit": "tokens/s",
                          "sample": f"head 0, first {L1} tokens, 1 thread, {t1:.2f} s; tokens/s of the whole "
                                    f"workload (all {cfg.H} heads) at that rate"}}
    parity = None
    if gpu_out is not None:
        o = gpu_out[0, :, :L].float().cpu().numpy()
        err = np.abs(o - ro[0]).max(axis=(1, 2)) / np.abs(ro[0]).max(axis=(1, 2))
        parity = {"max_rel_err_o": float(err.max()), "sample": f"first {L} tokens of all heads"}
        if gpu_hf is not None and L == cfg.L:
            h = gpu_hf[0].float().cpu().numpy()
            eh = np.abs(h - rh[0]).max(axis=(1, 2)) / np.abs(rh[0]).max(axis=(1, 2))
            parity["max_rel_err_h_final"] = float(eh.max())
    return out, parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed calls first (the clocks settle over the first tens of milliseconds)")
    ap.add_argument("--no-components", action="store_true", help="time only the 128K prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run this many prefill steps after warm-up (for profilers), no JSON")
    ap.add_argument("--variant", default=None, choices=("skip", "band1"),
                    help="with --profile-steps: time gdn_prefill_skip_fwd (29%% kept) or gdn_prefill_banded_fwd (band 1)")
    ap.add_argument("--gate-dist", default="config", choices=("config", "long"),
                    help="with --profile-steps: the log-gate distribution (config: -softplus(N(0,1)+2); "
                         "long: -U(0, 0.01), a long memory)")
    ap.add_argument("--profile-decode", type=int, default=0,
                    help="only run this many decode steps (for profilers), no JSON")
    ap.add_argument("--profile-linattn", type=int, default=0,
                    help="only run this many plain, this many per-token gated and this many per-dimension "
                         "gated linear-attention calls at B=4 H=16 L=8192 after warm-up (for profilers), no JSON")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES device-to-device three times (counter calibration), no JSON")
    ap.add_argument("--copy-bandwidth", type=int, default=0, metavar="BYTES",
                    help="only time device-to-device copies of BYTES (HIP events) and print the HBM rate "
                         "(bytes read + written per second), no JSON")
    ap.add_argument("--source-hash", action="store_true", help="print kernel_source_hash() and exit")
    ap.add_argument("--counters", metavar="DIR", help="print the per-kernel counter figures of the rocprofv3 runs "
                    "under DIR (see counters_from) and exit; no GPU needed")
    args = ap.parse_args()
    if args.source_hash:
        print(kernel_source_hash())
        return
    if args.counters:
        print(json.dumps(counters_from(args.counters), indent=1))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (heads and sequences shard "
              "across GPUs with no communication; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_deltanet_chunked_rule_amd import ops
    torch.cuda.set_device(0)
    log = lambda m: print(m, file=sys.stderr, flush=True)

    cfg = inputs.GDN_128K
    if args.copy_calibrate:
        src = torch.ones(args.copy_calibrate // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {src.numel() * 4} bytes three times")
        return
    if args.copy_bandwidth:
        src = torch.ones(args.copy_bandwidth // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        ms, _ = time_loop(torch, lambda: dst.copy_(src), 20, 3)
        log(f"device copy of {src.numel() * 4} bytes: {ms:.4f} ms, {2 * src.numel() * 4 / (ms * 1e-3) / 1e9:.0f} GB/s "
            f"read + written")
        return
    if args.profile_decode:
        c = inputs.DECODE_256x32
        r = bench_decode(torch, ops, c, args.profile_decode)
        log(f"profiled {args.profile_decode} decode steps: {r['ms_per_step']:.4f} ms/step")
        return
    if args.profile_linattn:
        c = inputs.LINATTN_8K
        r = bench_prefill(torch, ops, c, args.profile_linattn, args.warmup, gdn=False)[0]
        rg = bench_prefill(torch, ops, c.with_(gates=True, gate_dist="long"), args.profile_linattn, args.warmup,
                           gdn=False, variant="gla")[0]
        rv = bench_prefill(torch, ops, c.with_(gate_dist="config"), args.profile_linattn, args.warmup, gdn=False,
                           variant="gla_vec")[0]
        log(f"profiled {args.profile_linattn} linear-attention calls: plain {r['ms']:.4f} ms, gated {rg['ms']:.4f} ms, "
            f"gated per key dimension {rv['ms']:.4f} ms")
        return
    if args.profile_steps:
        log("generating inputs")
        res, bufs = bench_prefill(torch, ops, cfg.with_(gate_dist=args.gate_dist), args.profile_steps, args.warmup,
                                  verbose=True, kernel_times=True, variant=args.variant)
        log(f"profiled {args.profile_steps} steps: {res['ms']:.3f} ms/step; kernels (HIP events): "
            + ", ".join(f"{n} {x['ms_avg']:.4f} ms" for n, x in res["kernels"].items()))
        return

    log(f"[bench] {cfg.name}: generating inputs")
    res, bufs = bench_prefill(torch, ops, cfg, args.steps, args.warmup, kernel_times=True)
    log(f"[bench] {cfg.name}: {res['ms']:.3f} ms/step, {res['tokens_per_s']:.3e} tokens/s; kernels: "
        + ", ".join(f"{n} {x['ms_avg']:.4f} ms" for n, x in res["kernels"].items()))
    gpu_o, gpu_hf = bufs[6], bufs[7]

    components = {}
    if not args.no_components:
        del bufs
        torch.cuda.empty_cache()
        log("[bench] decode")
        components["decode"] = bench_decode(torch, ops, inputs.DECODE_256x32, inputs.DECODE_256x32.steps)
        log(f"[bench] decode: {components['decode']['ms_per_step']:.4f} ms/step")
        log("[bench] linear attention")
        r, b = bench_prefill(torch, ops, inputs.LINATTN_8K, max(5, args.steps // 2), args.warmup, gdn=False)
        components["linattn"] = r
        del b
        log("[bench] bidirectional linear attention")
        components["linattn_bidir"] = bench_bidir(torch, ops, inputs.LINATTN_8K, max(5, args.steps // 2), args.warmup)
        log("[bench] gdn 32K")
        r, b = bench_prefill(torch, ops, inputs.GDN_32K, max(5, args.steps // 2), args.warmup)
        components["gdn_32k"] = r
        del b
        log("[bench] linear attention with per-token gates")
        r, b = bench_prefill(torch, ops, inputs.LINATTN_8K.with_(gates=True, gate_dist="long"),
                             max(5, args.steps // 2), args.warmup, gdn=False, variant="gla")
        components["linattn_gated"] = r
        del b
        log("[bench] linear attention with a gate per key dimension")
        r, b = bench_prefill(torch, ops, inputs.LINATTN_8K.with_(gate_dist="config"), max(5, args.steps // 2), args.warmup,
                             gdn=False, variant="gla_vec")
        components["linattn_gated_per_dim"] = r
        del b
        log("[bench] gdn 128K with long-memory gates")
        r, b = bench_prefill(torch, ops, cfg.with_(gate_dist="long"), max(5, args.steps // 2), args.warmup, kernel_times=True)
        components["gdn_128k_long_memory"] = r
        del b
        log("[bench] gdn 128K with skipped chunk updates (29% kept)")
        r, b = bench_prefill(torch, ops, cfg, max(5, args.steps // 2), args.warmup, variant="skip", kernel_times=True)
        components["gdn_128k_skip"] = r
        del b
        log("[bench] gdn 128K with long-memory gates and skipped chunk updates (29% kept)")
        r, b = bench_prefill(torch, ops, cfg.with_(gate_dist="long"), max(5, args.steps // 2), args.warmup,
                             variant="skip", kernel_times=True)
        components["gdn_128k_long_memory_skip"] = r
        del b
        log("[bench] gdn 128K with the block-adjacent intra-chunk solve (band 1)")
        r, b = bench_prefill(torch, ops, cfg, max(5, args.steps // 2), args.warmup, variant="band1", kernel_times=True)
        components["gdn_128k_banded1"] = r
        del b

    cpu, parity = (None, None)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle)")
        cpu, parity = cpu_baseline(cfg, args.cpu_seconds, gpu_out=gpu_o, gpu_hf=gpu_hf)

    # roofline of the output kernel (the call's dominant kernel): its algorithmic bytes and flops
    # per launch over its average launch time, measured with HIP events on the call's stream
    ko = res["kernels"]["out"]
    t_out = ko["ms_avg"] * 1e-3
    nchunk = cfg.B * cfg.H * ((cfg.L + 63) // 64)
    ob = out_kernel_bytes(cfg)
    oflops = nchunk * gdn_flops_per_chunk(64, cfg.Dk)
    cnt = COUNTERS_128K if COUNTERS_128K is not None and COUNTERS_128K["source_hash"] == kernel_source_hash() else None
    traffic = cnt["out"]["hbm_bytes"] if cnt else None
    mfma_counted = None
    if cnt and "mfma_bf16_flops" in cnt["out"]:
        c = cnt["out"]
        mfma_counted = {"bf16_flops_per_launch": c["mfma_bf16_flops"], "f32_flops_per_launch": c["mfma_f32_flops"],
                        "bf16_tflops": c["mfma_bf16_flops"] / t_out / 1e12,
                        "frac_of_bf16_peak": c["mfma_bf16_flops"] / t_out / 1e12 / PEAK_BF16_TFLOPS,
                        "busy_frac": c.get("mfma_busy_frac")}
    call_traffic = None
    if cnt:
        call_traffic = {"bytes": sum(cnt[k]["hbm_bytes"] for k in KERNELS if k in cnt),
                        "alg_bytes": res["alg_bytes"]}
        call_traffic["ratio"] = call_traffic["bytes"] / call_traffic["alg_bytes"]
        call_traffic["per_kernel"] = {k: cnt[k]["hbm_bytes"] for k in KERNELS if k in cnt}
    line = {
        "metric": METRIC,
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), beta=sigmoid(N), "
                "log a=-softplus(N+2), h0 N(0,0.01))",
        "config": {"workload": "gdn_prefill_B1_H16_L131072_d128_chunk64", "B": cfg.B, "H": cfg.H,
                   "L": cfg.L, "d_k": cfg.Dk, "d_v": cfg.Dv, "chunk": 64, "qkv": "bf16", "gates_state": "fp32"},
        # the whole call: algorithmic flops (triangles exact) and whole 64 x 64 tiles over the call's time
        "mfma": {"alg_tflops": res["alg_tflops"], "dense_tile_tflops": res["dense_tile_tflops"],
                 "peak_tflops": PEAK_BF16_TFLOPS, "frac": res["mfma_frac"],
                 "dense_tile_frac": res["dense_tile_tflops"] / PEAK_BF16_TFLOPS,
                 "out_kernel_alg_frac": oflops / t_out / 1e12 / PEAK_BF16_TFLOPS,
                 "counted_out_kernel": mfma_counted},
        "roofline": {"bound": "hbm", "kernel": "out_kernel<128, BF16> (outputs and final state of each block)",
                     "achieved": ob / t_out / 1e9, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": ob / t_out / 1e9 / PEAK_HBM_GBPS, "traffic": traffic,
                     "alg_bytes_per_launch": ob, "launch_ms": ko["ms_avg"], "launches": ko["launches"]},
        "kernels_ms": {k: v["ms_avg"] for k, v in res["kernels"].items()},
        "call_traffic": call_traffic,
        "cpu_baseline": cpu,
        "parity_sample": parity,
        "components": components,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
