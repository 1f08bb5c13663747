"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments on the
host before touching a GPU (fake pointer values are never dereferenced)."""
import ctypes
import os
import re

import pytest

from gated_deltanet_chunked_rule_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, WORKSPACE = 0, -1, -2, -3, -4, -5, -6


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_]+)\s*\(", text)) - {"if", "sizeof", "defined"})


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert _lib.status_string(code).startswith("GDN_")
    assert _lib.status_string(17) == "unknown status"


def test_prefill_timing_switch(lib):
    """Turning per-kernel timing on and off touches no device; with nothing recorded the
    query returns zero time and zero launches for all three kernels."""
    ms = (ctypes.c_float * 3)(1.0, 2.0, 3.0)
    n = (ctypes.c_int * 3)(7, 7, 7)
    assert lib.gdn_prefill_timing(1) == OK
    assert lib.gdn_prefill_timing(0) == OK
    assert lib.gdn_prefill_kernel_times(ctypes.addressof(ms), ctypes.addressof(n)) == OK
    assert list(ms) == [0.0, 0.0, 0.0] and list(n) == [0, 0, 0]
    assert lib.gdn_prefill_kernel_times(None, None) == OK


def test_workspace_size_query(lib):
    """The prefill workspace holds (2 NB - 1) block records of 4 Dk Dv bytes per slice for NB blocks
    and NB - 1 four-byte flags rounded up to 256 bytes; the preferred NB gives about two output
    workgroups per CU (256 CUs when no GPU answers)."""
    f = lib.gdn_prefill_workspace_size
    rec = lambda d: 4 * d * d
    assert f(1, 1, 64, 128, 128, 0) == 0                  # one chunk: one block, no workspace
    assert f(1, 1, 64 * 5, 128, 128, 0) == 9 * rec(128) + 256     # five chunks, five blocks of one
    big = f(1, 16, 131072, 128, 128, 0)                    # 2048 chunks: 32 blocks of 64 per slice
    assert big == 16 * ((2 * 32 - 1) * rec(128) + 256)
    assert f(1, 32, 32768, 128, 128, 0) == 32 * ((2 * 16 - 1) * rec(128) + 256)
    assert f(1, 16, 131072, 64, 64, 1) == 16 * ((2 * 32 - 1) * rec(64) + 256)   # sizes do not depend on dtype
    assert f(1, 1, 64 * 100, 128, 128, 0) == 199 * rec(128) + 512    # 100 blocks: 99 flags, 396 bytes
    assert f(2, 128, 4096, 128, 128, 0) == 0                # 256 slices fill the device alone
    assert f(1, 2, 0, 128, 128, 0) == 0
    assert f(1, 1, 64, 96, 96, 0) == 0        # unsupported head size
    assert f(1, 1, 64, 128, 64, 0) == 0       # Dk != Dv
    assert f(1, 1, 64, 128, 128, 2) == 0      # bad dtype
    assert f(0, 1, 64, 128, 128, 0) == 0
    # any workspace is accepted, none included (one block per slice then)
    for ws, wsb in ((None, 0), (0x100000000, 1), (0x100000000, 1 << 30)):
        assert _prefill(lib, L=4096, ws=ws, wsb=wsb) not in (NULL, ALIGN, ALIAS, WORKSPACE)


def _prefill(lib, q=0x10000, k=0x20000000, v=0x40000000, beta=0x60000000, la=0x60100000, h0=None,
             o=0x70000000, hf=0x7f000000, B=1, H=1, L=64, D=128, dt=0, ws=0x100000000, wsb=1 << 30, gdn=True):
    f = lib.gdn_prefill_fwd if gdn else lib.linattn_prefill_fwd
    return f(q, k, v, beta, la, h0, o, hf, B, H, L, D, D, dt, ws, wsb, None)


def test_prefill_host_validation(lib):
    assert _prefill(lib, q=None) == NULL
    assert _prefill(lib, beta=None) == NULL
    assert _prefill(lib, gdn=False) == NULL            # linear attention takes no beta
    assert _prefill(lib, gdn=False, beta=None) not in (NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, ALIAS)  # gates optional
    assert _prefill(lib, D=96) == SHAPE
    assert _prefill(lib, L=-1) == SHAPE
    assert _prefill(lib, B=0) == SHAPE
    assert _prefill(lib, dt=5) == DTYPE
    assert _prefill(lib, q=0x10008) == ALIGN
    assert _prefill(lib, ws=0x100000010) == ALIGN      # workspace needs 256-byte alignment
    assert _prefill(lib, ws=0x100000010, wsb=0) not in (NULL, ALIGN, ALIAS, WORKSPACE)   # an empty one is unused
    assert _prefill(lib, ws=0x40000000 - 256) == ALIAS  # workspace runs into v
    assert _prefill(lib, o=0x20000000) == ALIAS        # o == k
    assert _prefill(lib, hf=0x40000000 + 4096) == ALIAS  # h_final inside v
    assert _prefill(lib, h0=0x7f000000 + 16) == ALIAS  # partial h0 / h_final overlap


def test_noalloc_host_validation(lib):
    """The prefill entry point without a workspace argument: a request for more static scratch
    than the library holds is refused first; the other checks are gdn_prefill_fwd's."""
    f = lib.gdn_prefill_fwd_noalloc
    SCRATCH = -9
    args = lambda q=0x10000, D=128, L=64, sb=0: (q, 0x20000000, 0x40000000, 0x60000000, 0x60100000, None,
                                                 0x70000000, 0x7f000000, 1, 1, L, D, D, 0, sb, None)
    assert _lib.GDN_PREFILL_NOALLOC_MAX_BYTES == 80 << 20
    assert f(*args(sb=(80 << 20) + 1)) == SCRATCH
    assert f(*args(q=None, sb=(80 << 20) + 1)) == SCRATCH
    assert f(*args(q=None)) == NULL
    assert f(*args(D=96)) == SHAPE
    assert f(*args(q=0x10008)) == ALIGN
    for sb in (0, 1 << 20, 80 << 20):
        assert f(*args(L=4096, sb=sb)) not in (NULL, SHAPE, ALIGN, ALIAS, WORKSPACE, SCRATCH)


def test_linattn_workspace(lib):
    f = lib.linattn_prefill_workspace_size
    blk = 128 * 128 * 4 + 4                             # one block's state and its summed log-gate
    assert f(1, 1, 64, 128, 128, 0) == blk               # one chunk: one block
    assert f(2, 2, 64 * 1000, 128, 128, 0) % (4 * blk) == 0
    assert f(1, 1, 64 * 1000, 64, 64, 1) % (64 * 64 * 4 + 4) == 0
    assert f(1, 1, 0, 128, 128, 0) == 0
    assert f(1, 1, 64, 96, 96, 0) == 0
    # smallest accepted: one block per (batch, head)
    assert _prefill(lib, gdn=False, beta=None, H=3, L=1000, wsb=3 * blk - 1) == WORKSPACE
    assert _prefill(lib, gdn=False, beta=None, H=3, L=1000, wsb=3 * blk) not in (NULL, ALIGN, ALIAS, WORKSPACE)
    assert _prefill(lib, gdn=False, beta=None, L=0, ws=None, wsb=0) not in (NULL, ALIGN, ALIAS, WORKSPACE)


def _prefill_skip(lib, keep=0x60200000, o=0x70000000, **kw):
    a = dict(q=0x10000, k=0x20000000, v=0x40000000, beta=0x60000000, la=0x60100000, h0=None, hf=0x7f000000,
             L=200, ws=0x100000000, wsb=1 << 30)
    a.update(kw)
    return lib.gdn_prefill_skip_fwd(a["q"], a["k"], a["v"], a["beta"], a["la"], keep, a["h0"], o, a["hf"], 1, 2,
                                    a["L"], 128, 128, 0, a["ws"], a["wsb"], None)


def test_prefill_skip_host_validation(lib):
    assert _prefill_skip(lib, keep=None) == NULL                 # the keep mask is required
    assert _prefill_skip(lib, keep=None, L=0) != NULL            # ... unless there are no tokens
    assert _prefill_skip(lib, beta=None) == NULL
    assert _prefill_skip(lib, keep=0x70000000 + 8) == ALIAS      # mask inside o
    assert _prefill_skip(lib, keep=0x60200003) not in (NULL, ALIGN, ALIAS)   # any alignment


def test_decode_host_validation(lib):
    f = lib.gdn_decode_step
    args = dict(q=0x10000, k=0x20000, v=0x30000, beta=0x40000, la=0x50000, st=0x1000000, o=0x60000)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["beta"], a["la"], a["st"], a["o"], kw.get("N", 4), 2, 128, 128,
                 kw.get("dt", 0), None)

    assert call(st=None) == NULL
    assert call(N=0) == SHAPE
    assert call(dt=3) == DTYPE
    assert call(o=0x60004) == ALIGN
    assert call(o=0x1000000 + 4096) == ALIAS           # o inside the state
    assert call(q=0x1000000) == ALIAS


def _bidir(lib, **kw):
    a = dict(q=0x10000, k=0x20000000, v=0x40000000, o=0x60000000, kv=None, B=1, H=2, L=300, D=128, dt=0, flags=3,
             ws=0x100000000, wsb=1 << 30)
    a.update(kw)
    return lib.linattn_bidir_fwd(a["q"], a["k"], a["v"], a["o"], a["kv"], a["B"], a["H"], a["L"], a["D"], a["D"],
                                 a["dt"], a["flags"], a["ws"], a["wsb"], None)


def test_bidir_host_validation(lib):
    assert _bidir(lib, q=None) == NULL
    assert _bidir(lib, q=None, k=None, v=None, o=None, L=0, ws=None, wsb=0) not in (NULL, ALIGN, ALIAS, WORKSPACE)
    assert _bidir(lib, flags=4) == SHAPE                        # unknown flag bit
    assert _bidir(lib, D=96) == SHAPE
    assert _bidir(lib, dt=2) == DTYPE
    assert _bidir(lib, o=0x60000008) == ALIGN
    assert _bidir(lib, kv=0x70000004) == ALIGN
    assert _bidir(lib, ws=0x100000010) == ALIGN                # workspace needs 256-byte alignment
    assert _bidir(lib, ws=None) == WORKSPACE
    need = lib.linattn_bidir_workspace_size(1, 2, 300, 128, 128, 0)
    assert _bidir(lib, wsb=need - 1) == WORKSPACE
    assert _bidir(lib, wsb=need) not in (NULL, SHAPE, ALIGN, ALIAS, WORKSPACE)
    assert _bidir(lib, o=0x20000000 + 256) == ALIAS            # o inside k
    assert _bidir(lib, kv=0x60000000 + 512) == ALIAS           # kv inside o
    assert _bidir(lib, ws=0x40000000 - 256) == ALIAS           # workspace runs into v


def test_bidir_workspace_size(lib):
    f = lib.linattn_bidir_workspace_size
    assert f(1, 2, 0, 128, 128, 0) == 0
    assert f(1, 2, 10, 96, 96, 0) == 0
    # one head, one chunk: one block of 64 partial tiles, its key sums, 32 fragments, the key sums
    assert f(1, 1, 64, 128, 128, 0) == (64 * 1024 + 512 + 32 * 1024 + 512 + 255) // 256 * 256
    # grows with the number of heads and never shrinks with L
    assert f(4, 16, 8192, 128, 128, 0) > f(1, 16, 8192, 128, 128, 0)
    assert f(1, 1, 64 * 1000, 64, 64, 1) >= f(1, 1, 64 * 10, 64, 64, 1)


def test_banded_host_validation(lib):
    def call(band, **kw):
        a = dict(q=0x10000, k=0x20000000, v=0x40000000, beta=0x60000000, la=0x60100000, o=0x70000000,
                 hf=0x7f000000)
        a.update(kw)
        return lib.gdn_prefill_banded_fwd(a["q"], a["k"], a["v"], a["beta"], a["la"], None, a["o"], a["hf"], 1, 2,
                                          200, 128, 128, 0, band, 0x100000000, 1 << 30, None)
    assert call(-1) == SHAPE and call(4) == SHAPE
    for band in range(4):
        assert call(band) not in (NULL, SHAPE, ALIGN, ALIAS, WORKSPACE)
    assert call(1, beta=None) == NULL


def _gla(lib, q=0x10000, k=0x20000000, v=0x40000000, la=0x60000000, h0=None, o=0x70000000, hf=0x7f000000, B=1,
         H=1, L=64, D=128, dt=0, ws=0x100000000, wsb=1 << 30):
    return lib.gla_prefill_fwd(q, k, v, la, h0, o, hf, B, H, L, D, D, dt, ws, wsb, None)


def test_gla_host_validation(lib):
    passed = (NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, ALIAS)
    assert _gla(lib) not in passed
    assert _gla(lib, la=None) == NULL                  # the per-dimension gates are required
    assert _gla(lib, L=0, q=None, k=None, v=None, la=None, o=None, ws=None, wsb=0) not in passed
    assert _gla(lib, hf=None) == NULL
    assert _gla(lib, D=96) == SHAPE
    assert _gla(lib, dt=3) == DTYPE
    assert _gla(lib, la=0x60000008) == ALIGN
    assert _gla(lib, ws=0x100000010) == ALIGN
    # log_alpha is [B,H,L,Dk] fp32: 64 x 128 x 4 bytes; an output inside it is an alias
    assert _gla(lib, o=0x60000000 + 64 * 128 * 4 - 16) == ALIAS
    assert _gla(lib, o=0x60000000 + 64 * 128 * 4) not in passed
    blk = 128 * 128 * 4 + 128 * 4                      # one block's state and summed log gates
    assert _gla(lib, H=3, L=1000, wsb=3 * blk - 1) == WORKSPACE
    assert _gla(lib, H=3, L=1000, wsb=3 * blk) not in passed
    f = lib.gla_prefill_workspace_size
    assert f(1, 1, 64, 128, 128, 0) == blk
    assert f(2, 2, 64 * 1000, 64, 64, 1) % (4 * (64 * 64 * 4 + 64 * 4)) == 0
    assert f(1, 1, 0, 128, 128, 0) == 0 and f(1, 1, 64, 96, 96, 0) == 0


# HIP runtime calls the library may make. Kernel launches, their error check, device queries,
# kernel attributes and the scratch's device address; events only for the opt-in per-kernel timing
# (gdn_prefill_timing) and its query. No allocation, free, memset, copy or stream/device
# synchronisation: a call records only kernel launches on the caller's stream, so it can be
# captured into a HIP graph and needs no memory of its own.
HIP_CALLS_ALLOWED = {
    "hipLaunchKernelGGL", "hipGetLastError", "hipGetDevice", "hipGetDeviceProperties", "hipDeviceGetAttribute",
    "hipFuncSetAttribute", "hipGetSymbolAddress",
    "hipEventCreate", "hipEventRecord", "hipEventSynchronize", "hipEventElapsedTime",
}


def test_library_makes_only_launch_query_and_timing_calls():
    csrc = os.path.join(ROOT, "gated_deltanet_chunked_rule_amd", "csrc")
    used = {}
    for name in sorted(os.listdir(csrc)):
        text = open(os.path.join(csrc, name)).read()
        text = re.sub(r"//[^\n]*|/\*.*?\*/", "", text, flags=re.S)
        for call in re.findall(r"\b(hip[A-Z]\w*)\s*\(", text):
            used.setdefault(call, set()).add(name)
    assert "hipLaunchKernelGGL" in used
    extra = {c: sorted(f) for c, f in used.items() if c not in HIP_CALLS_ALLOWED}
    assert not extra, f"HIP calls outside the allowed set: {extra}"
    # the events belong to the timing switch in the prefill's launch code only
    for c in ("hipEventCreate", "hipEventRecord", "hipEventSynchronize", "hipEventElapsedTime"):
        assert used.get(c, {"gdn_prefill.hip"}) == {"gdn_prefill.hip"}, c
