"""ctypes binding of libgdn.so (the C ABI declared in include/gdn.h). Marshalling only."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; GDN_LIBRARY names another build of the same sources (an instrumented one)
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(_HERE, "libgdn.so")

GDN_BF16, GDN_F32 = 0, 1
GDN_BIDIR_NORMALIZE, GDN_BIDIR_ELU1 = 1, 2
GDN_OK = 0
GDN_PREFILL_NOALLOC_MAX_BYTES = 80 << 20

# every symbol the header declares, with (restype, argtypes)
_vp, _fp, _i, _sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "gdn_status_string": (ctypes.c_char_p, [_i]),
    "gdn_prefill_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "gdn_prefill_fwd": (_i, [_vp, _vp, _vp, _fp, _fp, _fp, _vp, _fp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "gdn_prefill_fwd_noalloc": (_i, [_vp, _vp, _vp, _fp, _fp, _fp, _vp, _fp, _i, _i, _i, _i, _i, _i, _sz, _vp]),
    "gdn_prefill_skip_fwd": (_i, [_vp, _vp, _vp, _fp, _fp, _vp, _fp, _vp, _fp, _i, _i, _i, _i, _i, _i, _vp, _sz,
                                  _vp]),
    "gdn_prefill_banded_fwd": (_i, [_vp, _vp, _vp, _fp, _fp, _fp, _vp, _fp, _i, _i, _i, _i, _i, _i, _i, _vp, _sz,
                                    _vp]),
    "linattn_prefill_fwd": (_i, [_vp, _vp, _vp, _fp, _fp, _fp, _vp, _fp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "gdn_decode_step": (_i, [_vp, _vp, _vp, _fp, _fp, _fp, _vp, _i, _i, _i, _i, _i, _vp]),
    "linattn_prefill_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "gla_prefill_fwd": (_i, [_vp, _vp, _vp, _fp, _fp, _vp, _fp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "gla_prefill_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "linattn_bidir_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "gdn_prefill_timing": (_i, [_i]),
    "gdn_prefill_kernel_times": (_i, [_vp, _vp]),
    "linattn_bidir_fwd": (_i, [_vp, _vp, _vp, _vp, _fp, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
}

_lib = None


class GDNError(RuntimeError):
    pass


def load():
    """Load the in-tree libgdn.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise GDNError(f"{LIB_PATH} is missing: build it first (python -m gated_deltanet_chunked_rule_amd.build "
                           "or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def status_string(code: int) -> str:
    return load().gdn_status_string(code).decode()


def check(code: int, what: str):
    if code != GDN_OK:
        raise GDNError(f"{what} failed: {status_string(code)} ({code})")
