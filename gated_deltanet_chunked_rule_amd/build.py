"""Build libgdn.so in-tree with hipcc for gfx950 (one shared library, C ABI in include/gdn.h)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["gdn_api.cpp", "gdn_decode.hip", "gdn_prefill.hip", "gdn_bidir.hip", "gdn_linattn.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off: the kernels use plain fp32 arithmetic only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]

# Where MFMA accumulators live, per source. The linear-attention, bidirectional and decode
# kernels rescale and pack their accumulator tiles every chunk, which with AGPR accumulators
# costs a copy per element, so they keep them in VGPRs. The prefill kernels hold two fp32 state
# blocks plus the intra-chunk operands per wave and need the AGPR file as well.
SOURCE_FLAGS = {
    "gdn_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=0"],
    "gdn_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "gdn_bidir.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "gdn_linattn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def flags_for(src: str) -> list:
    """Compiler flags for one source (without -shared / -o)."""
    return [f for f in FLAGS if f != "-shared"] + SOURCE_FLAGS.get(os.path.basename(src), [])


def _clean(text: str) -> str:
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    objs = [tmp + "." + s + ".o" for s in SOURCES]

    def compile_one(i):
        src = os.path.join(CSRC, SOURCES[i])
        cmd = [HIPCC] + flags_for(src) + ["-c", "-o", objs[i], src]
        return cmd, subprocess.run(cmd, capture_output=True, text=True)

    out = []
    try:
        with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
            for cmd, r in ex.map(compile_one, range(len(SOURCES))):
                if r.returncode != 0:
                    raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + _clean(r.stdout + r.stderr))
                out.append(_clean(r.stdout + r.stderr))
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + " ".join(cmd) + "\n" + _clean(r.stdout + r.stderr))
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    text = "\n".join(o for o in out if o.strip())
    if verbose and text.strip():
        print(text, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
