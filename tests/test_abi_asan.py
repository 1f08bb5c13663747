"""The host-side argument checks of the C ABI under AddressSanitizer: libgdn.so's sources are
built again with the host code instrumented (device code unchanged) and test_abi.py runs against
that build in a child process with the sanitizer runtime preloaded. Any out-of-bounds access,
use after free or similar in the validation code aborts the child. CPU only."""
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from gated_deltanet_chunked_rule_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(not os.path.exists(build.HIPCC) or _asan_runtime() is None,
                    reason="needs hipcc and the clang AddressSanitizer runtime")
def test_abi_validation_under_address_sanitizer(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(name):
        src = os.path.join(build.CSRC, name)
        obj = str(tmp_path / (name + ".o"))
        r = subprocess.run([build.HIPCC] + build.flags_for(src) + san + ["-c", "-o", obj, src],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(len(build.SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, build.SOURCES))
    lib = str(tmp_path / "libgdn_asan.so")
    r = subprocess.run([build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + san[:2] + ["-o", lib] + objs,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, GDN_LIBRARY=lib, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], capture_output=True, text=True, env=env, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
    # the child really loaded the instrumented build
    r = subprocess.run(["nm", "-D", lib], capture_output=True, text=True)
    if r.returncode == 0:
        assert "__asan_" in r.stdout
