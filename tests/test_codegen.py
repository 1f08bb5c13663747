"""Checks on the gfx950 assembly the kernels compile to (CPU only: hipcc cross-compiles).

Matrix-core (MFMA) instructions write their result whatever the lane mask. A branch that the
compiler sees as divergent turns into a lane-masked block, and when such a block is short the
compiler may drop the branch around it and issue the MFMA with an all-zero mask, which then
still overwrites its accumulator. Every MFMA therefore has to sit in scalar control flow: the
kernels read their wave index into a scalar register, and this test checks that no MFMA is
issued between a lane-mask save (s_*_saveexec, s_and/xor/andn2 on exec) and the restore that
ends the block. (Nested masked blocks are approximated by the outermost; that can only miss
a case, not report a false one.)
"""
import os
import re
import shutil
import subprocess

import pytest

from gated_deltanet_chunked_rule_amd import build

HIPCC = build.HIPCC
pytestmark = pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not found")

SOURCES = ["gdn_prefill.hip", "gdn_decode.hip", "gdn_bidir.hip"]


def _device_asm(src, tmp_path):
    out = tmp_path / (src + ".s")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [HIPCC] + flags + ["--cuda-device-only", "-S", "-o", str(out), os.path.join(build.CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def masked_mfmas(asm):
    """{kernel symbol: number of MFMAs issued while a lane mask may be active}."""
    found, cur, masked = {}, None, False
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur, masked = m.group(1), False
        ins = line.split(";")[0].strip()
        if re.match(r"s_(and|or|andn2|xor)_saveexec_b64", ins) or re.match(r"s_(and|xor|andn2)_b64 exec, exec", ins):
            masked = True
        elif re.match(r"s_or_b64 exec, exec", ins) or re.match(r"s_mov_b64 exec, -1", ins):
            masked = False
        if ins.startswith("v_mfma") and masked:
            found[cur] = found.get(cur, 0) + 1
    return found


def test_detector_sees_a_masked_mfma():
    asm = "\n".join(["_Zk:", "v_cmp_eq_u32_e32 vcc, 1, v1", "s_and_saveexec_b64 s[0:1], vcc",
                     "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]", "s_or_b64 exec, exec, s[0:1]",
                     "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]"])
    assert masked_mfmas(asm) == {"_Zk": 1}


@pytest.mark.parametrize("src", SOURCES)
def test_no_mfma_under_a_lane_mask(src, tmp_path):
    asm = _device_asm(src, tmp_path)
    assert "v_mfma" in asm or src == "gdn_decode.hip"
    assert masked_mfmas(asm) == {}
