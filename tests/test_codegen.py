"""Checks on the gfx950 assembly the kernels compile to (CPU only: hipcc cross-compiles).

Matrix-core (MFMA) instructions write their result whatever the lane mask. A branch that the
compiler sees as divergent turns into a lane-masked block, and when such a block is short the
compiler may drop the branch around it and issue the MFMA with an all-zero mask, which then
still overwrites its accumulator. Every MFMA therefore has to sit in scalar control flow: the
kernels read their wave index into a scalar register, and this test checks that no MFMA is
issued between a lane-mask save (s_*_saveexec, s_and/xor/andn2 on exec) and the restore that
ends the block, following branches and fall-through in the listing. (A restore inside a nested
masked block is taken to end the outer one too, so an MFMA after it in the outer block would
be missed.)
"""
import os
import re
import shutil
import subprocess

import pytest

from gated_deltanet_chunked_rule_amd import build

HIPCC = build.HIPCC
pytestmark = pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not found")

SOURCES = ["gdn_prefill.hip", "gdn_decode.hip", "gdn_bidir.hip", "gdn_linattn.hip"]


def _device_asm(src, tmp_path):
    out = tmp_path / (src + ".s")
    flags = [f for f in build.flags_for(src) if f != "-fPIC"]
    cmd = [HIPCC] + flags + ["--cuda-device-only", "-S", "-o", str(out), os.path.join(build.CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def masked_mfmas(asm):
    """{kernel symbol: number of MFMAs issued while a lane mask may be active}.

    Follows the control flow of the listing: a masked region opens at a lane-mask save and closes
    at the restore; a label is masked when it is reached by falling through from a masked block
    or by a branch taken inside one (no fall-through past s_branch or s_endpgm). Branches to
    earlier labels are handled by repeating the pass until the set of masked labels is stable."""
    lines = [l.split(";")[0].strip() for l in asm.splitlines()]
    found = {}
    masked_labels = set()
    while True:
        found, cur, masked, falls, grow = {}, None, False, True, set()
        for ins in lines:
            m = re.match(r"^(_Z\w+):", ins)
            if m:
                cur, masked, falls = m.group(1), False, True
                continue
            m = re.match(r"^(\.L\w+):", ins)
            if m:
                masked = (masked and falls) or m.group(1) in masked_labels
                falls = True
                continue
            if not ins or ins.startswith("."):
                continue
            if re.match(r"s_(and|or|andn2|xor)_saveexec_b64", ins) or re.match(r"s_(and|xor|andn2)_b64 exec, exec", ins):
                masked = True
            elif re.match(r"s_or_b64 exec, exec", ins) or re.match(r"s_mov_b64 exec, -1", ins):
                masked = False
            b = re.match(r"s_c?branch\w*\s+(\.L\w+)", ins)
            if b and masked:
                grow.add(b.group(1))
            falls = not (ins.startswith("s_branch") or ins.startswith("s_endpgm") or ins.startswith("s_setpc"))
            if ins.startswith("v_mfma") and masked:
                found[cur] = found.get(cur, 0) + 1
        if grow <= masked_labels:
            return found
        masked_labels |= grow


def test_detector_sees_a_masked_mfma():
    asm = "\n".join(["_Zk:", "v_cmp_eq_u32_e32 vcc, 1, v1", "s_and_saveexec_b64 s[0:1], vcc",
                     "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]", "s_or_b64 exec, exec, s[0:1]",
                     "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]"])
    assert masked_mfmas(asm) == {"_Zk": 1}


def test_detector_follows_branches():
    # a masked block that ends the program is not the code laid out after it ...
    asm = "\n".join(["_Zk:", "s_cbranch_scc1 .LBB0_2", "s_and_b64 exec, exec, vcc", "global_store_dword v0, v1, s[0:1]",
                     "s_endpgm", ".LBB0_2:", "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]"])
    assert masked_mfmas(asm) == {}
    # ... but a label reached by a branch taken under a mask is masked
    asm = "\n".join(["_Zk:", "s_and_saveexec_b64 s[0:1], vcc", "s_cbranch_execz .LBB0_3", "s_nop 0", "s_endpgm",
                     ".LBB0_3:", "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]"])
    assert masked_mfmas(asm) == {"_Zk": 1}
    # and a loop whose back edge is taken under a mask masks its header
    asm = "\n".join(["_Zk:", ".LBB0_1:", "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]",
                     "s_and_saveexec_b64 s[0:1], vcc", "s_cbranch_execnz .LBB0_1", "s_or_b64 exec, exec, s[0:1]"])
    assert masked_mfmas(asm) == {"_Zk": 1}


@pytest.mark.parametrize("src", SOURCES)
def test_no_mfma_under_a_lane_mask(src, tmp_path):
    asm = _device_asm(src, tmp_path)
    assert "v_mfma" in asm or src == "gdn_decode.hip"
    assert masked_mfmas(asm) == {}
