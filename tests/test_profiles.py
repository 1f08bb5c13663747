"""The committed profile summaries and the bench's stored counter figures belong to the current kernel
sources: each summary names the sources it was measured on by hash, and a kernel change that is
not measured again leaves a summary (or the traffic and MFMA figures bench.py reports from its
stored counters) describing code that no longer exists. CPU only."""
import hashlib
import os
import re

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "gated_deltanet_chunked_rule_amd", "csrc")


def _file_hash(name):
    with open(os.path.join(CSRC, name), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def _summaries():
    return {n: open(os.path.join(PROFILES, n)).read() for n in sorted(os.listdir(PROFILES)) if n.endswith(".md")}


def test_prefill_summaries_name_the_current_sources():
    current = bench.kernel_source_hash()
    named = {n: re.findall(r"`bench\.py --source-hash` = `([0-9a-f]{16})`", t) for n, t in _summaries().items()}
    prefill = {n: h for n, h in named.items() if n.startswith("gdn_prefill") and h}
    assert prefill, "no prefill summary names its sources"
    for n, hashes in prefill.items():
        assert set(hashes) == {current}, f"{n} was measured on sources {hashes}, the current ones are {current}"


def test_per_file_hashes_match():
    found = 0
    for n, text in _summaries().items():
        for name, h in re.findall(r"`(gdn_\w+\.(?:hip|h))`,? (?:sha256 )?`([0-9a-f]{16})", text):
            found += 1
            assert _file_hash(name) == h, f"{n}: {name} has changed since it was measured ({h})"
    assert found >= 4


def test_stored_counters_belong_to_the_current_sources():
    assert bench.COUNTERS_128K is not None
    assert bench.COUNTERS_128K["source_hash"] == bench.kernel_source_hash()
