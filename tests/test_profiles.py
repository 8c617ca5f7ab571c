"""The counter summaries under profiles/ describe the kernels as committed:
each names the sha256 prefix of the kernel source it was taken from, and
that must be the source in the tree (a kernel changed after its counters
were taken makes its figures stale)."""
import hashlib
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_prefill_swa_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# profile file name prefix -> kernel source it measures
SOURCES = {
    "band_persist_": "band_persist.hip",
    "band_roll_": "band_roll.hip",
    "band_bwd_": "band_bwd.hip",
    "splitkv_": "splitkv_mfma.hip",
}


def _sha16(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _hashed_profiles():
    out = []
    for name in sorted(os.listdir(PROFILES)):
        text = open(os.path.join(PROFILES, name)).read()
        m = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
        if m:
            out.append((name, m.group(1)))
    return out


def test_every_kernel_profile_names_its_source():
    names = [n for n, _ in _hashed_profiles()]
    for prefix in SOURCES:
        assert any(n.startswith(prefix) for n in names), prefix


@pytest.mark.parametrize("name,sha", _hashed_profiles())
def test_profile_matches_committed_kernel(name, sha):
    src = [s for p, s in SOURCES.items() if name.startswith(p)]
    assert len(src) == 1, f"{name}: no kernel source mapped"
    assert _sha16(os.path.join(CSRC, src[0])) == sha, (
        f"{name} was taken from another version of {src[0]}")
