"""The committed rocprofv3 summaries describe the current kernels.

Every summary under profiles/ states the command that produced it, and
names the sources of the kernels it measures with a hash of their text
(``<file> sha256_16 <hash>``, or the ``kernel_source`` /
``kernel_source_sha256_16`` pair of the traffic files that bench.py reads).
A summary whose hash no longer matches its source measures code that has
since changed: retake it.
"""
import glob
import hashlib
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lossless_speculative_decoding_vc_amd", "csrc")


def _sha16(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _profiles():
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt")))
    assert paths, "no profile summaries"
    return paths


def test_every_summary_states_its_command():
    for p in _profiles():
        text = open(p).read()
        assert re.search(r"^# (command|commands)", text, re.M), f"{os.path.basename(p)} states no command"
        assert "rocprofv3" in text, f"{os.path.basename(p)} does not name rocprofv3"


def test_source_hashes_match_the_tree():
    stale = []
    for p in _profiles():
        text = open(p).read()
        for name, h in re.findall(r"([\w.]+\.(?:hip|cpp)) sha256_16 ([0-9a-f]{16})", text):
            if _sha16(os.path.join(CSRC, name)) != h:
                stale.append(f"{os.path.basename(p)}: {name}")
        m = re.search(r"^kernel_source: (\S+)\nkernel_source_sha256_16: ([0-9a-f]{16})", text, re.M)
        if m and _sha16(os.path.join(ROOT, m.group(1))) != m.group(2):
            stale.append(f"{os.path.basename(p)}: {m.group(1)}")
    assert not stale, "summaries taken on older sources (retake them):\n" + "\n".join(stale)


def test_kernel_summaries_name_their_sources():
    # every kernel-trace or traffic summary of the library's kernels is keyed to its sources
    for p in _profiles():
        name = os.path.basename(p)
        if name.startswith("copy1g") or name.endswith("_memory_copies.txt"):
            continue   # torch's copy kernel (the traffic reference); the runtime's copy engines and blits
        text = open(p).read()
        assert "sha256_16" in text, f"{name} names no source hash"
