"""The committed rocprofv3 summaries name a hash of the kernel sources they
were measured on; each must still match the sources in the tree, so that no
figure under profiles/ describes code that has since changed."""

import hashlib
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "context_attention_ra_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
LINE = re.compile(r"^Hash of (.+) when measured: ([0-9a-f]{16})\s*$")


def source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def hash_lines():
    out = []
    for fn in sorted(os.listdir(PROFILES)):
        if not fn.endswith(".md"):
            continue
        with open(os.path.join(PROFILES, fn)) as f:
            for line in f:
                m = LINE.match(line)
                if m:
                    out.append((fn, [s.strip() for s in m.group(1).split("+")], m.group(2)))
    return out


def test_every_kernel_profile_names_its_sources():
    lines = hash_lines()
    assert lines, "no profile names the sources it was measured on"
    named = {fn for fn, _, _ in lines}
    for fn in os.listdir(PROFILES):
        if fn.endswith(".md"):
            assert fn in named, f"{fn} names no source hash"


def test_profile_hashes_match_the_sources():
    for fn, names, want in hash_lines():
        assert source_hash(names) == want, f"{fn}: {' + '.join(names)} changed since it was measured"


def test_traffic_counters_match_the_step_kernel_sources():
    # bench.py reports roofline.traffic only while this hash matches; the
    # committed value should be current, not silently dropped to null
    import json
    with open(os.path.join(PROFILES, "traffic.json")) as f:
        rec = json.load(f)
    for key, v in rec.items():
        assert key.startswith("ra_step:")
        assert v["source_hash"] == source_hash(["step_mfma.hip", "ra_device.h", "ra_launch.h"]), key
        assert abs(v["read_bytes"] + v["write_bytes"] - v["bytes_per_launch"]) < 1.0
        assert os.path.exists(os.path.join(ROOT, v["profile"]))
