"""Consistency of the committed profiler evidence under profiles/ with the sources at hand.

bench.py reports a kernel's measured HBM traffic only while the SHA-256 of that kernel's
sources still equals the one stored with the counters (profiles/traffic.json), so a kernel
change without a new counter run shows up here, on the CPU, instead of as a silent null in the
bench line.
"""
import hashlib
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")

with open(os.path.join(PROFILES, "traffic.json")) as _f:
    TRAFFIC = json.load(_f)


def _sha256(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


@pytest.mark.parametrize("key", sorted(TRAFFIC))
def test_traffic_counters_match_current_sources(key):
    e = TRAFFIC[key]
    assert _sha256(e["sources"]) == e["sha256"], (
        f"{key}: sources changed since its FETCH_SIZE / WRITE_SIZE runs; measure again")


@pytest.mark.parametrize("key", sorted(TRAFFIC))
def test_traffic_bytes_follow_from_the_counters(key):
    e = TRAFFIC[key]
    # The copy probe reads and writes 1 GiB; each counter's scale is what makes it read that.
    assert e["fetch_scale"] == pytest.approx(2**20 / e["probe_fetch_kib"], rel=1e-5)
    assert e["write_scale"] == pytest.approx(2**20 / e["probe_write_kib"], rel=1e-5)
    kib = e["fetch_kib_per_dispatch"] * e["fetch_scale"] + e["write_kib_per_dispatch"] * e["write_scale"]
    assert e["bytes_per_launch"] == pytest.approx(kib * 1024, rel=1e-5)
    # Measured traffic below the algorithmic bytes would mean a wrong scale or a wrong kernel.
    assert e["bytes_per_launch"] >= e["algorithmic_bytes_per_launch"] * 0.999
    assert os.path.exists(os.path.join(ROOT, e["summary"]))


@pytest.mark.parametrize("name", sorted(f for f in os.listdir(PROFILES) if f.endswith(".md")))
def test_each_summary_gives_the_command_that_made_it(name):
    with open(os.path.join(PROFILES, name)) as f:
        text = f.read()
    assert "rocprofv3" in text and "bench.py" in text, name
