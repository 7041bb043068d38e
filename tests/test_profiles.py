"""The rocprofv3 summaries under profiles/ belong to the kernels in this tree.

bench.py reports a kernel's measured HBM traffic only when the summary's
recorded source hash matches the current kernel source, so a kernel edited
without re-taking its profile would silently lose that figure.  These checks
run on the CPU."""
import json

import pytest

import bench

CSRC = bench.ROOT / "transformer_scaled_dot_flash_amd" / "csrc"


@pytest.mark.parametrize("name", sorted(bench.KERNELS))
def test_profile_matches_current_kernel_source(name):
    sub, files = bench.KERNELS[name]
    traffic = bench.PROFILES / f"{name}_traffic.json"
    summary = bench.PROFILES / f"{name}.md"
    assert traffic.exists() and summary.exists(), f"missing profile for {name}"
    rec = json.loads(traffic.read_text())
    assert sub in rec["kernel"], f"{name}: profiled kernel {rec['kernel']} is not {sub}"
    digest = bench.source_digest([CSRC / f for f in files])
    assert rec["source_sha256"] == digest, f"{name}: profile taken on other kernel source; re-take it"
    assert bench.traffic_from_profile(name, digest) == rec["hbm_bytes_per_launch"]
    # the summary names the same kernel and quotes the command that made it
    text = summary.read_text()
    assert rec["kernel"] in text and "rocprofv3" in text


def test_traffic_records_are_consistent():
    for name in bench.KERNELS:
        rec = json.loads((bench.PROFILES / f"{name}_traffic.json").read_text())
        total = rec["hbm_fetch_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
        assert abs(rec["hbm_bytes_per_launch"] - total) <= 1  # each figure rounded on its own
        assert rec["algorithmic_bytes_per_launch"] == bench.algorithmic_bytes(name)
        assert rec["avg_duration_us"] >= rec["min_duration_us"] > 0


@pytest.mark.parametrize("path", sorted(bench.PROFILES.glob("*_counters.json")), ids=lambda p: p.stem)
def test_counter_profiles_match_current_kernel_source(path):
    name = path.stem[: -len("_counters")]
    sub, files = bench.KERNELS[name]
    rec = json.loads(path.read_text())
    assert sub in rec["kernel"]
    assert rec["source_sha256"] == bench.source_digest([CSRC / f for f in files]), \
        f"{name}: shader counters taken on other kernel source; re-take them"
    assert (bench.PROFILES / f"{name}_counters.md").exists()
