"""Host-side checks of the benchmark and profiling drivers (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_unknown_leg_is_refused():
    r = _bench("--legs", "decode,nonsense")
    assert r.returncode == 2
    assert "nonsense" in r.stderr


def test_profile_entries_name_existing_sources():
    import profile_kernels

    for kern, wname, src, pmc, _ in profile_kernels.entries():
        assert pmc in profile_kernels.PMC_BENCHES
        assert len(profile_kernels.source_sha(src)) == 64, (kern, wname)


def test_dispatches_split_between_workloads_by_duration():
    import profile_kernels

    # two workloads of one kernel, 0.12 ms and 5.8 ms per launch
    durs = [118_000, 5_900_000, 121_000, 5_750_000, 130_000]
    got = profile_kernels._attribute(durs, {"small": 0.12, "large": 5.8})
    assert sorted(got["small"]) == [118_000, 121_000, 130_000]
    assert sorted(got["large"]) == [5_750_000, 5_900_000]
