"""Host logic of bench.py: which committed traffic summary a run reports."""
import importlib.util
import os

import pytest

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(_ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_summary_is_matched_by_exact_workload_key(bench, tmp_path):
    """A summary titled for the cascade call must not serve the plain decode of
    the same batch, and a stale source hash disables every summary."""
    import hashlib
    csrc = os.path.join(_ROOT, "paged_kv_cache_135_amd", "csrc")
    h = hashlib.sha256()
    for name in ("decode.hip", "tile.h"):
        h.update(open(os.path.join(csrc, name), "rb").read())
    sha = h.hexdigest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "a_pmc_traffic.md").write_text(
        f"# rocprofv3 PMC byte counters: c3_shared_prefix+cascade decode step\n"
        f"decode.hip+tile.h sha256: {sha}\nkernel: call\ntraffic_bytes_per_launch: 111\n")
    (prof / "b_pmc_traffic.md").write_text(
        f"# rocprofv3 PMC byte counters: c2_qwen_decode decode step\n"
        f"decode.hip+tile.h sha256: {'0' * 64}\nkernel: k\ntraffic_bytes_per_launch: 222\n")
    root = str(tmp_path)
    assert bench.measured_traffic("c3_shared_prefix+cascade", root) == (111, "call")
    assert bench.measured_traffic("c3_shared_prefix", root) == (None, None)
    assert bench.measured_traffic("c2_qwen_decode", root) == (None, None)  # stale hash


def test_committed_summaries_name_distinct_workloads(bench):
    keys = []
    for name in sorted(os.listdir(os.path.join(_ROOT, "profiles"))):
        if name.endswith("_pmc_traffic.md"):
            first = open(os.path.join(_ROOT, "profiles", name)).readline()
            keys.append(first.split(":", 1)[-1].strip())
    assert keys and len(keys) == len(set(keys))
