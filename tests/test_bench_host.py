"""Host-side logic of the benchmark (no GPU): the measured HBM traffic it reports is taken from the
committed rocprofv3 counters only while they belong to the current attention source, and the
oracle baseline records the host it ran on."""
import json

import bench
from lossless_kv_cache_vc_amd import profiling


def _write(path, source_hash):
    rec = {"source_hash": source_hash, "fetch_scale": 2.0, "write_scale": 1.0, "copy_bytes": 1,
           "configs": {"C2": {"command": "x", "kernels": {"verify": {"bytes_per_launch": 123}}}}}
    path.write_text(json.dumps(rec))


def test_traffic_is_reported_only_for_the_current_kernels(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("C2", "verify") is None            # no counters at all
    _write(f, profiling.attn_source_hash())
    assert bench.measured_traffic("C2", "verify") == 123
    assert bench.measured_traffic("C2", "draft") is None             # kernel not profiled
    assert bench.measured_traffic("C3", "verify") is None            # workload not profiled
    _write(f, "0" * 16)                                              # taken on other kernel code
    assert bench.measured_traffic("C2", "verify") is None


def test_host_info_names_the_host():
    h = bench.host_info()
    assert set(h) == {"cpu_model", "logical_cpus", "ram_gib"}
    assert h["logical_cpus"] >= 1


def test_short_steps_are_timed_over_a_minimum_span():
    assert bench.timed_steps(3, 0.06, 0.15) == 3                 # 60 ms rounds: the count holds
    assert bench.timed_steps(3, 0.0008, 0.15) == 188             # 0.8 ms launches: 0.15 s of them
    assert bench.timed_steps(3, 1e-6, 0.15) == 4000              # capped
    assert bench.timed_steps(10, 0.0008, 0.0) == 10              # the headline keeps --steps
