"""bench.py logic that needs no GPU: the single-GPU contract and the rule
that HBM traffic is reported only for the kernel source it was measured on."""
import hashlib
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_headline_metric_names_decode_bandwidth_and_step_time():
    assert bench.METRIC.startswith("paged-decode KV GB/s (% of HBM peak)")
    assert "\u00b5s/step" in bench.METRIC and "LLaMA-7B" in bench.METRIC


def test_traffic_requires_matching_source_hash(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    digest = hashlib.sha256(b"kernel v1\n").hexdigest()
    (prof / "x_pmc.md").write_text(f"notes\ntraffic_bytes_per_launch: 12345\nsource_sha256: {digest}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("x_pmc.md", ("k.hip",)) == 12345
    src.write_text("kernel v2\n")                      # the kernel changed since profiling
    assert bench.profiled_traffic("x_pmc.md", ("k.hip",)) is None
    assert bench.profiled_traffic("missing.md", ("k.hip",)) is None


def test_committed_decode_profiles_parse():
    for wl in ("llama7b", "llama8b_gqa"):
        path = os.path.join(ROOT, "profiles", f"decode_{wl}_pmc.md")
        text = open(path).read()
        assert "traffic_bytes_per_launch:" in text and "source_sha256:" in text


def test_each_workload_names_its_own_metric():
    """Only the 7B batch carries the headline metric; every other workload's
    line says which shape it measured."""
    names = ["llama7b", "llama8b_gqa", "llama13b_shared", "mixed", "tiny", "prefill", "llama8b_long"]
    assert set(bench.WORKLOAD_METRIC) == set(names)
    assert bench.WORKLOAD_METRIC["llama7b"] == bench.METRIC
    assert len(set(bench.WORKLOAD_METRIC.values())) == len(names)


def test_step_statistics():
    xs = [0.001 * i for i in range(1, 11)]        # 1 .. 10 us, in ms
    st = bench.step_stats(xs)
    assert st["us_per_step"] == 5.5 and st["us_per_step_p10"] == 1.0 and st["us_per_step_p90"] == 9.0
    assert st["us_per_step_median"] == 6.0
    assert bench.percentile([], 50) == 0.0


def test_cpu_baseline_records_the_host():
    line = bench.cpu_baseline_line(1.5, "GB/s", 3, "sample text")
    assert line["cores"] == line["threads_used"] == 3 and line["kind"] == "oracle"
    assert line["host_cores"] == len(os.sched_getaffinity(0))
    assert "cpu_model" in line and "blas" in line
