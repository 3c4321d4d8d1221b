"""CPU checks of bench.py's host logic: a committed counter summary supplies
the HBM traffic of a bench line only for the workload, step mode, block size
and kernel code it was taken on."""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _record(tmp_path, **over):
    rec = {"source_sha256_16": bench.src_hash(bench.DECODE_SRC), "step_mode": "separate",
           "block_size": 256, "config": "qwen3-8b", "traffic_bytes_per_launch": 123}
    rec.update(over)
    path = tmp_path / "pmc.json"
    path.write_text(json.dumps(rec))
    return str(path)


def test_traffic_only_for_the_profiled_workload(tmp_path):
    p = _record(tmp_path)
    assert bench.traffic_from_profile(p, bench.DECODE_SRC, "separate", 256, "qwen3-8b") == 123
    assert bench.traffic_from_profile(p, bench.DECODE_SRC, "separate", 256, "long") is None
    assert bench.traffic_from_profile(p, bench.DECODE_SRC, "fused", 256, "qwen3-8b") is None
    assert bench.traffic_from_profile(p, bench.DECODE_SRC, "separate", 16, "qwen3-8b") is None
    stale = _record(tmp_path, source_sha256_16="0" * 16)
    assert bench.traffic_from_profile(stale, bench.DECODE_SRC, "separate", 256, "qwen3-8b") is None
    assert bench.traffic_from_profile(str(tmp_path / "missing.json"), bench.DECODE_SRC,
                                      "separate", 256, "qwen3-8b") is None


def test_source_digest_ignores_comments(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    a.write_text("int x = 1;  // one\n\n// note\nint y;\n")
    b.write_text("int x = 1;\nint y;  // another\n")
    assert bench.src_hash(str(a)) == bench.src_hash(str(b))
    b.write_text("int x = 2;\nint y;\n")
    assert bench.src_hash(str(a)) != bench.src_hash(str(b))


def test_committed_decode_records_name_their_workloads():
    """Every decode workload the default bench line reports (and the larger
    GQA groups) has a counter record for the current decode source, so its
    roofline carries measured traffic."""
    for config in ("qwen3-8b", "qwen3-0.6b", "long", "skewed", "gqa8", "gqa16"):
        rec = json.load(open(bench.pmc_decode_file(config)))
        assert rec["config"] == config and rec["step_mode"] == "separate"
        assert rec["block_size"] == 256 and rec["traffic_bytes_per_launch"] > 0
        assert rec["source_sha256_16"] == bench.src_hash(bench.DECODE_SRC), config
    for path, src in ((bench.PMC_PREFILL_FILE, bench.PREFILL_SRC),
                      (bench.PMC_STORE_FILE, bench.STORE_SRC)):
        rec = json.load(open(path))
        assert rec["source_sha256_16"] == bench.src_hash(src) and rec["traffic_bytes_per_launch"] > 0


def test_more_than_one_gpu_is_refused_before_any_device_work():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and r.stdout == ""
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
