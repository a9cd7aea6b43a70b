"""bench.py host logic, on the CPU: the one-GPU refusal and the stamp that ties an HBM counter record to
the kernel sources it was taken from."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line for a run that did not happen


def test_source_stamp_follows_each_workloads_kernel_files():
    b = _bench()
    stamps = {dt: b.kernel_source_hash(dt) for dt in ("bf16", "f16", "f32", "fp8")}
    for s in stamps.values():
        assert len(s) == 16 and int(s, 16) >= 0
    # the 16-bit workloads launch the same kernel file; the others launch their own
    assert stamps["bf16"] == stamps["f16"]
    assert len({stamps["bf16"], stamps["f32"], stamps["fp8"]}) == 3


def test_counter_record_is_used_only_while_its_sources_are_unchanged(tmp_path, monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "PROFILES", str(tmp_path))
    rec = {"hbm_bytes_per_launch": 12345, "kernel_source_sha256_16": b.kernel_source_hash("f16")}
    (tmp_path / "traffic_cfg4.json").write_text(json.dumps(rec))
    assert b.load_traffic(4, "f16") == 12345
    rec["kernel_source_sha256_16"] = "0" * 16  # taken from other sources: no traffic figure
    (tmp_path / "traffic_cfg4.json").write_text(json.dumps(rec))
    assert b.load_traffic(4, "f16") is None
    assert b.load_traffic(3, "f16") is None  # no record at all
