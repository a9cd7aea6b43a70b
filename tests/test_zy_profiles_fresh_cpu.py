"""The HBM counter records under profiles/ belong to the kernel sources in the tree: bench.py reports a
roofline traffic figure only for a record stamped with the current sources, so every forward workload
whose record is committed must still match (a kernel change without new counters fails here)."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_forward_traffic_records_match_the_kernel_sources():
    spec = importlib.util.spec_from_file_location("bench_profiles_check", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    for config, dtype in ((2, "bf16"), (3, "bf16"), (4, "f16"), (5, "fp8")):
        assert b.load_traffic(config, dtype) is not None, f"profiles/traffic_cfg{config}.json is stale or missing"
