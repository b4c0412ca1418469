"""The benchmark's contract checks that need no GPU: one GPU only, and the
counter-derived traffic is taken only from a summary of the same sources."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_only_from_a_summary_of_the_same_sources():
    b = _bench()
    with open(b.PMC_SUMMARY) as fh:
        fields = dict(line.split(":", 1) for line in fh.read().splitlines() if ":" in line)
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    recorded, workload = fields["kernel_sources"], fields["workload"]
    t = b.measured_traffic(workload, recorded)
    assert isinstance(t, int) and t > 0
    assert b.measured_traffic(workload, "0" * 16) is None
    assert b.measured_traffic("another_workload", recorded) is None
    assert len(b.gather_source_hash()) == 16
