"""bench.py's command line on a host without a GPU: more than one GPU is refused with a
message (this path measures one GPU), and the per-workload trace cases are the ones the
profile summaries name."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_trace_cases_are_listed():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0
    for name in ("tiny", "deep", "deep_f32out", "scale7_ndhwc", "scale7_fp16", "scale7_relu", "census", "shard8"):
        assert name in r.stdout, name
