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


def test_threaded_oracle_baseline_splits_into_independent_groups():
    """The CPU baseline's threaded run calls the oracle once per (n, g) group on its channel
    slice; a group's slice with one group must give the whole call's outputs for it, bitwise
    (groups share nothing in the definition), and the run reports the threads it used."""
    import types

    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import bench
    from oracle import oracle as O
    gen = torch.Generator().manual_seed(5)
    N, C, G = 2, 12, 3
    x = (torch.randn(N, C, 4, 6, 5, generator=gen) * 2 + 0.5).to(torch.bfloat16)
    dy = torch.randn(N, C, 4, 6, 5, generator=gen).to(torch.bfloat16)
    gm, bt = torch.randn(C, generator=gen), torch.randn(C, generator=gen)
    whole_y = O.forward(x, G, gm, bt, eps=1e-5)["y"]
    whole = O.backward(dy, x, G, gm, eps=1e-5)
    Cg = C // G
    for n in range(N):
        for g in range(G):
            sl = slice(g * Cg, (g + 1) * Cg)
            xs, ds = x[n:n + 1, sl].contiguous(), dy[n:n + 1, sl].contiguous()
            assert np.array_equal(O.forward(xs, 1, gm[sl], bt[sl], eps=1e-5)["y"], whole_y[n:n + 1, sl])
            part = O.backward(ds, xs, 1, gm[sl], eps=1e-5)
            assert np.array_equal(part["dx"], whole["dx"][n:n + 1, sl])
    r = types.SimpleNamespace(x=x, dy=dy, gamma=gm, beta=bt, G=G, eps=1e-5,
                              case=types.SimpleNamespace(N=N, C=C), step_bytes=16 * x.numel())
    out = bench._oracle_threads(r, min_seconds=0.0, max_reps=2)
    assert 1 <= out["cores"] <= min(16, N * G) and out["value"] > 0
