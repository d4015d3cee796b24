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


def test_all_core_oracle_gives_the_whole_calls_bits():
    """The CPU baseline's all-core run splits each direction into per-(n, g) group calls and
    per-(n, c) row calls of the oracle; every output must be the whole-volume call's, bitwise
    (the definition's sums run over the same elements in the same order), on a ragged shape
    with several samples and groups."""
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
    f = O.forward(x, G, gm, bt, eps=1e-5)
    b = O.backward(dy, x, G, gm, eps=1e-5)
    out = bench.oracle_all_cores(x, dy, gm, bt, G, 1e-5, min_seconds=0.0, max_reps=1, workers=3)
    o = out["_outputs"]
    for k in ("mean", "rstd", "y"):
        assert np.array_equal(o[k], f[k]), k
    for k in ("dx", "dgamma", "dbeta"):
        assert np.array_equal(o[k], b[k]), k
    assert out["cores"] == 3 and out["forward"]["seconds"] > 0 and out["backward"]["seconds"] > 0
