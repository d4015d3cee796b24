"""gn_forward_noalloc, the allocation-free forward, called through the C ABI: its mean,
rstd and y must be bitwise those of gn_forward on the same inputs (the same kernels with the
library's static scratch as the workspace), on calls in a row whose shapes shrink, so that
each call finds the previous call's contents in the shared scratch."""
import ctypes

import pytest
import torch

import unet_groupnorm_amd as gn
import workloads
from unet_groupnorm_amd._lib import GN_NOALLOC_SCRATCH_BYTES, lib

pytestmark = pytest.mark.gpu

_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


def say(msg):
    print(f"[noalloc] {msg}", flush=True)


def _args(x, G):
    N, C = x.shape[:2]
    return N, C, x.numel() // (N * C), G


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


# Calls in a row, each smaller than the one before: the 128^3 site (two-pass kernels), a
# ragged bf16 shape with the relu (two-pass kernels with edge vectors), the tiny fp32
# configuration (the resident kernel), a 2-sample fp32-output shape.
CASES = [
    (workloads.SCALE7, None, None),
    (workloads.custom(2, 48, 12, (17, 19, 23), torch.bfloat16, dist="unet", seed=61), "relu", None),
    (workloads.TINY, None, None),
    (workloads.custom(2, 16, 4, (5, 6, 7), torch.bfloat16, dist="deep", seed=62), None, torch.float32),
]


def test_noalloc_forward_matches_gn_forward_bitwise():
    stream = torch.cuda.current_stream().cuda_stream
    prev = None
    for case, act, out_dtype in CASES:
        assert prev is None or case.numel < prev
        prev = case.numel
        inp = workloads.make(case, "cuda", with_dy=False)
        x, G, eps = inp["x"], inp["G"], inp["eps"]
        N, C, S, G = _args(x, G)
        assert 0 < lib.gn_workspace_bytes(N, C, S, G) <= GN_NOALLOC_SCRATCH_BYTES
        say(f"{case.name} {tuple(x.shape)} {x.dtype} act={act} out={out_dtype}: gn_forward_noalloc vs gn_forward")
        y_ref, m_ref, r_ref = gn.gn_forward(x, inp["gamma"], inp["beta"], G, eps, out_dtype, activation=act)
        y = torch.full_like(y_ref, float("nan"))
        mean = torch.full_like(m_ref, float("nan"))
        rstd = torch.full_like(r_ref, float("nan"))
        rc = lib.gn_forward_noalloc(
            x.data_ptr(), _CODE[x.dtype], inp["gamma"].data_ptr(), inp["beta"].data_ptr(), N, C, S, G,
            ctypes.c_float(eps), 1 if act == "relu" else 0, y.data_ptr(), _CODE[y.dtype], mean.data_ptr(),
            rstd.data_ptr(), ctypes.c_void_p(stream))
        assert rc == 0, lib.gn_status_string(rc)
        torch.cuda.synchronize()
        assert torch.equal(_bits(mean), _bits(m_ref))
        assert torch.equal(_bits(rstd), _bits(r_ref))
        assert torch.equal(_bits(y), _bits(y_ref))
        say(f"{case.name}: bitwise equal")


def test_noalloc_binding_and_oversize_shape():
    case = workloads.custom(1, 8, 4, (9, 10, 11), torch.float32, dist="tiny", seed=63)
    inp = workloads.make(case, "cuda", with_dy=False)
    say(f"{case.name}: binding gn_forward_noalloc vs gn_forward")
    a = gn.gn_forward_noalloc(inp["x"], inp["gamma"], inp["beta"], 4, inp["eps"])
    b = gn.gn_forward(inp["x"], inp["gamma"], inp["beta"], 4, inp["eps"])
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(_bits(u), _bits(v))
    # a shape needing more workspace than the scratch holds is refused before any launch
    x = torch.empty((64, 1024, 2, 2, 2), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gn.GnError) as e:
        gn.gn_forward_noalloc(x, None, None, 32)
    assert e.value.status == 12


def test_noalloc_forward_replayed_from_a_captured_graph():
    """The callers the entry point is for include code under graph capture: one call captured
    (outputs and inputs allocated before the capture, nothing allocated inside it), then the
    graph replayed three times, new inputs copied in and the program's own eager work and a
    synchronization between the replays, each replay bitwise equal to an eager gn_forward."""
    case = workloads.custom(2, 32, 8, (20, 18, 16), torch.bfloat16, dist="unet", seed=64)
    say(f"{case.name}: gn_forward_noalloc captured in a graph, replayed 3 times")
    inp = workloads.make(case, "cuda", with_dy=False)
    x, gamma, beta, G, eps = inp["x"].clone(), inp["gamma"], inp["beta"], inp["G"], inp["eps"]
    y = torch.empty_like(x)
    mean = torch.empty((x.shape[0], G), dtype=torch.float32, device="cuda")
    rstd = torch.empty_like(mean)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gn.gn_forward_noalloc(x, gamma, beta, G, eps, out=y, mean=mean, rstd=rstd)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gn.gn_forward_noalloc(x, gamma, beta, G, eps, out=y, mean=mean, rstd=rstd)
    for seed in (65, 66, 67):
        x.copy_(workloads.make(workloads.custom(2, 32, 8, (20, 18, 16), torch.bfloat16, dist="unet", seed=seed),
                               "cuda", with_dy=False)["x"])
        y_ref, m_ref, r_ref = gn.gn_forward(x, gamma, beta, G, eps)   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(mean), _bits(m_ref)) and torch.equal(_bits(rstd), _bits(r_ref))
        assert torch.equal(_bits(y), _bits(y_ref))
        say(f"replay with inputs of seed {seed}: bitwise equal")
    del graph
