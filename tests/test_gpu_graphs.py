"""The library under HIP graph capture: it allocates nothing, never synchronizes and
enqueues only kernels on the caller's stream, so one fwd+bwd step can be captured in a
graph and replayed. Every replay (with eager work on the outputs between replays) must
give the eager step's bits."""
import pytest
import torch

import unet_groupnorm_amd as gn
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(f"[gpu-graphs] {msg}", flush=True)


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


CASES = [
    (workloads.DEEP, None, "ncdhw"),                     # resident path, one kernel a direction
    (workloads.TINY, None, "ncdhw"),
    (workloads.custom(1, 128, 16, (32, 32, 32), torch.bfloat16, dist="unet", seed=91), None, "ncdhw"),
    (workloads.custom(2, 24, 6, (17, 13, 11), torch.float16, dist="normal", seed=92), "relu", "ncdhw"),
    (workloads.custom(1, 64, 8, (24, 24, 24), torch.bfloat16, dist="unet", seed=93, out_dtype=torch.float32),
     None, "ncdhw"),
    (workloads.custom(1, 32, 8, (20, 20, 20), torch.bfloat16, dist="unet", seed=94), "relu", "ndhwc"),
]


@pytest.mark.parametrize("case,act,layout", CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_captured_step_replays_bitwise(case, act, layout):
    say(f"{case.name} act={act} layout={layout}: capture one fwd+bwd step, replay 3 times")
    inp = workloads.make(case, DEV)
    x, dy = gn.as_layout(inp["x"], layout), gn.as_layout(inp["dy"], layout)
    gamma, beta, G, eps = inp["gamma"], inp["beta"], inp["G"], inp["eps"]
    y = torch.empty_like(x, dtype=inp["out_dtype"])
    mean = torch.empty((case.N, G), dtype=torch.float32, device=DEV)
    rstd = torch.empty_like(mean)
    dx = torch.empty_like(x)
    dg = torch.empty(case.C, dtype=torch.float32, device=DEV)
    db = torch.empty_like(dg)
    ws = gn.workspace_for(x, G)
    outs = (y, mean, rstd, dx, dg, db)

    def step():
        gn.gn_forward(x, gamma, beta, G, eps, activation=act, workspace=ws, out=y, mean=mean, rstd=rstd)
        gn.gn_backward(dy, x, mean, rstd, gamma, G, beta=beta, activation=act, workspace=ws, dx=dx,
                       dgamma=dg, dbeta=db)

    step()
    torch.cuda.synchronize()
    ref = [_bits(t).clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        for t in outs:
            t.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, t in zip(("y", "mean", "rstd", "dx", "dgamma", "dbeta"), ref, outs):
            assert torch.equal(a, _bits(t)), f"replay {r}: {name} differs from the eager step"
    say(f"{case.name}: 3 replays bitwise equal to the eager step")
