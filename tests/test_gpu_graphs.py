"""The library under HIP graph capture: it allocates nothing, never synchronizes and
enqueues only kernels on the caller's stream, so one fwd+bwd step, or the calls of many
sites and of GroupNorms in a chain, can be captured in one graph and replayed. Every replay (with eager work on the outputs between replays) must
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


class _Site:
    """Preallocated outputs and workspace of one GroupNorm site."""

    def __init__(self, x, gamma, beta, G, eps, out_dtype=None, layout="ncdhw"):
        self.x, self.gamma, self.beta, self.G, self.eps = gn.as_layout(x, layout), gamma, beta, G, eps
        N, C = x.shape[0], x.shape[1]
        self.y = torch.empty_like(self.x, dtype=out_dtype or x.dtype)
        self.mean = torch.empty((N, G), dtype=torch.float32, device=DEV)
        self.rstd = torch.empty_like(self.mean)
        self.dx = torch.empty_like(self.x)
        self.dg = torch.empty(C, dtype=torch.float32, device=DEV)
        self.db = torch.empty_like(self.dg)
        self.ws = gn.workspace_for(self.x, G)

    def outs(self):
        return (self.y, self.mean, self.rstd, self.dx, self.dg, self.db)

    def forward(self, x=None):
        gn.gn_forward(self.x if x is None else x, self.gamma, self.beta, self.G, self.eps, workspace=self.ws,
                      out=self.y, mean=self.mean, rstd=self.rstd)

    def backward(self, dy, x=None):
        gn.gn_backward(dy, self.x if x is None else x, self.mean, self.rstd, self.gamma, self.G, beta=self.beta,
                       workspace=self.ws, dx=self.dx, dgamma=self.dg, dbeta=self.db)


def test_one_graph_holds_several_sites_and_a_chain():
    """Sites on the resident, two-kernel and channels-last paths, and two GroupNorms in a
    chain (the second normalizes the first's output; its dx is the first's dy), all captured
    in one graph: every replay gives the eager pass's bits."""
    say("several sites and a chain in one graph, 3 replays")
    gen = torch.Generator().manual_seed(2024)
    sites, dys = [], []
    for case, layout in ((workloads.DEEP, "ncdhw"),
                         (workloads.custom(1, 128, 16, (32, 32, 32), torch.bfloat16, dist="unet", seed=95), "ncdhw"),
                         (workloads.custom(2, 32, 8, (12, 10, 9), torch.bfloat16, dist="unet", seed=96), "ndhwc")):
        inp = workloads.make(case, DEV)
        sites.append(_Site(inp["x"], inp["gamma"], inp["beta"], inp["G"], inp["eps"], inp["out_dtype"], layout))
        dys.append(gn.as_layout(inp["dy"], layout))
    shape = (1, 32, 16, 16, 16)
    xa = (torch.randn(shape, generator=gen) * 1.5 + 0.25).to(torch.bfloat16).to(DEV)
    a = _Site(xa, torch.randn(32, generator=gen).to(DEV), torch.randn(32, generator=gen).to(DEV), 8, 1e-5)
    b = _Site(a.y, (torch.randn(32, generator=gen) * 0.1 + 1).to(DEV), torch.randn(32, generator=gen).to(DEV),
              4, 1e-5)
    dyb = torch.randn(shape, generator=gen).to(torch.bfloat16).to(DEV)
    every = sites + [a, b]

    def one_pass():
        for s, dy in zip(sites, dys):
            s.forward()
            s.backward(dy)
        a.forward()
        b.forward()          # b.x is a.y
        b.backward(dyb)
        a.backward(b.dx)     # the chain's gradient flows back through a

    one_pass()
    torch.cuda.synchronize()
    ref = [[_bits(t).clone() for t in s.outs()] for s in every]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one_pass()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass()
    torch.cuda.synchronize()
    for r in range(3):
        for s in every:
            for t in s.outs():
                t.fill_(float("nan"))
            s.ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (s, want) in enumerate(zip(every, ref)):
            for name, w, t in zip(("y", "mean", "rstd", "dx", "dgamma", "dbeta"), want, s.outs()):
                assert torch.equal(w, _bits(t)), f"replay {r}: site {i} {name} differs from the eager pass"
    say("several sites and a chain: 3 replays bitwise equal to the eager pass")
