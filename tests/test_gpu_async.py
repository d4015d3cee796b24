"""The per-step calls only enqueue: queued on the stream behind tens of milliseconds of copies,
gn_forward and gn_backward return while that work is still running (an event recorded right
after them has not completed), and their results, once the stream drains, are bitwise the
ones of an unqueued call. A call that synchronized the device or the stream, or copied
anything to the host, would return only after the copies, with the event complete."""
import time

import pytest
import torch

import unet_groupnorm_amd as gn
import workloads

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-async] {msg}", flush=True)


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("layout", ["ncdhw", "ndhwc"])
def test_calls_return_before_their_work_runs(layout):
    case = workloads.custom(1, 32, 8, (64, 64, 64), torch.bfloat16, dist="unet", seed=99)
    inp = workloads.make(case, "cuda")
    x, dy = gn.as_layout(inp["x"], layout), gn.as_layout(inp["dy"], layout)
    G, eps, gamma, beta = inp["G"], inp["eps"], inp["gamma"], inp["beta"]
    say(f"{case.name} {layout}: reference step, then the same step queued behind 32 copies of 512 MiB")

    def step():
        y, mean, rstd = gn.gn_forward(x, gamma, beta, G, eps)
        dx, dg, db = gn.gn_backward(dy, x, mean, rstd, gamma, G)
        return [y, mean, rstd, dx, dg, db]

    ref = [t.clone() for t in step()]
    torch.cuda.synchronize()
    src = torch.ones(1 << 27, dtype=torch.int32, device="cuda")   # 512 MiB
    dst = torch.empty_like(src)
    done = torch.cuda.Event()
    t0 = time.perf_counter()
    for _ in range(32):          # about 5 ms of copying at 6 TB/s, enqueued in well under that
        dst.copy_(src)
    t1 = time.perf_counter()
    outs = step()
    t2 = time.perf_counter()
    done.record()
    pending = not done.query()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    say(f"enqueue copies {1e3 * (t1 - t0):.2f} ms, GroupNorm calls {1e3 * (t2 - t1):.2f} ms, "
        f"drain {1e3 * (t3 - t2):.2f} ms, event pending after the calls: {pending}")
    assert pending, "the calls returned only after the queued work had run"
    for a, b in zip(ref, outs):
        assert torch.equal(_bits(a), _bits(b))
