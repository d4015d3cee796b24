"""On the GPU: pointer arguments that are not device memory of x's device are refused with
GN_ERR_DEVICE before anything is enqueued, by the library itself (called through the C ABI
with a host or pinned-host pointer where a device buffer belongs), and by the binding for
tensors on the host."""
import ctypes

import numpy as np
import pytest
import torch

import unet_groupnorm_amd as gn
import workloads
from unet_groupnorm_amd._lib import GN_BF16, lib

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[validation] {msg}", flush=True)


@pytest.fixture(scope="module")
def bufs():
    case = workloads.custom(1, 8, 4, (8, 8, 8), torch.bfloat16, dist="unet", seed=71)
    inp = workloads.make(case, "cuda")
    N, C, S, G = 1, 8, 512, 4
    d = dict(inp)
    d.update(N=N, C=C, S=S, G=G, y=torch.empty_like(inp["x"]), dx=torch.empty_like(inp["x"]),
             mean=torch.empty(N * G, device="cuda"), rstd=torch.empty(N * G, device="cuda"),
             dgamma=torch.empty(C, device="cuda"), dbeta=torch.empty(C, device="cuda"),
             ws=torch.empty(lib.gn_workspace_bytes(N, C, S, G), dtype=torch.uint8, device="cuda"))
    d["host"] = np.zeros(1 << 16, dtype=np.float32)               # pageable host memory
    d["pinned"] = torch.zeros(1 << 14, dtype=torch.float32, pin_memory=True)
    return d


def _fwd(b, **over):
    p = dict(x=b["x"].data_ptr(), gamma=b["gamma"].data_ptr(), beta=b["beta"].data_ptr(), y=b["y"].data_ptr(),
             mean=b["mean"].data_ptr(), rstd=b["rstd"].data_ptr(), ws=b["ws"].data_ptr())
    p.update(over)
    return lib.gn_forward(p["x"], GN_BF16, p["gamma"], p["beta"], b["N"], b["C"], b["S"], b["G"], ctypes.c_float(1e-5),
                          0, p["y"], GN_BF16, p["mean"], p["rstd"], p["ws"], b["ws"].numel(), None)


def _bwd(b, **over):
    p = dict(dy=b["dy"].data_ptr(), x=b["x"].data_ptr(), mean=b["mean"].data_ptr(), rstd=b["rstd"].data_ptr(),
             gamma=b["gamma"].data_ptr(), beta=b["beta"].data_ptr(), dx=b["dx"].data_ptr(),
             dgamma=b["dgamma"].data_ptr(), dbeta=b["dbeta"].data_ptr(), ws=b["ws"].data_ptr())
    p.update(over)
    return lib.gn_backward(p["dy"], GN_BF16, p["x"], GN_BF16, p["mean"], p["rstd"], p["gamma"], p["beta"], 0,
                           b["N"], b["C"], b["S"], b["G"], p["dx"], p["dgamma"], p["dbeta"], p["ws"],
                           b["ws"].numel(), None)


def test_correct_pointers_run(bufs):
    assert _fwd(bufs) == 0
    assert _bwd(bufs) == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("arg", ["y", "mean", "rstd", "gamma", "beta", "ws"])
@pytest.mark.parametrize("mem", ["host", "pinned"])
def test_forward_refuses_host_memory(bufs, arg, mem):
    say(f"gn_forward with {arg} in {mem} memory")
    ptr = bufs["host"].ctypes.data if mem == "host" else bufs["pinned"].data_ptr()
    assert _fwd(bufs, **{arg: ptr}) == 8


@pytest.mark.parametrize("arg", ["dy", "mean", "rstd", "gamma", "beta", "dx", "dgamma", "dbeta", "ws"])
@pytest.mark.parametrize("mem", ["host", "pinned"])
def test_backward_refuses_host_memory(bufs, arg, mem):
    say(f"gn_backward with {arg} in {mem} memory")
    ptr = bufs["host"].ctypes.data if mem == "host" else bufs["pinned"].data_ptr()
    assert _bwd(bufs, **{arg: ptr}) == 8


def test_binding_refuses_tensors_off_x_device(bufs):
    x = bufs["x"]
    with pytest.raises(ValueError):
        gn.gn_backward(bufs["dy"].cpu(), x, bufs["mean"], bufs["rstd"], bufs["gamma"], 4)
    with pytest.raises(ValueError):
        gn.gn_backward(bufs["dy"], x, bufs["mean"][:3], bufs["rstd"], bufs["gamma"], 4)
    with pytest.raises(ValueError):
        gn.gn_backward(bufs["dy"], x, bufs["mean"], bufs["rstd"], bufs["gamma"], 4, dgamma=torch.empty(8))
    with pytest.raises(ValueError):
        gn.gn_forward(x, bufs["gamma"], bufs["beta"], 4, out=torch.empty_like(x, device="cpu"))
    with pytest.raises(ValueError):
        gn.gn_forward(x, bufs["gamma"], bufs["beta"], 4, workspace=torch.empty(1 << 16, dtype=torch.uint8))
