"""The library driven through its C ABI alone: device memory from hipMalloc (no torch
allocation), the NULL stream, inputs and results moved with hipMemcpy, outputs compared
element by element with the fp64 oracle. Nothing on the device side comes from torch, so
this shows the boundary needs no torch state (torch on the host only generates the seeded
inputs).
"""
import ctypes

import numpy as np
import pytest
import torch

import unet_groupnorm_amd as gn
import workloads
from oracle import oracle as O
from tests import parity as P
from unet_groupnorm_amd._lib import GN_ACT_NONE, GN_ACT_RELU, GN_BF16, GN_F16, GN_F32, lib

pytestmark = pytest.mark.gpu
H2D, D2H = 1, 2
_CODE = {torch.float32: GN_F32, torch.bfloat16: GN_BF16, torch.float16: GN_F16}


def say(msg):
    print(f"[gpu-c-abi] {msg}", flush=True)


def _hip():
    """The HIP runtime libgn.so is bound to in this process (the same file, so one runtime)."""
    paths = sorted({line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line})
    assert paths, "no HIP runtime loaded"
    h = ctypes.CDLL(paths[0])
    h.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    h.hipFree.argtypes = [ctypes.c_void_p]
    h.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    return h


class Device:
    """hipMalloc'd buffers, freed when the test ends."""

    def __init__(self):
        self.h = _hip()
        self.ptrs = []

    def alloc(self, nbytes):
        p = ctypes.c_void_p()
        assert self.h.hipMalloc(ctypes.byref(p), max(int(nbytes), 256)) == 0
        self.ptrs.append(p)
        return p

    def put(self, arr):
        arr = np.ascontiguousarray(arr)
        p = self.alloc(arr.nbytes)
        assert self.h.hipMemcpy(p, arr.ctypes.data, arr.nbytes, H2D) == 0
        return p

    def get(self, p, like):
        out = np.empty_like(like)
        assert self.h.hipMemcpy(out.ctypes.data, p, out.nbytes, D2H) == 0   # synchronous
        return out

    def free(self):
        for p in self.ptrs:
            self.h.hipFree(p)


def _host_bits(t):
    """The tensor's storage as a numpy array in the form the parity checks read: bf16 as its
    uint16 bits, fp16 and fp32 as themselves."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


CASES = [
    (workloads.custom(2, 12, 3, (9, 7, 5), torch.bfloat16, dist="unet", seed=91), "ncdhw", False),
    (workloads.custom(1, 16, 4, (12, 10, 8), torch.float32, dist="tiny", seed=92), "ncdhw", True),
    (workloads.custom(3, 32, 8, (6, 5, 4), torch.float16, dist="deep", seed=93), "ncdhw", False),
    (workloads.custom(2, 32, 8, (8, 6, 5), torch.bfloat16, dist="unet", seed=94), "ndhwc", True),
]


@pytest.mark.parametrize("case,layout,relu", CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_c_abi_with_hip_memory_and_the_null_stream(case, layout, relu):
    say(f"{case.name}: {layout} relu={relu}, hipMalloc'd buffers, NULL stream")
    inp = workloads.make(case, "cpu")
    x, dy, G, eps, gamma, beta = inp["x"], inp["dy"], inp["G"], inp["eps"], inp["gamma"], inp["beta"]
    N, C = x.shape[:2]
    S = x.numel() // (N * C)
    cl = layout == "ndhwc"
    perm = (0, *range(2, x.dim()), 1)
    to_dev = (lambda t: t.permute(perm)) if cl else (lambda t: t)
    xh, dyh = _host_bits(to_dev(x)), _host_bits(to_dev(dy))
    act = GN_ACT_RELU if relu else GN_ACT_NONE
    d = Device()
    try:
        xp, dyp = d.put(xh), d.put(dyh)
        gp, bp = d.put(gamma.numpy()), d.put(beta.numpy())
        yp, dxp = d.alloc(xh.nbytes), d.alloc(xh.nbytes)
        mp, rp = d.alloc(N * G * 4), d.alloc(N * G * 4)
        dgp, dbp = d.alloc(C * 4), d.alloc(C * 4)
        wsb = (lib.gn_workspace_bytes_cl if cl else lib.gn_workspace_bytes)(N, C, S, G)
        assert wsb > 0
        wsp = d.alloc(wsb)
        fwd, bwd = (lib.gn_forward_cl, lib.gn_backward_cl) if cl else (lib.gn_forward, lib.gn_backward)
        code = _CODE[x.dtype]
        assert fwd(xp, code, gp, bp, N, C, S, G, eps, act, yp, code, mp, rp, wsp, wsb, None) == 0
        assert bwd(dyp, _CODE[dy.dtype], xp, code, mp, rp, gp, bp, act, N, C, S, G, dxp, dgp, dbp, wsp, wsb,
                   None) == 0
        y = d.get(yp, xh)
        dx = d.get(dxp, xh)
        mean = d.get(mp, np.empty(N * G, np.float32))
        rstd = d.get(rp, np.empty(N * G, np.float32))
        dgamma = d.get(dgp, np.empty(C, np.float32))
        dbeta = d.get(dbp, np.empty(C, np.float32))
    finally:
        d.free()
    if cl:   # back to NCDHW element order
        shape_cl = tuple(x.shape[i] for i in perm)
        inv = (0, x.dim() - 1, *range(1, x.dim() - 1))
        y = np.ascontiguousarray(y.reshape(shape_cl).transpose(inv))
        dx = np.ascontiguousarray(dx.reshape(shape_cl).transpose(inv))
    f = O.forward(x, G, gamma, beta, eps=eps, relu=relu)
    rep = P.check_stats(mean, rstd, f["mean"], f["var"], f["rstd"])
    idx = np.arange(x.numel())
    rep.update(P.check_y(y.reshape(-1), f["y"].reshape(-1), *P.channel_params_at(idx, tuple(x.shape), gamma.numpy(),
                                                                                   beta.numpy())))
    b = O.backward(dy, x, G, gamma, eps=eps, beta=beta, relu=relu)
    band = P.ReluBand(x, dy, G, gamma, beta, b["mean"], b["rstd"]) if relu else None
    dx64 = b["dx"].reshape(-1)
    rep.update(P.check_dx(dx.reshape(-1), dx64, band=None if band is None else band.dx_terms(idx, dx64)))
    a_dy, a_dyx = O.channel_abs_sums(dy, x, G, b["mean"], b["rstd"], gamma=gamma, beta=beta, relu=relu)
    depth = P.reduction_depth(gn.gn_plan_query(N, C, S, G), N)   # as the other parity tests take it
    rep.update(P.check_param("dgamma", dgamma, b["dgamma"], a_dyx, depth,
                             (0.0 if band is None else band.dgamma)
                             + P.stats_slack(b["mean"], b["rstd"], a_dy, b["dgamma"], C)))
    rep.update(P.check_param("dbeta", dbeta, b["dbeta"], a_dy, depth, 0.0 if band is None else band.dbeta))
    say(f"{case.name}: ok {rep}")
