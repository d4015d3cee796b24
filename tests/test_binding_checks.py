"""The binding's checks of caller-supplied tensors, on the host: a buffer of the wrong
size, dtype, layout or device is refused before any pointer reaches the library, which can
check where memory lives but not how large a buffer is. With every tensor right, the call
does reach the library, which then refuses host memory (GN_ERR_DEVICE)."""
import os

import pytest
import torch

import unet_groupnorm_amd as gn
from unet_groupnorm_amd.gn import GnError

N, C, G, SP = 2, 8, 4, (4, 4, 4)


def _x(dtype=torch.bfloat16):
    return torch.randn((N, C) + SP, generator=torch.Generator().manual_seed(3)).to(dtype)


def _vec(n=C):
    return torch.ones(n, dtype=torch.float32)


def test_forward_reaches_the_library_when_every_tensor_is_right():
    x = _x()
    with pytest.raises(GnError) as e:
        gn.gn_forward(x, _vec(), _vec(), G, out=torch.empty_like(x), mean=torch.empty(N, G),
                      rstd=torch.empty(N, G), workspace=torch.empty(1 << 16, dtype=torch.uint8))
    assert e.value.status == 8


@pytest.mark.parametrize("bad", ["mean_numel", "rstd_dtype", "out_dtype", "out_shape", "out_layout",
                                 "gamma_numel", "ws_layout"])
def test_forward_refuses_bad_buffers(bad):
    x = _x()
    kw = dict(out=torch.empty_like(x), mean=torch.empty(N, G), rstd=torch.empty(N, G),
              workspace=torch.empty(1 << 16, dtype=torch.uint8))
    gamma = _vec()
    if bad == "mean_numel":
        kw["mean"] = torch.empty(N * G - 1)
    elif bad == "rstd_dtype":
        kw["rstd"] = torch.empty(N, G, dtype=torch.float64)
    elif bad == "out_dtype":
        kw["out"] = torch.empty_like(x, dtype=torch.int16)
    elif bad == "out_shape":
        kw["out"] = torch.empty((N, C, 4, 4, 3), dtype=x.dtype)
    elif bad == "out_layout":
        kw["out"] = torch.empty_like(x).transpose(2, 3).contiguous().transpose(2, 3)
    elif bad == "gamma_numel":
        gamma = _vec(C - 1)
    elif bad == "ws_layout":
        kw["workspace"] = torch.empty(1 << 17, dtype=torch.uint8)[::2]
    with pytest.raises((ValueError, TypeError)):
        gn.gn_forward(x, gamma, _vec(), G, **kw)


@pytest.mark.parametrize("bad", ["dy_shape", "dy_dtype", "dx_dtype", "dx_shape", "mean_numel",
                                 "dgamma_numel", "dbeta_dtype"])
def test_backward_refuses_bad_buffers(bad):
    x = _x()
    kw = dict(dx=torch.empty_like(x), dgamma=torch.empty(C), dbeta=torch.empty(C),
              workspace=torch.empty(1 << 16, dtype=torch.uint8))
    dy, mean = _x(), torch.empty(N, G)
    if bad == "dy_shape":
        dy = torch.empty((N, C, 4, 4, 5), dtype=x.dtype)
    elif bad == "dy_dtype":
        dy = dy.to(torch.float64)
    elif bad == "dx_dtype":
        kw["dx"] = torch.empty_like(x, dtype=torch.float32)   # dx is written in x's dtype
    elif bad == "dx_shape":
        kw["dx"] = torch.empty((N - 1, C) + SP, dtype=x.dtype)
    elif bad == "mean_numel":
        mean = torch.empty(N * G + 1)
    elif bad == "dgamma_numel":
        kw["dgamma"] = torch.empty(C - 2)
    elif bad == "dbeta_dtype":
        kw["dbeta"] = torch.empty(C, dtype=torch.float16)
    with pytest.raises((ValueError, TypeError)):
        gn.gn_backward(dy, x, mean, torch.empty(N, G), _vec(), G, **kw)


def test_backward_reaches_the_library_when_every_tensor_is_right():
    x = _x()
    with pytest.raises(GnError) as e:
        gn.gn_backward(_x(), x, torch.empty(N, G), torch.empty(N, G), _vec(), G, dx=torch.empty_like(x),
                       dgamma=torch.empty(C), dbeta=torch.empty(C),
                       workspace=torch.empty(1 << 16, dtype=torch.uint8))
    assert e.value.status == 8


def test_split_phase_and_noalloc_refuse_bad_buffers():
    x = _x()
    ws = torch.empty(1 << 16, dtype=torch.uint8)
    with pytest.raises(ValueError):
        gn.gn_forward_stats(x, _vec(), _vec(), G, 1e-5, torch.empty(N * G - 1), torch.empty(N, G), ws)
    with pytest.raises(TypeError):
        gn.gn_backward_apply(_x(), x, G, torch.empty_like(x, dtype=torch.int32), ws)
    with pytest.raises(ValueError):
        gn.gn_backward_finish(_x(), x, torch.empty(N, G), torch.empty(N, G), _vec(), G, None,
                              torch.empty(C + 1), None, ws)
    with pytest.raises(ValueError):
        gn.gn_forward_noalloc(x, _vec(), _vec(), G, mean=torch.empty(3), rstd=torch.empty(N, G))
    with pytest.raises(GnError) as e:
        gn.gn_forward_noalloc(x, _vec(), _vec(), G)
    assert e.value.status == 8


def test_compiled_binding_is_the_in_tree_module_over_the_same_library():
    from unet_groupnorm_amd import _gnbind
    from unet_groupnorm_amd._lib import lib
    assert _gnbind.abi_version() == lib.gn_abi_version()
    here = os.path.dirname(os.path.abspath(gn.__file__))
    assert os.path.dirname(os.path.abspath(_gnbind.__file__)) == here


def test_compiled_binding_refuses_what_the_helpers_refuse():
    x = _x()
    with pytest.raises(ValueError, match="layout"):
        gn.gn_forward(x, _vec(), _vec(), G, layout="nchw")
    with pytest.raises(ValueError, match="layout"):
        gn.gn_forward(x, _vec(), _vec(), G, layout="ndhwc")      # x is NCDHW-contiguous, C > 1
    with pytest.raises(TypeError):
        gn.gn_forward(x, _vec(), _vec(), G, out_dtype=torch.float64)
    with pytest.raises(TypeError):
        gn.gn_forward(x.to(torch.int32), _vec(), _vec(), G)
    with pytest.raises(ValueError, match="activation"):
        gn.gn_backward(_x(), x, torch.empty(N, G), torch.empty(N, G), _vec(), G, activation="gelu")
    with pytest.raises(ValueError):
        gn.gn_forward(torch.zeros(4), None, None, 1)
    # a shape with no plan reports the planner's status under the size query's name
    with pytest.raises(GnError, match="gn_workspace_bytes") as e:
        gn.gn_forward(torch.zeros((1, 6, 2, 2, 2), dtype=torch.bfloat16), None, None, 4)
    assert e.value.status == 3


def test_compiled_binding_takes_the_layout_from_the_strides():
    # every buffer right but in host memory: the outputs are allocated before the library
    # refuses the call, so their absence cannot be what it reports
    x = _x().contiguous(memory_format=torch.channels_last_3d)
    with pytest.raises(GnError) as e:
        gn.gn_forward(x, _vec(), _vec(), G)
    assert e.value.status == 8 and "gn_forward_cl" in str(e.value)
    with pytest.raises(GnError) as e:
        gn.gn_backward(_x().contiguous(memory_format=torch.channels_last_3d), x, torch.empty(N, G),
                       torch.empty(N, G), _vec(), G, need_dx=False)
    assert e.value.status == 8 and "gn_backward_cl" in str(e.value)
