"""The dgamma bar against an implementation that is exact except for consuming fp32-
rounded statistics: the fp64 sum with the oracle's mean and rstd rounded to fp32 must sit
well inside the bar, on cases where the mean dwarfs the spread (the 'deep' distribution)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import oracle as O
from tests import parity as P


def _dgamma_with_fp32_stats(x, dy, G, b):
    N, C = x.shape[:2]
    m32 = b["mean"].astype(np.float32).astype(np.float64)
    r32 = b["rstd"].astype(np.float32).astype(np.float64)
    xx = x.double().numpy().reshape(N, G, C // G, -1)
    g = dy.double().numpy().reshape(N, G, C // G, -1)
    return (g * (xx - m32[:, :, None, None]) * r32[:, :, None, None]).sum(axis=(0, 3)).reshape(C)


@pytest.mark.parametrize("shape", [(1, 128, 16, (2, 2, 2)), (3, 48, 16, (266,)), (1, 16, 2, (213,))])
def test_fp32_statistics_fit_the_dgamma_bar(shape):
    N, C, G, sp = shape
    case = workloads.custom(N, C, G, sp, torch.float32, torch.bfloat16, dist="deep", seed=4242)
    inp = workloads.make(case, "cpu")
    x, dy = inp["x"], inp["dy"]
    b = O.backward(dy, x, G, inp["gamma"], eps=inp["eps"])
    a_dy, a_dyx = O.channel_abs_sums(dy, x, G, b["mean"], b["rstd"])
    got = _dgamma_with_fp32_stats(x, dy, G, b)
    rep = P.check_param("dgamma", got, b["dgamma"], a_dyx, 1,
                        P.stats_slack(b["mean"], b["rstd"], a_dy, b["dgamma"], C))
    assert rep["dgamma_of_bar"] < 0.5


@pytest.fixture(scope="module")
def scale7_offset_reference():
    """The oracle's dgamma/dbeta and per-channel magnitudes on the 128^3 site with a dy whose
    channel sums do not cancel (the case the GPU's full-size check runs)."""
    case = workloads.SCALE7_DY_OFFSET
    inp = workloads.make(case, "cpu")
    x, dy, G = inp["x"], inp["dy"], inp["G"]
    b = O.backward(dy, x, G, inp["gamma"], eps=inp["eps"], want_dx=False)
    a_dy, a_dyx = O.channel_abs_sums(dy, x, G, b["mean"], b["rstd"])
    return case, b, a_dy, a_dyx


def test_full_size_param_bar_binds_at_the_stated_tolerance(scale7_offset_reference):
    """At 128^3 the dgamma/dbeta bar is 1e-4 of the reference on every channel of this case:
    a 1e-3 relative error is refused, a 5e-5 one accepted, whatever the summation depth."""
    case, b, a_dy, a_dyx = scale7_offset_reference
    depth = 54  # the depth of the kernels' summation tree at this shape (it must not matter here)
    for name, ref, terms in (("dgamma", b["dgamma"], a_dyx), ("dbeta", b["dbeta"], a_dy)):
        assert P.well_conditioned(ref, terms).all(), name
        slack = P.stats_slack(b["mean"], b["rstd"], a_dy, ref, case.C) if name == "dgamma" else 0.0
        assert np.all(slack < 1e-6 * np.abs(ref))
        sign = np.where(np.arange(case.C) % 2 == 0, 1.0, -1.0)
        rep = P.check_param(name, ref * (1 + 5e-5 * sign), ref, terms, depth, slack)
        assert rep[f"{name}_well_conditioned"] == case.C and 0.45 < rep[f"{name}_of_bar"] < 0.55
        for c in (0, 17, case.C - 1):
            bad = ref.copy()
            bad[c] *= 1 + 1e-3 * sign[c]
            with pytest.raises(AssertionError):
                P.check_param(name, bad, ref, terms, depth, slack)


def test_zero_mean_dy_leaves_every_channel_to_the_summation_floor():
    """With the zero-mean dy of the other recipes the channel sums cancel, and no channel is
    held to the relative bar alone (the floor applies)."""
    case = workloads.custom(1, 8, 4, (48, 48, 48), torch.bfloat16, dist="unet", seed=4243)
    inp = workloads.make(case, "cpu")
    b = O.backward(inp["dy"], inp["x"], 4, inp["gamma"], eps=inp["eps"], want_dx=False)
    a_dy, a_dyx = O.channel_abs_sums(inp["dy"], inp["x"], 4, b["mean"], b["rstd"])
    assert not P.well_conditioned(b["dbeta"], a_dy).any()
    assert not P.well_conditioned(b["dgamma"], a_dyx).any()
