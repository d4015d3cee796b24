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
