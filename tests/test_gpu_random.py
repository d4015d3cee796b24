"""Seeded random shapes through the HIP path, element by element against the fp64 oracle.

Each case draws N, C, G, a ragged spatial extent, the input / output / dy dtypes, the
value distribution, the fused relu and (where the shape allows) the channels-last layout,
so that plan branches (resident or two-pass, one or many jobs per row, masked edges,
every slot arrangement of the channels-last kernels) are hit in combinations no named
case lists. The draw is fixed by the seed: a failing case is reproduced by its id.
"""
import numpy as np
import pytest
import torch

import workloads
from tests.test_gpu_parity import full_check

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.bfloat16, torch.float16]


def _draw(i):
    rng = np.random.default_rng(9000 + i)
    G = int(rng.choice([1, 2, 3, 4, 8, 16]))
    cg = int(rng.choice([1, 2, 3, 4, 8, 16]))
    C = G * cg
    N = int(rng.integers(1, 5))
    nd = int(rng.integers(1, 4))
    budget = int(rng.choice([200, 3000, 40000, 300000])) // max(1, N * C)
    budget = max(budget, 1)
    spatial = []
    for _ in range(nd):
        spatial.append(int(max(1, round(budget ** (1.0 / nd) * rng.uniform(0.6, 1.4)))))
    if N * cg * int(np.prod(spatial)) == 1:
        spatial[0] += 1
    x_dtype = DTYPES[int(rng.integers(0, 3))]
    out_dtype = torch.float32 if (x_dtype != torch.float32 and rng.random() < 0.3) else None
    dy_dtype = DTYPES[int(rng.integers(0, 3))] if out_dtype is None else torch.float32
    dist = str(rng.choice(["unet", "normal", "tiny", "deep"]))
    relu = bool(rng.random() < 0.3)
    cl_ok = C % 8 == 0 and 256 % (C // 8) == 0 and (cg % 8 == 0 or 8 % cg == 0)
    layout = "ndhwc" if (cl_ok and rng.random() < 0.5) else "ncdhw"
    case = workloads.custom(N, C, G, tuple(spatial), x_dtype, dy_dtype, dist=dist, seed=9000 + i,
                            out_dtype=out_dtype)
    return case, relu, layout


def _draw_large(i):
    """Volumes of 0.5-4 million elements and wider groups: many reduction jobs per row,
    folded jobs split across rows, both sides of the resident limit."""
    rng = np.random.default_rng(9500 + i)
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    cg = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    C = G * cg
    N = int(rng.integers(1, 5))
    nd = int(rng.integers(1, 4))
    budget = max(1, int(rng.choice([500000, 1500000, 4000000])) // (N * C))
    spatial = [int(max(1, round(budget ** (1.0 / nd) * rng.uniform(0.7, 1.3)))) for _ in range(nd)]
    x_dtype = DTYPES[int(rng.integers(0, 3))]
    dy_dtype = DTYPES[int(rng.integers(0, 3))]
    dist = str(rng.choice(["unet", "normal", "deep"]))
    relu = bool(rng.random() < 0.3)
    cl_ok = C % 8 == 0 and 256 % (C // 8) == 0 and (cg % 8 == 0 or 8 % cg == 0)
    layout = "ndhwc" if (cl_ok and rng.random() < 0.5) else "ncdhw"
    case = workloads.custom(N, C, G, tuple(spatial), x_dtype, dy_dtype, dist=dist, seed=9500 + i)
    return case, relu, layout


def _draw_large16(i):
    """Large volumes of 16-bit inputs (whose full steps are read through buffer resources)
    with the relu on half the time (the relu and plain builds of every kernel)."""
    rng = np.random.default_rng(9700 + i)
    G = int(rng.choice([2, 4, 8, 16]))
    cg = int(rng.choice([1, 2, 4, 8]))
    C = G * cg
    N = int(rng.integers(1, 4))
    nd = int(rng.integers(1, 4))
    budget = max(1, int(rng.choice([1000000, 3000000])) // (N * C))
    spatial = [int(max(1, round(budget ** (1.0 / nd) * rng.uniform(0.7, 1.3)))) for _ in range(nd)]
    x_dtype = [torch.bfloat16, torch.float16][int(rng.integers(0, 2))]
    dy_dtype = DTYPES[int(rng.integers(0, 3))]
    relu = bool(rng.random() < 0.5)
    case = workloads.custom(N, C, G, tuple(spatial), x_dtype, dy_dtype, dist="unet", seed=9700 + i)
    return case, relu, "ncdhw"


CASES = [_draw(i) for i in range(32)] + [_draw_large(i) for i in range(16)] + [_draw_large16(i) for i in range(8)]


def _id(v):
    case, relu, layout = v
    return (f"{case.name}_{str(case.x_dtype).split('.')[-1]}_{str(case.dy_dtype).split('.')[-1]}"
            f"{'_relu' if relu else ''}_{layout}")


@pytest.mark.parametrize("draw", CASES, ids=_id)
def test_random_shape_elementwise(draw):
    case, relu, layout = draw
    inp = workloads.make(case, "cpu")
    full_check(inp, _id(draw), relu=relu, layout=layout)
