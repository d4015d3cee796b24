"""Global statistics over spatial shards, on one GPU: a volume is split along D into P
contiguous shards (uneven where D is not a multiple of P), each shard plays a rank, the
records are gathered by stacking them in shard order (what one all-gather does between
GPUs), and the reassembled outputs are compared with the fp64 oracle on the whole volume.
Every rank's merged statistics and parameter gradients must be bitwise identical.
"""
import numpy as np
import pytest
import torch

import unet_groupnorm_amd as gn
import workloads
from oracle import oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(f"[gpu-shards] {msg}", flush=True)


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


def run_sharded(inp, nshards, relu=False):
    """The sharded forward and backward; returns outputs of the whole volume plus every
    rank's merged statistics and parameter gradients."""
    x, dy, G, eps = inp["x"], inp["dy"], inp["G"], inp["eps"]
    gamma, beta = inp["gamma"], inp["beta"]
    act = "relu" if relu else None
    xs = [t.contiguous() for t in torch.tensor_split(x, nshards, dim=2)]
    dys = [t.contiguous() for t in torch.tensor_split(dy, nshards, dim=2)]
    wss = [gn.workspace_for(t, G) for t in xs]
    recs = torch.stack([gn.gn_forward_shard_stats(t, G, workspace=w) for t, w in zip(xs, wss)])
    stats = [gn.gn_forward_shard_merge(recs, gamma, beta, t.shape, G, eps, workspace=w) for t, w in zip(xs, wss)]
    ys = []
    for t, w in zip(xs, wss):
        yy = torch.empty_like(t, dtype=inp["out_dtype"])
        gn.gn_forward_apply(t, G, yy, w, activation=act)
        ys.append(yy)
    mean, rstd = stats[0]
    sums = torch.stack([gn.gn_backward_shard_sums(d, t, mean, rstd, gamma, G, beta=beta, activation=act, workspace=w)
                        for d, t, w in zip(dys, xs, wss)])
    S_total = x.numel() // (x.shape[0] * x.shape[1])
    params = [gn.gn_backward_shard_merge(sums, mean, rstd, gamma, t.shape, S_total, G, beta=beta, workspace=w)
              for t, w in zip(xs, wss)]
    dxs = []
    for d, t, w in zip(dys, xs, wss):
        dd = torch.empty_like(t)
        gn.gn_backward_apply(d, t, G, dd, w, activation=act)
        dxs.append(dd)
    torch.cuda.synchronize()
    return {"y": torch.cat(ys, dim=2), "dx": torch.cat(dxs, dim=2), "mean": mean, "rstd": rstd,
            "dgamma": params[0][0], "dbeta": params[0][1], "stats": stats, "params": params}


def check_ranks_agree(r):
    m0, r0 = r["stats"][0]
    for m, rs in r["stats"][1:]:
        assert torch.equal(_bits(m), _bits(m0)) and torch.equal(_bits(rs), _bits(r0))
    g0, b0 = r["params"][0]
    for g, b in r["params"][1:]:
        assert torch.equal(_bits(g), _bits(g0)) and torch.equal(_bits(b), _bits(b0))


def depth_bound(x, G, nshards):
    """A bound on the depth of the fp32 summation tree behind dgamma/dbeta: the deepest
    shard's per-row tree plus the shards and samples added in order."""
    N, C = x.shape[:2]
    S = max(t.numel() // (N * C) for t in torch.tensor_split(x, nshards, dim=2))
    return P.reduction_depth(gn.gn_plan_query(N, C, S, G), 1) + 8 + nshards + N


def full_compare(inp, r, tag, nshards, relu=False):
    x, dy, G, eps = inp["x"].cpu(), inp["dy"].cpu(), inp["G"], inp["eps"]
    gamma, beta = inp["gamma"].cpu(), inp["beta"].cpu()
    f = O.forward(x, G, gamma, beta, eps=eps, relu=relu)
    rep = P.check_stats(P.to_np(r["mean"]), P.to_np(r["rstd"]), f["mean"], f["var"], f["rstd"])
    idx = np.arange(x.numel())
    rep.update(P.check_y(P.to_np(r["y"]).reshape(-1), f["y"].reshape(-1),
                         *P.channel_params_at(idx, tuple(x.shape), gamma.numpy(), beta.numpy())))
    b = O.backward(dy, x, G, gamma, eps=eps, beta=beta, relu=relu)
    band = P.ReluBand(x, dy, G, gamma, beta, b["mean"], b["rstd"]) if relu else None
    dx64 = b["dx"].reshape(-1)
    rep.update(P.check_dx(P.to_np(r["dx"]).reshape(-1), dx64, band=None if band is None else band.dx_terms(idx, dx64)))
    a_dy, a_dyx = O.channel_abs_sums(dy, x, G, b["mean"], b["rstd"], gamma=gamma, beta=beta, relu=relu)
    depth = depth_bound(x, G, nshards)
    rep.update(P.check_param("dgamma", P.to_np(r["dgamma"]), b["dgamma"], a_dyx, depth,
                             (0.0 if band is None else band.dgamma)
                             + P.stats_slack(b["mean"], b["rstd"], a_dy, b["dgamma"], x.shape[1])))
    rep.update(P.check_param("dbeta", P.to_np(r["dbeta"]), b["dbeta"], a_dy, depth,
                             0.0 if band is None else band.dbeta))
    say(f"{tag}: ok {rep}")


CASES = [
    workloads.custom(2, 32, 8, (24, 17, 19), torch.bfloat16, dist="unet", seed=81),
    workloads.custom(1, 16, 4, (33, 32, 33), torch.float32, dist="tiny", seed=82),
    workloads.custom(3, 12, 3, (9, 7, 5), torch.float16, dist="deep", seed=83),
]


@pytest.mark.parametrize("nshards", [1, 2, 3, 8])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_shards_match_the_whole_volume(case, nshards):
    say(f"{case.name}: {nshards} shards along D")
    inp = workloads.make(case, DEV)
    r = run_sharded(inp, nshards)
    check_ranks_agree(r)
    full_compare(inp, r, f"{case.name}_p{nshards}", nshards)


def test_shards_with_relu():
    case = CASES[0]
    say(f"{case.name}: 3 shards, relu")
    inp = workloads.make(case, DEV)
    r = run_sharded(inp, 3, relu=True)
    check_ranks_agree(r)
    full_compare(inp, r, f"{case.name}_p3_relu", 3, relu=True)


def test_shards_nan_and_inf_reach_the_whole_group():
    """A NaN in one shard makes its group NaN on every rank; +Inf (alone) gives mean +Inf."""
    case = workloads.custom(2, 8, 4, (12, 6, 6), torch.float32, dist="unet", seed=84)
    inp = workloads.make(case, "cpu")
    x = inp["x"].clone()
    x[0, 2, 10, 1, 1] = float("nan")       # last shard, group (0, 1)
    x[1, 7, 0, 0, 0] = float("inf")        # first shard, group (1, 3)
    inp["x"] = x
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    r = run_sharded(g, 4)
    check_ranks_agree(r)
    full_compare(inp, r, "nan_inf_p4", 4)


def test_top_site_in_eight_shards():
    """The 128^3, C=32, G=8 site split in 8 (16 planes a shard): statistics and parameter
    gradients in full against the oracle, y and dx on a sample."""
    case = workloads.SCALE7
    say(f"{case.name}: 8 shards")
    inp = workloads.make(case, DEV)
    r = run_sharded(inp, 8)
    check_ranks_agree(r)
    x, dy, G, eps = inp["x"].cpu(), inp["dy"].cpu(), inp["G"], inp["eps"]
    gamma, beta = inp["gamma"].cpu(), inp["beta"].cpu()
    mean64, var64, rstd64 = O.group_stats(x, G, eps)
    rep = P.check_stats(P.to_np(r["mean"]), P.to_np(r["rstd"]), mean64, var64, rstd64)
    rng = np.random.default_rng(85)
    idx = np.unique(np.concatenate([rng.integers(0, x.numel(), 1 << 18), np.arange(0, x.numel(), 128 * 128 * 16)]))
    it = torch.from_numpy(idx).to(DEV)
    y64 = O.forward_at(x, G, idx, mean64, rstd64, gamma, beta)
    rep.update(P.check_y(P.to_np(r["y"].reshape(-1)[it]), y64,
                         *P.channel_params_at(idx, tuple(x.shape), gamma.numpy(), beta.numpy())))
    b = O.backward(dy, x, G, gamma, eps=eps, want_dx=False)
    dx64 = O.backward_at(dy, x, G, idx, b["mean"], b["rstd"], b["c1"], b["c2"], gamma)
    rep.update(P.check_dx(P.to_np(r["dx"].reshape(-1)[it]), dx64))
    a_dy, a_dyx = O.channel_abs_sums(dy, x, G, b["mean"], b["rstd"])
    depth = depth_bound(x, G, 8)
    rep.update(P.check_param("dgamma", P.to_np(r["dgamma"]), b["dgamma"], a_dyx, depth,
                             P.stats_slack(b["mean"], b["rstd"], a_dy, b["dgamma"], x.shape[1])))
    rep.update(P.check_param("dbeta", P.to_np(r["dbeta"]), b["dbeta"], a_dy, depth))
    say(f"{case.name}_p8: ok {rep}")


def test_one_voxel_shards_of_single_channel_groups():
    """Groups of one channel (C/G = 1) split into one-voxel shards: each shard's piece of a
    group is a single element, but the group is not; dx must be the whole group's, not the
    exact zero that a single-element group gets."""
    case = workloads.custom(2, 4, 4, (3, 1, 1), torch.float32, dist="unet", seed=86)
    say(f"{case.name}: 3 one-voxel shards, C/G = 1")
    inp = workloads.make(case, DEV)
    r = run_sharded(inp, 3)
    check_ranks_agree(r)
    assert torch.count_nonzero(r["dx"]) > 0
    full_compare(inp, r, "one_voxel_shards_p3", 3)
