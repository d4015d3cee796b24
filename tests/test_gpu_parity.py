"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Small and ragged shapes are compared element by element; the 128^3 / 256^3 sites and
the > 2^31-element volume are compared on every statistic and parameter gradient and
on a sample of y and dx (random elements plus the edges of jobs), at the plan and
launch configuration the benchmark times. Tolerances are documented in tests/parity.py.
"""
import math

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
    print(f"[gpu-parity] {msg}", flush=True)


def _on_gpu(inp):
    out = dict(inp)
    for k in ("x", "gamma", "beta", "dy"):
        if out[k] is not None:
            out[k] = out[k].to(DEV)
    return out


def _run(inp, out_dtype=None, dy=None, relu=False, layout=None):
    x, G, eps = inp["x"], inp["G"], inp["eps"]
    act = "relu" if relu else None
    y, mean, rstd = gn.gn_forward(x, inp["gamma"], inp["beta"], G, eps, out_dtype or inp["out_dtype"],
                                  activation=act, layout=layout)
    dy = inp["dy"] if dy is None else dy
    dx, dg, db = gn.gn_backward(dy, x, mean, rstd, inp["gamma"], G, beta=inp["beta"], activation=act,
                                layout=layout)
    torch.cuda.synchronize()
    return {"y": y, "mean": mean, "rstd": rstd, "dx": dx, "dgamma": dg, "dbeta": db}


def _run_layout(inp, relu, layout):
    """Runs the GPU path with x and dy in `layout`; returns outputs as contiguous NCDHW."""
    if layout == "ndhwc":
        inp = dict(inp)
        inp["x"] = gn.as_layout(inp["x"], "ndhwc")
        inp["dy"] = gn.as_layout(inp["dy"], "ndhwc")
    r = _run(inp, relu=relu, layout=layout)
    if layout == "ndhwc":
        assert r["y"].stride() == inp["x"].stride() and r["dx"].stride() == inp["x"].stride()
        r["y"], r["dx"] = r["y"].contiguous(), r["dx"].contiguous()
    return r


def _chan_at(idx, x, gamma, beta):
    return P.channel_params_at(idx, tuple(x.shape), gamma.cpu().numpy(), beta.cpu().numpy())


def full_check(inp, tag, relu=False, layout="ncdhw"):
    """Element-by-element comparison of every output."""
    say(f"{tag}: shape {tuple(inp['x'].shape)} x {inp['x'].dtype} dy {inp['dy'].dtype} "
        f"out {inp['out_dtype']} G={inp['G']} relu={relu} {layout} -> gn_forward + gn_backward")
    g = _on_gpu(inp)
    r = _run_layout(g, relu, layout)
    x, dy, G, eps = inp["x"].cpu(), inp["dy"].cpu(), inp["G"], inp["eps"]
    gamma, beta = inp["gamma"].cpu(), inp["beta"].cpu()
    f = O.forward(x, G, gamma, beta, eps=eps, relu=relu)
    rep = P.check_stats(P.to_np(r["mean"]), P.to_np(r["rstd"]), f["mean"], f["var"], f["rstd"])
    idx = np.arange(x.numel())
    rep.update(P.check_y(P.to_np(r["y"]).reshape(-1), f["y"].reshape(-1), *_chan_at(idx, x, gamma, beta)))
    b = O.backward(dy, x, G, gamma, eps=eps, beta=beta, relu=relu)
    dx64 = b["dx"].reshape(-1)
    band = P.ReluBand(x, dy, G, gamma, beta, b["mean"], b["rstd"]) if relu else None
    rep.update(P.check_dx(P.to_np(r["dx"]).reshape(-1), dx64,
                          band=None if band is None else band.dx_terms(idx, dx64)))
    a_dy, a_dyx = O.channel_abs_sums(dy, x, G, b["mean"], b["rstd"], gamma=gamma, beta=beta, relu=relu)
    N, C = x.shape[:2]
    depth = P.reduction_depth(gn.gn_plan_query(N, C, x.numel() // (N * C), G), N)
    rep.update(P.check_param("dgamma", P.to_np(r["dgamma"]), b["dgamma"], a_dyx, depth,
                             (0.0 if band is None else band.dgamma)
                             + P.stats_slack(b["mean"], b["rstd"], a_dy, b["dgamma"], x.shape[1])))
    rep.update(P.check_param("dbeta", P.to_np(r["dbeta"]), b["dbeta"], a_dy, depth,
                             0.0 if band is None else band.dbeta))
    say(f"{tag}: ok {rep}")
    return r


def _sample_indices(x, G, n_random, seed):
    N, C = x.shape[:2]
    S = x.numel() // (N * C)
    plan = gn.gn_plan_query(N, C, S, G)
    rng = np.random.default_rng(seed)
    parts = [rng.integers(0, x.numel(), n_random)]
    # edges of up to 512 jobs: first and last 64 elements of each
    K, chunk = plan["chunks_per_row"], plan["chunk"]
    jobs = rng.choice(plan["jobs"], min(512, plan["jobs"]), replace=False)
    for j in jobs:
        row, k = divmod(int(j), K)
        lo, hi = row * S + k * chunk, row * S + min((k + 1) * chunk, S)
        parts.append(np.arange(lo, min(lo + 64, hi)))
        parts.append(np.arange(max(hi - 64, lo), hi))
    parts.append(np.array([0, x.numel() - 1]))
    return np.unique(np.concatenate(parts)).astype(np.int64)


def sampled_check(inp, tag, n_random=1 << 20, seed=0, relu=False, layout="ncdhw"):
    """Full statistics and parameter gradients; y and dx on sampled elements."""
    say(f"{tag}: shape {tuple(inp['x'].shape)} x {inp['x'].dtype} G={inp['G']} relu={relu} {layout} "
        f"(sampled) -> gn_forward + gn_backward")
    r = _run_layout(inp, relu, layout)
    x, dy, G, eps = inp["x"].cpu(), inp["dy"].cpu(), inp["G"], inp["eps"]
    gamma, beta = inp["gamma"].cpu(), inp["beta"].cpu()
    say(f"{tag}: oracle statistics")
    mean64, var64, rstd64 = O.group_stats(x, G, eps)
    rep = P.check_stats(P.to_np(r["mean"]), P.to_np(r["rstd"]), mean64, var64, rstd64)
    idx = _sample_indices(x, G, n_random, seed)
    it = torch.from_numpy(idx).to(DEV)
    y64 = O.forward_at(x, G, idx, mean64, rstd64, gamma, beta, relu=relu)
    rep.update(P.check_y(P.to_np(r["y"].reshape(-1)[it]), y64, *_chan_at(idx, x, gamma, beta)))
    say(f"{tag}: oracle backward")
    b = O.backward(dy, x, G, gamma, eps=eps, want_dx=False, beta=beta, relu=relu)
    dx64 = O.backward_at(dy, x, G, idx, b["mean"], b["rstd"], b["c1"], b["c2"], gamma, beta=beta, relu=relu)
    band = P.ReluBand(x, dy, G, gamma, beta, b["mean"], b["rstd"]) if relu else None
    rep.update(P.check_dx(P.to_np(r["dx"].reshape(-1)[it]), dx64,
                          band=None if band is None else band.dx_terms(idx, dx64)))
    a_dy, a_dyx = O.channel_abs_sums(dy, x, G, b["mean"], b["rstd"], gamma=gamma, beta=beta, relu=relu)
    N, C = x.shape[:2]
    depth = P.reduction_depth(gn.gn_plan_query(N, C, x.numel() // (N * C), G), N)
    rep.update(P.check_param("dgamma", P.to_np(r["dgamma"]), b["dgamma"], a_dyx, depth,
                             (0.0 if band is None else band.dgamma)
                             + P.stats_slack(b["mean"], b["rstd"], a_dy, b["dgamma"], x.shape[1])))
    rep.update(P.check_param("dbeta", P.to_np(r["dbeta"]), b["dbeta"], a_dy, depth,
                             0.0 if band is None else band.dbeta))
    if band is not None:
        rep["band_total"] = band.count
    say(f"{tag}: ok ({idx.size} sampled elements) {rep}")
    r["report"] = rep
    return r


# ----------------------------------------------------------------------------- named workloads

@pytest.mark.parametrize("case", [workloads.TINY, workloads.DEEP, workloads.DEEP_F32OUT],
                         ids=lambda c: c.name)
def test_small_workloads_elementwise(case):
    full_check(workloads.make(case, "cpu"), case.name)


RAGGED = [
    workloads.custom(2, 6, 2, (5, 7, 3), torch.bfloat16, dist="unet", seed=11),
    workloads.custom(3, 12, 3, (17, 17, 17), torch.bfloat16, dist="normal", seed=12),
    workloads.custom(1, 4, 2, (40, 40, 41), torch.float32, dist="tiny", seed=13),
    workloads.custom(2, 8, 4, (33, 31, 29), torch.bfloat16, dist="deep", seed=14),
    workloads.custom(1, 2, 1, (3 * 8192 + 5,), torch.float32, dist="unet", seed=15),
    workloads.custom(5, 10, 5, (7, 7, 7), torch.bfloat16, dist="unet", seed=16, out_dtype=torch.float32),
    workloads.custom(2, 3, 3, (65537,), torch.float32, dist="normal", seed=17),
    workloads.custom(1, 16, 4, (64, 64, 65), torch.bfloat16, dist="unet", seed=18),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: c.name)
def test_ragged_shapes_elementwise(case):
    full_check(workloads.make(case, "cpu"), case.name)


CENSUS = workloads.census_cases()


@pytest.mark.parametrize("case,layout", [
    (workloads.custom(70000, 4, 2, (8,), torch.bfloat16, dist="unet", seed=19), "ncdhw"),
    (workloads.custom(70000, 8, 8, (2,), torch.bfloat16, dist="normal", seed=20), "ndhwc"),
], ids=lambda v: getattr(v, "name", str(v)))
def test_many_samples_past_the_grid_y_limit(case, layout):
    """More samples than a launch's y extent holds (65535): the plans leave the per-(n, g)
    grids of the resident path and run the flat-grid kernels; every element checked."""
    p = gn.gn_plan_query(case.N, case.C, case.S, case.G) if layout == "ncdhw" else \
        gn.gn_plan_query_cl(case.N, case.C, case.S, case.G)
    assert p["resident_forward"] == 0
    full_check(workloads.make(case, "cpu"), case.name + "_" + layout, layout=layout)


@pytest.mark.parametrize("case", CENSUS, ids=lambda c: c.name)
def test_census_sites(case):
    if case.numel <= (1 << 23):
        full_check(workloads.make(case, "cpu"), case.name)
    else:
        sampled_check(workloads.make(case, DEV), case.name, n_random=1 << 18, seed=case.seed)


@pytest.mark.parametrize("case", [workloads.SCALE7, workloads.SCALE8], ids=lambda c: c.name)
def test_unet_top_sites_sampled(case):
    sampled_check(workloads.make(case, DEV), case.name, seed=case.seed)


@pytest.mark.parametrize("case,layout", [(workloads.SCALE7_DY_OFFSET, "ncdhw"), (workloads.SCALE8_DY_OFFSET, "ncdhw"),
                                         (workloads.SCALE7_DY_OFFSET, "ndhwc")],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_param_gradients_hold_the_relative_bar_at_full_size(case, layout):
    """The 128^3 and 256^3 sites with a dy whose channel sums do not cancel: every channel's
    dgamma and dbeta within 1e-4 of the oracle's, with no summation floor (every channel is
    well conditioned, which the report confirms), at the plan and launch configuration the
    benchmark times."""
    r = sampled_check(workloads.make(case, DEV), f"{case.name}_{layout}", n_random=1 << 18, seed=case.seed,
                      layout=layout)
    rep = r["report"]
    for name in ("dgamma", "dbeta"):
        assert rep[f"{name}_well_conditioned"] == case.C, rep
        assert rep[f"{name}_max_rel_err"] <= 1e-4, rep


# ----------------------------------------------------------------------------- closed forms on the GPU

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape,G", [((2, 6, 9, 10, 11), 3), ((1, 32, 128, 128, 128), 8),
                                     ((2, 8, 8, 8, 8), 4)])
def test_constant_input_gives_beta_bitwise(dtype, shape, G):
    say(f"constant input {shape} {dtype}")
    N, C = shape[:2]
    # one constant per group (n, g), shared by the group's C/G channels
    consts = torch.linspace(-3.0, 100.0, N * G).view(N, G, 1).expand(N, G, C // G).reshape(N, C)
    x = consts.view(N, C, *([1] * (len(shape) - 2))).expand(shape).to(dtype).contiguous().to(DEV)
    beta = torch.linspace(-0.5, 0.5, C, device=DEV)
    gamma = torch.linspace(0.5, 1.5, C, device=DEV)
    y, mean, rstd = gn.gn_forward(x, gamma, beta, G, 1e-5)
    torch.cuda.synchronize()
    expect = beta.view(1, C, *([1] * (len(shape) - 2))).expand(shape).to(dtype)
    assert torch.equal(y, expect)
    assert torch.all(rstd == rstd.flatten()[0]).item()
    assert abs(rstd.flatten()[0].item() - 1 / math.sqrt(np.float32(1e-5))) <= 1e-5 * 316.3


def test_single_element_groups():
    say("single-element groups (2, 4, 1, 1, 1), G=4")
    rng = np.random.default_rng(3)
    x = torch.tensor(rng.normal(size=(2, 4, 1, 1, 1)), dtype=torch.float32, device=DEV)
    dy = torch.tensor(rng.normal(size=(2, 4, 1, 1, 1)), dtype=torch.float32, device=DEV)
    gamma = torch.tensor([1.1, 0.9, 1.3, 0.7], device=DEV)
    beta = torch.tensor([0.1, -0.2, 0.3, -0.4], device=DEV)
    y, mean, rstd = gn.gn_forward(x, gamma, beta, 4, 1e-5)
    dx, dg, db = gn.gn_backward(dy, x, mean, rstd, gamma, 4)
    torch.cuda.synchronize()
    assert torch.equal(y, beta.view(1, 4, 1, 1, 1).expand(2, 4, 1, 1, 1))
    assert torch.equal(mean, x.view(2, 4))
    assert torch.equal(dx.view(torch.int32), torch.zeros_like(dx).view(torch.int32))  # +0 exactly
    assert torch.equal(dg, torch.zeros_like(dg))
    assert torch.allclose(db, dy.sum(dim=(0, 2, 3, 4)), rtol=1e-6, atol=0)
    ref = 1 / math.sqrt(float(np.float32(1e-5)))
    assert torch.all((rstd - ref).abs() <= 1e-5 * ref).item()


def test_nan_and_inf_confined_to_their_group():
    say("NaN/Inf in two groups of (2, 8, 6, 6, 6), G=4")
    inp = workloads.make(workloads.custom(2, 8, 4, (6, 6, 6), torch.bfloat16, seed=21), "cpu")
    x = inp["x"].clone()
    x[0, 2, 1, 1, 1] = float("nan")
    x[1, 7, 0, 0, 0] = float("inf")
    inp["x"] = x
    full_check(inp, "nan_inf")


@pytest.mark.parametrize("spatial", [(32, 32, 32), (16, 16, 16)])
def test_large_mean_offset_keeps_variance(spatial):
    """fp32 input at mu/sigma = 1e5, where E[x^2] - E[x]^2 loses the variance (two-pass
    kernels at 32^3, the resident path at 16^3)."""
    say(f"mu/sigma = 1e5, fp32, (1, 4, {spatial}), G=2")
    rng = np.random.default_rng(7)
    x = (1e5 + rng.normal(size=(1, 4) + spatial)).astype(np.float32)
    xt = torch.from_numpy(x).to(DEV)
    y, mean, rstd = gn.gn_forward(xt, None, None, 2, 1e-5)
    torch.cuda.synchronize()
    f = O.forward(x, 2, eps=1e-5)
    P.check_stats(P.to_np(mean), P.to_np(rstd), f["mean"], f["var"], f["rstd"])
    P.check_y(P.to_np(y).reshape(-1), f["y"].reshape(-1), *P.channel_params_at(np.arange(x.size), x.shape, None, None))


@pytest.mark.parametrize("spatial", [(20, 18, 17), (16, 16, 16)])
def test_eps_zero(spatial):
    """eps = 0 is a valid argument: with spread in every group the statistics are 1/sigma
    exactly as the definition has them, and a constant group (variance 0, rstd = inf) gives
    NaN in that group's y and dx and nowhere else, as the fp64 definition does (0 * inf).
    Two-pass kernels at the ragged shape, the resident path at 16^3."""
    say(f"eps = 0, (2, 8, {spatial}), G=4, one constant group")
    inp = workloads.make(workloads.custom(2, 8, 4, spatial, torch.float32, dist="unet", seed=23), "cpu")
    inp["eps"] = 0.0
    x = inp["x"].clone()
    x[1, 2:4] = 0.75                     # group (1, 1): constant
    inp["x"] = x
    r = full_check(inp, "eps0")
    assert torch.isnan(r["y"][1, 2:4]).all() and not torch.isnan(r["y"][0]).any()
    assert torch.isnan(r["dx"][1, 2:4]).all() and not torch.isnan(r["dx"][1, 4:]).any()


@pytest.mark.parametrize("scale", [1e-12, 1e12])
def test_extreme_magnitudes(scale):
    """Values of 1e-12 and 1e12 times the usual spread, around offsets ten times the spread,
    fp32 throughout: every result stays within its relative bar (the statistics carry the
    scale through the shift and the head/tail mean). The group's sum of squared deviations
    is kept in fp32, so a group whose M * variance passes the fp32 range is out of the
    domain (M * sigma^2 < 3.4e38)."""
    say(f"fp32 input scaled by {scale:g}, (2, 16, 12, 11, 10), G=4")
    inp = workloads.make(workloads.custom(2, 16, 4, (12, 11, 10), torch.float32, dist="unet", seed=29), "cpu")
    inp["x"] = ((inp["x"].double() * scale) + 10 * scale).float()
    full_check(inp, f"scale_{scale:g}")


# ----------------------------------------------------------------------------- bitwise properties

@pytest.mark.parametrize("case", [workloads.DEEP, workloads.SCALE7], ids=lambda c: c.name)
def test_bf16_output_is_fp32_output_rounded_once(case):
    say(f"{case.name}: bf16 output vs fp32 output rounded once")
    inp = workloads.make(case, DEV, with_dy=False)
    x, G = inp["x"], inp["G"]
    y16, m16, r16 = gn.gn_forward(x, inp["gamma"], inp["beta"], G, inp["eps"], torch.bfloat16)
    y32, m32, r32 = gn.gn_forward(x, inp["gamma"], inp["beta"], G, inp["eps"], torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(m16, m32) and torch.equal(r16, r32)
    # fp32 -> bf16 round-to-nearest-even on the host (via fp64, exact for fp32 values)
    ref = O.round_bf16(y32.cpu().numpy().astype(np.float64).reshape(-1))
    got = P.to_np(y16).reshape(-1)
    nan = np.isnan(y32.cpu().numpy().reshape(-1))
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("case", [workloads.DEEP, workloads.SCALE7], ids=lambda c: c.name)
def test_dy_dtype_does_not_change_a_bit(case):
    say(f"{case.name}: dy bf16 vs the same values in fp32")
    inp = workloads.make(case, DEV)
    x, G = inp["x"], inp["G"]
    y, mean, rstd = gn.gn_forward(x, inp["gamma"], inp["beta"], G, inp["eps"])
    a = gn.gn_backward(inp["dy"], x, mean, rstd, inp["gamma"], G)
    b = gn.gn_backward(inp["dy"].float(), x, mean, rstd, inp["gamma"], G)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u.view(torch.int32),
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v.view(torch.int32))


@pytest.mark.parametrize("case", [workloads.SCALE7, workloads.DEEP], ids=lambda c: c.name)
def test_repeats_are_bitwise_identical_with_poisoned_workspace(case):
    say(f"{case.name}: 10 repeats, workspace poisoned with NaN before every call")
    inp = workloads.make(case, DEV)
    x, G = inp["x"], inp["G"]
    ws = gn.workspace_for(x, G)
    first = None
    for i in range(10):
        ws.view(torch.float32).fill_(float("nan"))
        y, mean, rstd = gn.gn_forward(x, inp["gamma"], inp["beta"], G, inp["eps"], workspace=ws)
        ws.view(torch.float32).fill_(float("nan"))
        dx, dg, db = gn.gn_backward(inp["dy"], x, mean, rstd, inp["gamma"], G, workspace=ws)
        torch.cuda.synchronize()
        outs = [t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
                for t in (y, mean, rstd, dx, dg, db)]
        if first is None:
            first = outs
        else:
            for u, v in zip(outs, first):
                assert torch.equal(u, v), f"repeat {i} differs"


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


def test_one_workspace_across_shapes():
    """One workspace, sized for the largest shape and poisoned with NaN before every call,
    serves fwd/bwd, relu and dx-only calls of several shapes (two-pass and resident);
    every output equals the one computed with a workspace of its own."""
    cases = [workloads.SCALE7, workloads.DEEP, RAGGED[3], RAGGED[1], workloads.TINY]
    big = max(gn.gn_workspace_bytes(c.N, c.C, c.numel // (c.N * c.C), c.G) for c in cases)
    shared = torch.empty(big, dtype=torch.uint8, device=DEV)
    for case in cases:
        say(f"shared workspace: {case.name}")
        inp = workloads.make(case, DEV)
        x, G, gamma, beta, dy = inp["x"], inp["G"], inp["gamma"], inp["beta"], inp["dy"]
        for act in (None, "relu"):
            ref_f = gn.gn_forward(x, gamma, beta, G, inp["eps"], activation=act)
            ref_b = gn.gn_backward(dy, x, ref_f[1], ref_f[2], gamma, G, beta=beta, activation=act)
            shared.fill_(0xFF)
            got_f = gn.gn_forward(x, gamma, beta, G, inp["eps"], activation=act, workspace=shared)
            shared.fill_(0xFF)
            got_b = gn.gn_backward(dy, x, got_f[1], got_f[2], gamma, G, beta=beta, activation=act,
                                   workspace=shared)
            shared.fill_(0xFF)
            dx_only = gn.gn_backward(dy, x, got_f[1], got_f[2], gamma, G, beta=beta, activation=act,
                                     need_dgamma=False, need_dbeta=False, workspace=shared)[0]
            torch.cuda.synchronize()
            for u, v in zip(ref_f + ref_b, got_f + got_b):
                assert torch.equal(_bits(u), _bits(v))
            assert torch.equal(_bits(dx_only), _bits(ref_b[0]))


SPLIT_CASES = [
    workloads.SCALE7, workloads.DEEP,
    # ragged rows (S not a multiple of 8) split into several folded jobs with edge steps
    workloads.custom(2, 24, 6, (33, 31, 29), torch.bfloat16, dist="unet", seed=71),
    workloads.custom(3, 12, 3, (40, 41, 37), torch.float16, torch.float32, dist="deep", seed=72),
    workloads.custom(1, 16, 4, (50, 60, 70), torch.float32, dist="normal", seed=73),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: c.name)
def test_split_phase_entry_points_match_fused(case):
    say(f"{case.name}: split-phase entry points vs gn_forward/gn_backward")
    inp = workloads.make(case, DEV)
    x, G, gamma, beta = inp["x"], inp["G"], inp["gamma"], inp["beta"]
    y, mean, rstd = gn.gn_forward(x, gamma, beta, G, inp["eps"])
    dx, dg, db = gn.gn_backward(inp["dy"], x, mean, rstd, gamma, G)
    ws = gn.workspace_for(x, G)
    y2, mean2, rstd2 = torch.empty_like(y), torch.empty_like(mean), torch.empty_like(rstd)
    gn.gn_forward_stats(x, gamma, beta, G, inp["eps"], mean2, rstd2, ws)
    gn.gn_forward_apply(x, G, y2, ws)
    dx2, dg2, db2 = torch.empty_like(dx), torch.empty_like(dg), torch.empty_like(db)
    gn.gn_backward_reduce(inp["dy"], x, mean2, rstd2, gamma, G, dg2, db2, ws)
    gn.gn_backward_apply(inp["dy"], x, G, dx2, ws)
    torch.cuda.synchronize()
    for u, v in ((y, y2), (mean, mean2), (rstd, rstd2), (dx, dx2), (dg, dg2), (db, db2)):
        assert torch.equal(u, v)
    say(f"{case.name}: the two-call halves of gn_forward/gn_backward vs the fused calls")
    ws.fill_(0xFF)
    gn.gn_forward_partials(x, G, ws)
    gn.gn_forward_finish(x, gamma, beta, G, inp["eps"], y2, mean2, rstd2, ws)
    gn.gn_backward_partials(inp["dy"], x, mean2, rstd2, gamma, G, ws)
    gn.gn_backward_finish(inp["dy"], x, mean2, rstd2, gamma, G, dx2, dg2, db2, ws)
    torch.cuda.synchronize()
    for u, v in ((y, y2), (mean, mean2), (rstd, rstd2), (dx, dx2), (dg, dg2), (db, db2)):
        assert torch.equal(u, v)
    say(f"{case.name}: split-phase entry points with relu vs fused")
    y, mean, rstd = gn.gn_forward(x, gamma, beta, G, inp["eps"], activation="relu")
    dx, dg, db = gn.gn_backward(inp["dy"], x, mean, rstd, gamma, G, beta=beta, activation="relu")
    gn.gn_forward_stats(x, gamma, beta, G, inp["eps"], mean2, rstd2, ws)
    gn.gn_forward_apply(x, G, y2, ws, activation="relu")
    gn.gn_backward_reduce(inp["dy"], x, mean2, rstd2, gamma, G, dg2, db2, ws, beta=beta, activation="relu")
    gn.gn_backward_apply(inp["dy"], x, G, dx2, ws, activation="relu")
    torch.cuda.synchronize()
    for u, v in ((y, y2), (mean, mean2), (rstd, rstd2), (dx, dx2), (dg, dg2), (db, db2)):
        assert torch.equal(u, v)


FOLD_ORDER_CASES = [
    workloads.SCALE7,                                                                        # 32 folded jobs a reduction job
    workloads.custom(1, 32, 8, (64, 64, 64), torch.bfloat16, dist="unet", seed=95),          # 2
    workloads.custom(1, 48, 8, (64, 64, 64), torch.bfloat16, dist="unet", seed=97),          # 2, 768 of them
    workloads.custom(1, 32, 8, (61, 64, 64), torch.float16, dist="normal", seed=96),         # short last job: index order
]


@pytest.mark.parametrize("case", FOLD_ORDER_CASES, ids=lambda c: c.name)
def test_folded_jobs_in_tail_first_order_write_every_element(case):
    """Where each reduction job is a whole number of folded jobs, the folded kernels take their
    jobs in a permuted order (the last folded job of every reduction job first), and the
    split-phase one-step kernels likewise over their own jobs. Every element of y and dx
    must still be written once: both paths' outputs start as NaN and must come out finite
    and bitwise equal to each other."""
    inp = workloads.make(case, DEV)
    x, G, gamma, beta, dy = inp["x"], inp["G"], inp["gamma"], inp["beta"], inp["dy"]
    N, C = x.shape[:2]
    S = x.numel() // (N * C)
    p = gn.gn_plan_query(N, C, S, G)
    nested = p["chunk"] % p["fold_chunk"] == 0 and \
        p["fold_chunks_per_row"] == p["chunks_per_row"] * (p["chunk"] // p["fold_chunk"])
    F = p["chunk"] // p["fold_chunk"] if nested else 1
    say(f"{case.name}: {F} folded jobs a reduction job, fused outputs poisoned with NaN")
    if case is not FOLD_ORDER_CASES[-1]:
        assert F > 1
    y = torch.full_like(x, float("nan"))
    dx = torch.full_like(x, float("nan"))
    mean = torch.full((N, G), float("nan"), device=DEV)
    rstd = torch.full((N, G), float("nan"), device=DEV)
    gn.gn_forward(x, gamma, beta, G, inp["eps"], out=y, mean=mean, rstd=rstd)
    gn.gn_backward(dy, x, mean, rstd, gamma, G, dx=dx)
    ws = gn.workspace_for(x, G)
    y2, dx2 = torch.full_like(y, float("nan")), torch.full_like(dx, float("nan"))
    mean2, rstd2 = torch.empty_like(mean), torch.empty_like(rstd)
    dg2, db2 = torch.empty(C, device=DEV), torch.empty(C, device=DEV)
    gn.gn_forward_stats(x, gamma, beta, G, inp["eps"], mean2, rstd2, ws)
    gn.gn_forward_apply(x, G, y2, ws)
    gn.gn_backward_reduce(dy, x, mean2, rstd2, gamma, G, dg2, db2, ws)
    gn.gn_backward_apply(dy, x, G, dx2, ws)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any() and not torch.isnan(dx).any()
    assert not torch.isnan(y2).any() and not torch.isnan(dx2).any()
    for u, v in ((y, y2), (mean, mean2), (rstd, rstd2), (dx, dx2)):
        assert torch.equal(_bits(u), _bits(v))


@pytest.mark.parametrize("shape", [(2, 64, 8, (16, 16, 20)), (1, 32, 8, (32, 32, 32))], ids=str)
def test_channels_last_streaming_jobs_in_tail_first_order_write_every_element(shape):
    """The channels-last normalize and dx kernels take their jobs in the same tail-first
    order where the streaming jobs nest in the reduction jobs (80 and 128 reduction jobs of
    2 streaming jobs here, through the multiply-shift and the shift forms of the map):
    outputs poisoned with NaN come out finite and bitwise equal to a second call's."""
    N, C, G, sp = shape
    case = workloads.custom(N, C, G, sp, torch.bfloat16, dist="unet", seed=98)
    inp = workloads.make(case, DEV)
    x, dy = gn.as_layout(inp["x"], "ndhwc"), gn.as_layout(inp["dy"], "ndhwc")
    p = gn.gn_plan_query_cl(N, C, x.numel() // (N * C), G)
    assert p["chunk"] == 2 * p["apply_chunk"] and p["apply_jobs_per_sample"] == 2 * p["jobs_per_sample"]
    assert not p["resident_forward"] and not p["resident_backward"]
    say(f"channels-last {shape}: {p['jobs']} reduction jobs of 2 streaming jobs, outputs poisoned with NaN")
    y = torch.full_like(x, float("nan"))
    dx = torch.full_like(x, float("nan"))
    y, mean, rstd = gn.gn_forward(x, inp["gamma"], inp["beta"], G, inp["eps"], out=y)
    dx = gn.gn_backward(dy, x, mean, rstd, inp["gamma"], G, dx=dx)[0]
    y2, mean2, rstd2 = gn.gn_forward(x, inp["gamma"], inp["beta"], G, inp["eps"])
    dx2 = gn.gn_backward(dy, x, mean2, rstd2, inp["gamma"], G)[0]
    torch.cuda.synchronize()
    assert not torch.isnan(y).any() and not torch.isnan(dx).any()
    assert torch.equal(_bits(y), _bits(y2)) and torch.equal(_bits(dx), _bits(dx2))


def test_optional_backward_outputs():
    case = workloads.DEEP
    say(f"{case.name}: backward with dx only, and with dgamma/dbeta only")
    inp = workloads.make(case, DEV)
    x, G, gamma = inp["x"], inp["G"], inp["gamma"]
    y, mean, rstd = gn.gn_forward(x, gamma, inp["beta"], G, inp["eps"])
    dx, dg, db = gn.gn_backward(inp["dy"], x, mean, rstd, gamma, G)
    dx_only, n1, n2 = gn.gn_backward(inp["dy"], x, mean, rstd, gamma, G, need_dgamma=False, need_dbeta=False)
    n3, dg_only, db_only = gn.gn_backward(inp["dy"], x, mean, rstd, gamma, G, need_dx=False)
    torch.cuda.synchronize()
    assert n1 is None and n2 is None and n3 is None
    assert torch.equal(dx, dx_only) and torch.equal(dg, dg_only) and torch.equal(db, db_only)


def test_autograd_function_matches_entry_points():
    say("GroupNormFn through autograd vs entry points (deep workload)")
    inp = workloads.make(workloads.DEEP, DEV)
    x = inp["x"].clone().requires_grad_(True)
    gamma = inp["gamma"].clone().requires_grad_(True)
    beta = inp["beta"].clone().requires_grad_(True)
    y, mean, rstd = gn.GroupNormFn.apply(x, gamma, beta, inp["G"], inp["eps"], None)
    assert not mean.requires_grad and not rstd.requires_grad
    y.backward(inp["dy"])
    y2, m2, r2 = gn.gn_forward(inp["x"], inp["gamma"], inp["beta"], inp["G"], inp["eps"])
    dx2, dg2, db2 = gn.gn_backward(inp["dy"], inp["x"], m2, r2, inp["gamma"], inp["G"])
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), y2) and torch.equal(x.grad, dx2)
    assert torch.equal(gamma.grad, dg2) and torch.equal(beta.grad, db2)


def test_autograd_relu_matches_entry_points():
    say("group_norm(activation='relu') through autograd vs entry points (deep workload)")
    inp = workloads.make(workloads.DEEP, DEV)
    x = inp["x"].clone().requires_grad_(True)
    gamma = inp["gamma"].clone().requires_grad_(True)
    beta = inp["beta"].clone().requires_grad_(True)
    y = gn.group_norm(x, inp["G"], gamma, beta, inp["eps"], activation="relu")
    y.backward(inp["dy"])
    y2, m2, r2 = gn.gn_forward(inp["x"], inp["gamma"], inp["beta"], inp["G"], inp["eps"], activation="relu")
    dx2, dg2, db2 = gn.gn_backward(inp["dy"], inp["x"], m2, r2, inp["gamma"], inp["G"],
                                   beta=inp["beta"], activation="relu")
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), y2) and torch.equal(x.grad, dx2)
    assert torch.equal(gamma.grad, dg2) and torch.equal(beta.grad, db2)


def test_binding_rejects_bad_arguments():
    say("argument errors")
    x = torch.zeros((0, 4, 2, 2, 2), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gn.GnError, match="GN_ERR_SHAPE"):
        gn.gn_forward(x, None, None, 2)
    x = torch.zeros((1, 6, 2, 2, 2), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gn.GnError, match="GN_ERR_GROUPS"):
        gn.gn_forward(x, None, None, 4)
    x = torch.zeros((1, 4, 1, 1, 1), dtype=torch.float32, device=DEV)
    with pytest.raises(gn.GnError, match="GN_ERR_SHAPE"):
        gn.gn_forward(x, None, None, 4)
    x = torch.zeros((1, 4, 8, 8, 8), dtype=torch.float32, device=DEV)
    with pytest.raises(gn.GnError, match="GN_ERR_EPS"):
        gn.gn_forward(x, None, None, 2, eps=-1.0)
    with pytest.raises(gn.GnError, match="GN_ERR_DTYPE"):
        gn.gn_forward(x, None, None, 2, out_dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gn.gn_forward(x.transpose(2, 3), None, None, 2)
    with pytest.raises(ValueError, match="activation"):
        gn.gn_forward(x, None, None, 2, activation="gelu")
    # every tensor in pinned host memory: the binding's checks pass, the library refuses
    with pytest.raises(gn.GnError, match="GN_ERR_DEVICE"):
        gn.gn_forward(x.cpu().pin_memory(), None, None, 2, out=torch.empty_like(x, device="cpu").pin_memory(),
                      mean=torch.empty(1, 2).pin_memory(), rstd=torch.empty(1, 2).pin_memory(),
                      workspace=gn.workspace_for(x, 2).cpu().pin_memory())
    # outputs on another device than x: the binding refuses before the library is called
    with pytest.raises(ValueError, match="device"):
        gn.gn_forward(x.cpu().pin_memory(), None, None, 2, out=torch.empty_like(x),
                      mean=torch.empty(1, 2, device=DEV), rstd=torch.empty(1, 2, device=DEV),
                      workspace=gn.workspace_for(x, 2))


# ----------------------------------------------------------------------------- fp16 input

F16 = torch.float16
FP16_CASES = [
    workloads.custom(2, 8, 4, (6, 7, 5), F16, dist="unet", seed=51),                      # two-pass, ragged
    workloads.custom(1, 16, 4, (16, 16, 16), F16, dist="unet", seed=52),                  # resident
    workloads.custom(2, 6, 2, (33, 17, 9), F16, dist="deep", seed=53, out_dtype=torch.float32),
    workloads.custom(3, 12, 4, (4, 4, 6), F16, torch.bfloat16, dist="normal", seed=54),   # bf16 dy
    workloads.custom(1, 4, 2, (64, 64, 65), F16, torch.float32, dist="tiny", seed=56),    # fp32 dy, multi-job rows
]


@pytest.mark.parametrize("case", FP16_CASES, ids=lambda c: c.name + "_" + str(c.dy_dtype).split(".")[-1])
def test_fp16_elementwise(case):
    full_check(workloads.make(case, "cpu"), case.name + "_fp16")


@pytest.mark.parametrize("case", FP16_CASES[:2], ids=lambda c: c.name)
def test_fp16_relu_elementwise(case):
    full_check(workloads.make(case, "cpu"), case.name + "_fp16_relu", relu=True)


FP16_SCALE7 = workloads.custom(1, 32, 8, (128, 128, 128), F16, dist="unet", seed=55)


def test_fp16_top_site_sampled():
    sampled_check(workloads.make(FP16_SCALE7, DEV), "fp16_128cube", n_random=1 << 18, seed=55)


@pytest.mark.parametrize("case", [FP16_CASES[0], FP16_CASES[1], FP16_SCALE7], ids=lambda c: c.name)
def test_fp16_output_is_fp32_output_rounded_once(case):
    say(f"{case.name}: fp16 output vs fp32 output rounded once")
    inp = workloads.make(case, DEV, with_dy=False)
    x, G = inp["x"], inp["G"]
    y16, m16, r16 = gn.gn_forward(x, inp["gamma"], inp["beta"], G, inp["eps"], torch.float16)
    y32, m32, r32 = gn.gn_forward(x, inp["gamma"], inp["beta"], G, inp["eps"], torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(m16, m32) and torch.equal(r16, r32)
    ref = O.round_f16(y32.cpu().numpy().astype(np.float64).reshape(-1))
    got = y16.cpu().numpy().reshape(-1).view(np.uint16)
    nan = np.isnan(y32.cpu().numpy().reshape(-1))
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("case", [FP16_CASES[0], FP16_CASES[1]], ids=lambda c: c.name)
def test_fp16_dy_and_fp32_dy_give_the_same_bits(case):
    say(f"{case.name}: dy fp16 vs the same values in fp32")
    inp = workloads.make(case, DEV)
    x, G = inp["x"], inp["G"]
    y, mean, rstd = gn.gn_forward(x, inp["gamma"], inp["beta"], G, inp["eps"])
    a = gn.gn_backward(inp["dy"], x, mean, rstd, inp["gamma"], G)
    b = gn.gn_backward(inp["dy"].float(), x, mean, rstd, inp["gamma"], G)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(_bits(u), _bits(v))


# ----------------------------------------------------------------------------- channels-last

CL_CASES = [
    workloads.custom(2, 32, 8, (6, 7, 5), torch.bfloat16, dist="unet", seed=61),           # C/G 4: 2 groups a vector
    workloads.custom(1, 64, 8, (16, 16, 17), torch.bfloat16, dist="normal", seed=62),      # C/G 8
    workloads.custom(3, 8, 8, (5, 5, 5), torch.float32, dist="tiny", seed=63),             # C/G 1: 8 groups a vector
    workloads.custom(2, 16, 1, (9, 9, 9), torch.bfloat16, dist="deep", seed=64, out_dtype=torch.float32),
    workloads.custom(1, 512, 32, (8, 8, 8), torch.bfloat16, dist="deep", seed=65),         # C/8 = 64
    workloads.custom(2, 1024, 16, (3, 4, 5), torch.float16, dist="normal", seed=66),       # C/8 = 128 > 64 lanes
    workloads.custom(1, 2048, 2048, (2, 2, 3), torch.bfloat16, dist="unet", seed=67),      # C/8 = 256, C/G 1
    workloads.custom(2, 32, 8, (4, 4, 4), torch.float16, torch.float32, dist="unet", seed=68),
    workloads.custom(2, 8, 8, (1, 1, 1), torch.float32, dist="normal", seed=69),           # M = 1
    workloads.custom(1, 16, 4, (40, 41, 42), torch.bfloat16, dist="unet", seed=70),        # many jobs, ragged
    workloads.custom(1, 128, 16, (9, 10, 11), torch.bfloat16, dist="unet", seed=91),       # C/8 = 16: two tree levels
]


@pytest.mark.parametrize("case", CL_CASES, ids=lambda c: c.name + "_" + str(c.x_dtype).split(".")[-1])
def test_channels_last_elementwise(case):
    full_check(workloads.make(case, "cpu"), case.name + "_cl", layout="ndhwc")


@pytest.mark.parametrize("case", CL_CASES[:3], ids=lambda c: c.name)
def test_channels_last_relu_elementwise(case):
    full_check(workloads.make(case, "cpu"), case.name + "_cl_relu", relu=True, layout="ndhwc")


def test_channels_last_nan_and_inf_confined_to_their_group():
    say("channels-last: NaN/Inf in two groups of (2, 32, 6, 6, 6), G=8")
    inp = workloads.make(workloads.custom(2, 32, 8, (6, 6, 6), torch.bfloat16, seed=71), "cpu")
    x = inp["x"].clone()
    x[0, 5, 1, 1, 1] = float("nan")
    x[1, 30, 0, 2, 0] = float("inf")
    inp["x"] = x
    full_check(inp, "nan_inf_cl", layout="ndhwc")


CL_RES_CASES = [  # (case, relu, resident forward, resident backward)
    (workloads.custom(1, 256, 32, (8, 8, 8), torch.bfloat16, dist="unet", seed=73), False, 1, 1),
    (workloads.custom(1, 256, 32, (16, 16, 16), torch.bfloat16, dist="unet", seed=80), False, 0, 0),
    (workloads.custom(1, 512, 32, (8, 8, 8), torch.bfloat16, dist="unet", seed=74), True, 1, 1),
    (workloads.custom(4, 512, 32, (8, 8, 8), torch.bfloat16, dist="deep", seed=75), False, 1, 0),
    (workloads.custom(2, 64, 8, (4, 4, 4), torch.float16, torch.float32, dist="normal", seed=76,
                      out_dtype=torch.float32), True, 1, 1),
    (workloads.custom(3, 128, 8, (2, 5, 1), torch.float32, dist="tiny", seed=77), False, 1, 0),
    (workloads.custom(2, 64, 1, (4, 4, 4), torch.bfloat16, dist="unet", seed=78), True, 1, 1),
]


@pytest.mark.parametrize("case,relu,rf,rb", CL_RES_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_channels_last_resident_elementwise(case, relu, rf, rb):
    """Groups of whole vectors small enough for one workgroup take the channels-last resident
    kernels (one launch a direction); every output element against the oracle."""
    p = gn.gn_plan_query_cl(case.N, case.C, case.S, case.G)
    assert (p["resident_forward"], p["resident_backward"]) == (rf, rb)
    full_check(workloads.make(case, "cpu"), case.name + "_cl_res", relu=relu, layout="ndhwc")


def test_channels_last_resident_nan_and_inf_confined_to_their_group():
    case = workloads.custom(2, 256, 32, (4, 4, 4), torch.bfloat16, seed=79)
    p = gn.gn_plan_query_cl(case.N, case.C, case.S, case.G)
    assert p["resident_forward"] == 1 and p["resident_backward"] == 1
    say("channels-last resident: NaN/Inf in two groups of (2, 256, 4, 4, 4), G=32")
    inp = workloads.make(case, "cpu")
    x = inp["x"].clone()
    x[0, 17, 1, 1, 1] = float("nan")
    x[1, 250, 0, 2, 3] = float("inf")
    inp["x"] = x
    full_check(inp, "nan_inf_cl_res", layout="ndhwc")


@pytest.mark.parametrize("case", [workloads.SCALE7], ids=lambda c: c.name)
def test_channels_last_top_site_sampled(case):
    sampled_check(workloads.make(case, DEV), case.name + "_cl", n_random=1 << 18, seed=case.seed, layout="ndhwc")


def test_channels_last_bitwise_properties():
    """bf16 output = fp32 output rounded once; bf16 and fp32 dy with the same values give
    the same bits; ten repeats are identical; constant input gives beta exactly."""
    case = workloads.custom(1, 64, 8, (32, 32, 32), torch.bfloat16, dist="unet", seed=72)
    say(f"channels-last bitwise properties on {case.name}")
    inp = workloads.make(case, DEV)
    x, G = gn.as_layout(inp["x"], "ndhwc"), inp["G"]
    dy = gn.as_layout(inp["dy"], "ndhwc")
    y16, m16, r16 = gn.gn_forward(x, inp["gamma"], inp["beta"], G, inp["eps"], torch.bfloat16)
    y32, m32, r32 = gn.gn_forward(x, inp["gamma"], inp["beta"], G, inp["eps"], torch.float32)
    a = gn.gn_backward(dy, x, m16, r16, inp["gamma"], G)
    b = gn.gn_backward(gn.as_layout(dy.float(), "ndhwc"), x, m16, r16, inp["gamma"], G)
    torch.cuda.synchronize()
    assert torch.equal(m16, m32) and torch.equal(r16, r32)
    ref = O.round_bf16(y32.contiguous().cpu().numpy().astype(np.float64).reshape(-1))
    assert np.array_equal(P.to_np(y16.contiguous()).reshape(-1), ref)
    for u, v in zip(a, b):
        assert torch.equal(_bits(u.contiguous()), _bits(v.contiguous()))
    for _ in range(9):
        c = gn.gn_backward(dy, x, m16, r16, inp["gamma"], G)
        y2, _, _ = gn.gn_forward(x, inp["gamma"], inp["beta"], G, inp["eps"], torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(_bits(y2), _bits(y16))
        for u, v in zip(a, c):
            assert torch.equal(_bits(u), _bits(v))
    const = torch.full_like(x, 3.25)
    yc, _, _ = gn.gn_forward(const, inp["gamma"], inp["beta"], G, inp["eps"])
    torch.cuda.synchronize()
    assert torch.equal(yc.contiguous(), inp["beta"].to(torch.bfloat16).view(1, -1, 1, 1, 1).expand_as(yc).contiguous())


@pytest.mark.parametrize("case", [CL_CASES[0], CL_CASES[4], CL_CASES[6]], ids=lambda c: c.name)
def test_channels_last_optional_backward_outputs(case):
    """The channels-last backward with dx only, and with dgamma/dbeta only, gives the bits of
    the full call."""
    say(f"{case.name} channels-last: backward with dx only, and with dgamma/dbeta only")
    inp = workloads.make(case, DEV)
    x, G = gn.as_layout(inp["x"], "ndhwc"), inp["G"]
    dy = gn.as_layout(inp["dy"], "ndhwc")
    y, mean, rstd = gn.gn_forward(x, inp["gamma"], inp["beta"], G, inp["eps"], inp["out_dtype"])
    dx, dg, db = gn.gn_backward(dy, x, mean, rstd, inp["gamma"], G)
    n1, dg2, db2 = gn.gn_backward(dy, x, mean, rstd, inp["gamma"], G, need_dx=False)
    dx3, n2, n3 = gn.gn_backward(dy, x, mean, rstd, inp["gamma"], G, need_dgamma=False, need_dbeta=False)
    torch.cuda.synchronize()
    assert n1 is None and n2 is None and n3 is None
    assert torch.equal(dg, dg2) and torch.equal(db, db2) and torch.equal(_bits(dx), _bits(dx3))


def test_channels_last_autograd_keeps_the_layout():
    say("group_norm on a channels_last_3d tensor through autograd")
    inp = workloads.make(workloads.custom(2, 32, 8, (8, 8, 8), torch.bfloat16, dist="unet", seed=73), DEV)
    x = inp["x"].contiguous(memory_format=torch.channels_last_3d).requires_grad_(True)
    gamma = inp["gamma"].clone().requires_grad_(True)
    beta = inp["beta"].clone().requires_grad_(True)
    y = gn.group_norm(x, inp["G"], gamma, beta, inp["eps"], activation="relu")
    assert y.is_contiguous(memory_format=torch.channels_last_3d)
    y.backward(inp["dy"])    # an NCDHW gradient is brought to x's layout
    assert x.grad.is_contiguous(memory_format=torch.channels_last_3d)
    y2, m2, r2 = gn.gn_forward(x.detach(), inp["gamma"], inp["beta"], inp["G"], inp["eps"], activation="relu")
    dx2, dg2, db2 = gn.gn_backward(gn.as_layout(inp["dy"], "ndhwc"), x.detach(), m2, r2, inp["gamma"], inp["G"],
                                   beta=inp["beta"], activation="relu")
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), y2) and torch.equal(x.grad, dx2)
    assert torch.equal(gamma.grad, dg2) and torch.equal(beta.grad, db2)


def test_channels_last_rejects_unsupported_shapes():
    x = torch.zeros((1, 24, 4, 4, 4), dtype=torch.bfloat16, device=DEV).contiguous(memory_format=torch.channels_last_3d)
    with pytest.raises(gn.GnError, match="GN_ERR_LAYOUT"):
        gn.gn_forward(x, None, None, 8, out=torch.empty_like(x), mean=torch.empty(1, 8, device=DEV),
                      rstd=torch.empty(1, 8, device=DEV), workspace=torch.empty(1 << 20, dtype=torch.uint8, device=DEV))


# ----------------------------------------------------------------------------- resident path

RESIDENT = [
    # (case, forward resident, backward resident)
    (workloads.custom(1, 16, 2, (16, 16, 16), torch.bfloat16, dist="unet", seed=41), True, True),   # M = 32768, the limit
    (workloads.custom(1, 16, 2, (8, 9, 57), torch.bfloat16, dist="unet", seed=42), False, False),   # M = 32832, just past it
    (workloads.custom(8, 8, 2, (8, 8, 16), torch.bfloat16, dist="normal", seed=43), True, True),    # N*M = 32768
    (workloads.custom(9, 8, 2, (8, 8, 16), torch.float32, dist="normal", seed=44), True, False),    # N*M past the limit
    (workloads.custom(3, 10, 2, (2, 3, 4), torch.bfloat16, dist="unet", seed=45), True, True),      # 15 vectors a group
    (workloads.custom(2, 64, 1, (2, 2, 2), torch.float32, dist="tiny", seed=46), True, True),       # one vector per row
    (workloads.custom(2, 16, 16, (2, 2, 2), torch.bfloat16, dist="deep", seed=47, out_dtype=torch.float32), True, True),
    (workloads.custom(3, 12, 4, (4, 4, 6), torch.bfloat16, torch.float32, dist="deep", seed=48), True, True),
    # backward split over samples: one workgroup gathers all 511 other samples' rows of its channel
    (workloads.custom(512, 2, 2, (8,), torch.bfloat16, dist="unet", seed=49), True, True),
    # C/G = 2 < N = 64: most (n, g) workgroups own no dgamma channel
    (workloads.custom(64, 4, 2, (2, 2, 2), torch.float32, dist="normal", seed=50), True, True),
]


@pytest.mark.parametrize("case,rf,rb", RESIDENT, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_resident_shapes_elementwise(case, rf, rb):
    p = gn.gn_plan_query(case.N, case.C, case.numel // (case.N * case.C), case.G)
    assert (bool(p["resident_forward"]), bool(p["resident_backward"])) == (rf, rb)
    full_check(workloads.make(case, "cpu"), case.name)


@pytest.mark.parametrize("case,rf,rb", RESIDENT[:5], ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_resident_shapes_relu(case, rf, rb):
    full_check(workloads.make(case, "cpu"), case.name + "_relu", relu=True)


# ----------------------------------------------------------------------------- fused relu

RELU_CASES = [workloads.TINY, workloads.DEEP, workloads.DEEP_F32OUT, RAGGED[0], RAGGED[2], RAGGED[3],
              RAGGED[5]]


@pytest.mark.parametrize("case", RELU_CASES, ids=lambda c: c.name)
def test_relu_elementwise(case):
    full_check(workloads.make(case, "cpu"), case.name + "_relu", relu=True)


def test_relu_nan_inf_confined_to_their_group():
    say("relu: NaN/Inf in two groups of (2, 8, 6, 6, 6), G=4")
    inp = workloads.make(workloads.custom(2, 8, 4, (6, 6, 6), torch.bfloat16, seed=22), "cpu")
    x = inp["x"].clone()
    x[0, 2, 1, 1, 1] = float("nan")
    x[1, 7, 0, 0, 0] = float("-inf")
    inp["x"] = x
    r = full_check(inp, "nan_inf_relu", relu=True)
    # relu passes NaN through (no clamp swallows it), in y and in the backward gate
    assert torch.isnan(r["y"][0, 2:4].float()).all() and torch.isnan(r["dx"][1, 6:8].float()).all()
    assert torch.isfinite(r["y"][0, 0:2].float()).all() and torch.isfinite(r["dx"][1, 0:6].float()).all()


def test_relu_scale7_sampled():
    case = workloads.SCALE7
    sampled_check(workloads.make(case, DEV), case.name + "_relu", seed=case.seed, relu=True)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("case", [workloads.DEEP, workloads.SCALE7], ids=lambda c: c.name)
def test_relu_forward_is_unfused_forward_then_relu_bitwise(case, out_dtype):
    """The fused store equals the unfused output with negatives replaced by +0, bit for
    bit: NaN stays NaN, -0.0 stays -0.0 (a channel with gamma = 0, beta = -0.0 makes them)."""
    say(f"{case.name}: fused relu forward vs unfused + relu, out {out_dtype}")
    inp = workloads.make(case, DEV, with_dy=False)
    x, G = inp["x"], inp["G"]
    gamma, beta = inp["gamma"].clone(), inp["beta"].clone()
    gamma[0], beta[0] = 0.0, -0.0
    x = x.clone()
    x.view(x.shape[0], G, -1)[0, G - 1, 5] = float("nan")
    y, m, r = gn.gn_forward(x, gamma, beta, G, inp["eps"], out_dtype)
    yr, mr, rr = gn.gn_forward(x, gamma, beta, G, inp["eps"], out_dtype, activation="relu")
    torch.cuda.synchronize()
    assert torch.equal(m.view(torch.int32), mr.view(torch.int32))
    assert torch.equal(r.view(torch.int32), rr.view(torch.int32))
    ref = torch.where(y < 0, torch.zeros_like(y), y)
    bits = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    assert torch.equal(yr.view(bits), ref.view(bits))
    assert torch.isnan(yr).sum().item() == torch.isnan(y).sum().item() > 0
    assert (yr.view(bits) == torch.tensor(-0.0, dtype=out_dtype).view(bits).item()).any()


@pytest.mark.parametrize("case", [workloads.DEEP, workloads.SCALE7], ids=lambda c: c.name)
def test_relu_gate_all_open_or_all_closed(case):
    """beta far above every |gamma * xhat|: every gate is open and the relu path equals the
    plain path bit for bit. beta far below: y is +0 everywhere and every gradient is 0."""
    say(f"{case.name}: relu with every gate open, then every gate closed")
    inp = workloads.make(case, DEV)
    x, G, gamma, dy = inp["x"], inp["G"], inp["gamma"], inp["dy"]
    for sign in (1.0, -1.0):
        beta = torch.full_like(inp["beta"], sign * 1e4)
        y, m, r = gn.gn_forward(x, gamma, beta, G, inp["eps"])
        a = gn.gn_backward(dy, x, m, r, gamma, G, beta=beta)
        yr, mr, rr = gn.gn_forward(x, gamma, beta, G, inp["eps"], activation="relu")
        b = gn.gn_backward(dy, x, mr, rr, gamma, G, beta=beta, activation="relu")
        torch.cuda.synchronize()
        if sign > 0:
            assert torch.equal(y.view(torch.int16), yr.view(torch.int16))
            for u, v in zip(a, b):
                assert torch.equal(u, v)
        else:
            assert torch.equal(yr.view(torch.int16), torch.zeros_like(yr).view(torch.int16))
            for t in b:
                assert (t == 0).all()


# ----------------------------------------------------------------------------- largest size

def test_volume_past_int32_indexing():
    """2^31 + 512 elements per tensor (bf16): int64 offsets, statistics of 2^28-element groups."""
    S = (1 << 28) + 64
    case = workloads.custom(1, 8, 8, (S,), torch.bfloat16, dist="unet", seed=31)
    sampled_check(workloads.make(case, DEV), "int64_volume", n_random=1 << 16, seed=31)


# ----------------------------------------------------------------------------- input addresses

def _placed(arena, nbytes, bit31):
    """A 256-byte aligned offset into `arena` where 2 * nbytes fit wholly on one side of bit 31
    of the address's low 32-bit word (set if bit31, clear otherwise)."""
    a0 = arena.data_ptr()
    for o in range(0, arena.numel() - 2 * nbytes + 1, 1 << 24):
        lo = (a0 + o) & 0xFFFFFFFF
        if bit31 and lo < 0x80000000:
            o += 0x80000000 - lo
        elif not bit31 and lo >= 0x80000000:
            o += 0x100000000 - lo
        lo = (a0 + o) & 0xFFFFFFFF
        if o + 2 * nbytes <= arena.numel() and bool(lo & 0x80000000) == bit31 \
                and ((lo + 2 * nbytes - 1) & 0x80000000 != 0) == bit31 and lo + 2 * nbytes <= 0x100000000:
            return o
    raise AssertionError("no placement found")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_inputs_whose_addresses_have_bit31_set_in_the_low_word(dtype):
    """The step loads of 16-bit inputs read through a buffer resource whose scalar base is the
    step's address, assembled from two 32-bit words. x and dy placed where the low word has bit
    31 set give the same bits as placed where it is clear (a low word sign-extended over the
    high one would send every such load outside the address space)."""
    case = workloads.custom(1, 32, 8, (64, 64, 48), dtype, dist="unet", seed=98)
    inp = _on_gpu(workloads.make(case, "cpu"))
    nbytes = inp["x"].numel() * inp["x"].element_size()
    arena = torch.empty((3 << 30) + 4 * nbytes, dtype=torch.uint8, device=DEV)
    outs = []
    for bit31 in (False, True):
        o = _placed(arena, nbytes, bit31)
        x = arena[o:o + nbytes].view(dtype).view(inp["x"].shape)
        dy = arena[o + nbytes:o + 2 * nbytes].view(dtype).view(inp["dy"].shape)
        x.copy_(inp["x"])
        dy.copy_(inp["dy"])
        for t in (x, dy):
            assert bool(t.data_ptr() & 0x80000000) == bit31
        say(f"{case.name}: x at {x.data_ptr():#x}, dy at {dy.data_ptr():#x} (bit 31 of the low word "
            f"{'set' if bit31 else 'clear'}) -> gn_forward + gn_backward")
        r = _run({**inp, "x": x, "dy": dy})
        outs.append({k: v.clone() for k, v in r.items()})
    for k in outs[0]:
        a, b = outs[0][k], outs[1][k]
        bits = (lambda t: t.view(torch.int16)) if a.element_size() == 2 else (lambda t: t.view(torch.int32))
        assert torch.equal(bits(a), bits(b)), k
    del arena
    torch.cuda.empty_cache()
