"""Tolerance checks of GPU results against the fp64 oracle.

The bars (the target's tolerances, with the readings that make them well posed where a
reference value is near zero):
  mean       |d| <= 1e-5 * max(|mu|, sigma)                       (sigma = sqrt(var))
  rstd       |d| <= 1e-5 * rstd
  y (fp32)   |d| <= 1e-5 * max(|y64|, |gamma_c| + |beta_c|): relative to |y| where |y| is
             at least the channel's output scale (xhat has unit variance); near y = 0 a
             relative bar is ill-posed, since any fp32 mean is off by O(u * sigma)
  y (bf16, fp16)  within 1 ulp of the fp64 answer rounded once to that format; elements
             whose fp32 terms cancel may instead meet the fp32 bar (counted and reported)
  dx (fp32)  |d| <= 1e-4 * max|dx64|
  dx (bf16, fp16)  |d| <= ulp(dx64) + 1e-4 * max|dx64|, ulp in dx's format
  dgamma/dbeta  on a channel whose sum does not cancel (|ref_c| >= 0.1 * sum|terms_c|):
             |d_c| <= 1e-4 * |ref_c|, the target's bar as stated. On a channel whose sum
             cancels (|ref_c| small next to its terms, as for any zero-mean dy), a relative
             bar is ill-posed and the a-priori bound of fp32 summation is the floor:
             |d_c| <= max(1e-4 * |ref_c|, 2 * D * 2^-24 * sum|terms_c|), D the depth of the
             kernel's fp32 summation tree for the shape. dgamma also gets the propagation of
             the published fp32 statistics' rounding, 4 * 2^-24 * (max_n |mean| * rstd *
             sum|g| + |ref_c|), since dgamma_c = sum g * (x - mean) * rstd moves by rstd *
             sum g per unit of mean and the backward consumes the forward's fp32 mean and
             rstd (stats_slack); it is negligible unless |mean| >> sigma
NaN must match NaN (position for position) and infinities must match exactly.

With the fused relu, the gate is a sign decision taken on the fp32 pre-activation. Where
the fp64 pre-activation lies within the y bar of zero (|pre| <= 1e-5 * (|gamma_c| +
|beta_c|)) either decision is correct to working precision: such an element's dx may be
either candidate, and the sums it feeds (dgamma_c, dbeta_c and the group's c1/c2) get the
slack one flipped gate can cause (ReluBand below). Everywhere else the gates must agree.
"""
import math

import numpy as np
import torch

from oracle import oracle as O

U32 = 2.0 ** -24


def to_np(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a):
    if a.dtype == np.uint16:
        return O.bf16_bits_to_f64(a)
    if a.dtype == np.float16:
        return O.f16_bits_to_f64(a.view(np.uint16))
    return a.astype(np.float64)


def _ordered(bits):
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _nan_inf_match(got, ref):
    gn, rn = np.isnan(got), np.isnan(ref)
    if not np.array_equal(gn, rn):
        return False, f"NaN positions differ: gpu {gn.sum()} oracle {rn.sum()}"
    gi, ri = np.isinf(got), np.isinf(ref)
    if not np.array_equal(gi, ri) or not np.array_equal(got[gi], ref[ri]):
        return False, "infinities differ"
    return True, ""


def check_stats(mean_gpu, rstd_gpu, mean64, var64, rstd64):
    mean_gpu = mean_gpu.reshape(mean64.shape).astype(np.float64)
    rstd_gpu = rstd_gpu.reshape(rstd64.shape).astype(np.float64)
    for name, got, ref in (("mean", mean_gpu, mean64), ("rstd", rstd_gpu, rstd64)):
        ok, why = _nan_inf_match(got, ref)
        assert ok, f"{name}: {why}"
    fin = np.isfinite(mean64) & np.isfinite(rstd64)
    sigma = np.sqrt(np.maximum(var64, 0))
    dm = np.abs(mean_gpu - mean64)[fin]
    bm = (1e-5 * np.maximum(np.abs(mean64), sigma))[fin]
    assert (dm <= bm).all(), f"mean: worst {np.max(dm / np.maximum(bm, 1e-300)):.3g} of the bar"
    dr = np.abs(rstd_gpu - rstd64)[fin]
    br = (1e-5 * rstd64)[fin]
    assert (dr <= br).all(), f"rstd: worst {np.max(dr / br):.3g} of the bar"
    return {"mean_rel": float(np.max(dm / np.maximum(bm, 1e-300)) * 1e-5) if dm.size else 0.0,
            "rstd_rel": float(np.max(dr / rstd64[fin])) if dr.size else 0.0}


def channel_params_at(idx, shape, gamma, beta):
    """(beta_c, gamma_c) for flat indices idx of an NC* volume; None means 0 / 1."""
    S = int(np.prod(shape[2:])) if len(shape) > 2 else 1
    c = (np.asarray(idx) // S) % shape[1]
    b = np.zeros(c.shape) if beta is None else np.asarray(beta, dtype=np.float64)[c]
    g = np.ones(c.shape) if gamma is None else np.asarray(gamma, dtype=np.float64)[c]
    return b, g


def check_y(y_gpu, y64, beta_at, gamma_at):
    """y_gpu: fp32 array or uint16 bf16 bits, flat; y64 fp64 flat; beta_at/gamma_at: the
    channel's beta and gamma per element."""
    fp32_floor = 1e-5 * np.maximum(np.abs(y64), np.abs(gamma_at) + np.abs(beta_at))
    if y_gpu.dtype in (np.uint16, np.float16):
        fmt = "bf16" if y_gpu.dtype == np.uint16 else "fp16"
        got = as_f64(y_gpu)
        ok, why = _nan_inf_match(got, y64)
        assert ok, f"y: {why}"
        fin = np.isfinite(y64)
        bits = y_gpu if fmt == "bf16" else y_gpu.view(np.uint16)
        ref_bits = O.round_bf16(y64) if fmt == "bf16" else O.round_f16(y64)
        dist = np.abs(_ordered(bits) - _ordered(ref_bits))
        bad = fin & (dist > 1)
        fallback = bad & (np.abs(got - y64) <= fp32_floor)
        hard = bad & ~fallback
        assert not hard.any(), (f"y({fmt}): {hard.sum()} elements beyond 1 ulp, e.g. gpu "
                                f"{got[hard][:4]} vs {y64[hard][:4]}")
        return {"max_ulp": int(dist[fin].max()) if fin.any() else 0, "fallback": int(fallback.sum())}
    got = y_gpu.astype(np.float64)
    ok, why = _nan_inf_match(got, y64)
    assert ok, f"y: {why}"
    fin = np.isfinite(y64)
    d = np.abs(got - y64)[fin]
    b = fp32_floor[fin]
    assert (d <= b).all(), f"y(fp32): worst {np.max(d / b):.3g} of the bar"
    return {"y_rel_of_bar": float(np.max(d / b)) if d.size else 0.0}


def bf16_ulp(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def f16_ulp(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def _ulp_of(dtype, v):
    if dtype == np.uint16:
        return bf16_ulp(v)
    if dtype == np.float16:
        return f16_ulp(v)
    return 0.0


def check_dx(dx_gpu, dx64, scale=None, band=None):
    """band: optional (mask, alt64, slack) from ReluBand.dx_terms: elements under mask may
    instead match alt64 (the other gate decision); slack widens every element's bar."""
    fin_ref = dx64[np.isfinite(dx64)]
    scale = (float(np.max(np.abs(fin_ref))) if fin_ref.size else 0.0) if scale is None else scale
    got = as_f64(dx_gpu)
    ok, why = _nan_inf_match(got, dx64)
    assert ok, f"dx: {why}"
    fin = np.isfinite(dx64)
    slack = 0.0 if band is None else band[2]
    bar = 1e-4 * scale + _ulp_of(dx_gpu.dtype, dx64) + slack
    bar = np.maximum(bar, 1e-300)
    d = np.abs(got - dx64)
    over = fin & (d > bar)
    alt_used = 0
    if band is not None:
        mask, alt64, _ = band
        bar_alt = 1e-4 * scale + _ulp_of(dx_gpu.dtype, alt64) + slack
        alt_ok = mask & (np.abs(got - alt64) <= bar_alt)
        alt_used = int((over & alt_ok).sum())
        over &= ~alt_ok
    assert not over.any(), (f"dx: {over.sum()} elements over the bar; worst "
                            f"{np.max((d / bar)[fin]):.3g}")
    rep = {"dx_of_bar": float(np.max(np.where(over | ~fin, 0, d / bar))) if fin.any() else 0.0}
    if band is not None:
        rep["gate_band"] = int(band[0].sum())
        rep["gate_flipped"] = alt_used
    return rep


def reduction_depth(plan, N):
    """Depth of the kernels' fp32 summation tree for dgamma/dbeta at a plan."""
    blk = plan["block"]
    waves = blk // 64
    step = blk * plan["vectors_per_step"] * 8
    steps = max(1, math.ceil(plan["chunk"] / step))
    per_job = 5 + (steps - 1) + 6 + (waves - 1)
    nk = N * plan["chunks_per_row"]
    across = (math.ceil(nk / blk) - 1) + 6 + (waves - 1)
    return per_job + across


# A channel sum that keeps at least this fraction of its terms' magnitude is held to the
# relative bar alone.
WELL_CONDITIONED = 0.1


def well_conditioned(ref, abs_terms):
    """Channels whose sum keeps at least WELL_CONDITIONED of its terms' magnitude (a channel
    whose terms are all zero has nothing to be relative to: its floor is zero anyway)."""
    ref = np.asarray(ref, dtype=np.float64)
    abs_terms = np.asarray(abs_terms, dtype=np.float64)
    return np.isfinite(ref) & (abs_terms > 0) & (np.abs(ref) >= WELL_CONDITIONED * abs_terms)


def check_param(name, got, ref, abs_terms, depth, slack=0.0):
    got = got.astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rel = 1e-4 * np.abs(ref)
    wc = well_conditioned(ref, abs_terms)
    bar = np.where(wc, rel, np.maximum(rel, 2 * depth * U32 * abs_terms)) + slack
    bar = np.maximum(bar, 1e-300)
    d = np.abs(got - ref)
    ok, why = _nan_inf_match(got, ref)
    assert ok, f"{name}: {why}"
    fin = np.isfinite(ref)
    assert (d[fin] <= bar[fin]).all(), f"{name}: worst {np.max(d[fin] / bar[fin]):.3g} of the bar"
    rep = {f"{name}_of_bar": float(np.max(d[fin] / bar[fin])) if fin.any() else 0.0,
           f"{name}_well_conditioned": int(wc.sum())}
    if wc.any():
        rep[f"{name}_max_rel_err"] = float(np.max(d[wc] / np.abs(ref[wc])))
    return rep


def stats_slack(mean64, rstd64, abs_dy, ref, C):
    """The part of dgamma's deviation owed to the fp32 rounding of the statistics the
    backward consumes: 4 * 2^-24 * (max_n |mean_g| * rstd_g * sum|g|_c + |ref_c|)."""
    mean64 = np.asarray(mean64, dtype=np.float64)
    rstd64 = np.asarray(rstd64, dtype=np.float64)
    G = mean64.shape[1]
    with np.errstate(invalid="ignore"):
        w = np.max(np.abs(mean64) * rstd64, axis=0)          # [G]
    w = np.repeat(np.where(np.isfinite(w), w, 0.0), C // G)  # [C]
    return 4 * U32 * (w * np.asarray(abs_dy) + np.abs(np.asarray(ref)))


class ReluBand:
    """The elements whose relu gate fp32 arithmetic may decide either way, and the slack a
    flipped gate moves into the backward.

    pre = gamma_c * xhat + beta_c from the oracle's fp64 statistics. An element with
    |pre| <= rel * (|gamma_c| + |beta_c|) is in the band. Flipping its gate moves its own dx
    by rstd * gamma_c * dy, dbeta_c by |dy|, dgamma_c by |dy * xhat|, and the group's
    c1 / c2 by |gamma_c * dy| / M and |gamma_c * dy * xhat| / M (so every dx of the group by
    rstd * (dc1 + |xhat| * dc2)). Non-finite pre (NaN groups) is never in the band: the
    gate passes NaN on both sides.
    """

    def __init__(self, x, dy, G, gamma, beta, mean64, rstd64, rel=1e-5):
        self.x = to_np(x)
        self.dy = to_np(dy)
        N, C = self.x.shape[:2]
        S = self.x.size // (N * C)
        self.x = self.x.reshape(N, C, S)
        self.dy = self.dy.reshape(N, C, S)
        self.N, self.C, self.S, self.G = N, C, S, G
        self.Cg = C // G
        self.gamma = np.ones(C) if gamma is None else to_np(gamma).astype(np.float64).reshape(C)
        self.beta = np.zeros(C) if beta is None else to_np(beta).astype(np.float64).reshape(C)
        self.mean = np.asarray(mean64, dtype=np.float64).reshape(N, G)
        self.rstd = np.asarray(rstd64, dtype=np.float64).reshape(N, G)
        self.rel = rel
        self.dbeta = np.zeros(C)
        self.dgamma = np.zeros(C)
        dc1 = np.zeros((N, G))
        dc2 = np.zeros((N, G))
        self.count = 0
        with np.errstate(invalid="ignore", over="ignore"):
            for n in range(N):
                for c in range(C):
                    g = c // self.Cg
                    xh = (as_f64(self.x[n, c]) - self.mean[n, g]) * self.rstd[n, g]
                    band = self._band(self.gamma[c] * xh + self.beta[c], c)
                    if not band.any():
                        continue
                    a = np.abs(as_f64(self.dy[n, c][band]))
                    ax = a * np.abs(xh[band])
                    self.count += int(band.sum())
                    self.dbeta[c] += a.sum()
                    self.dgamma[c] += ax.sum()
                    dc1[n, g] += abs(self.gamma[c]) * a.sum()
                    dc2[n, g] += abs(self.gamma[c]) * ax.sum()
        M = self.Cg * S
        self.dc1, self.dc2 = dc1 / M, dc2 / M

    def _band(self, pre, c):
        return np.isfinite(pre) & (np.abs(pre) <= self.rel * (np.abs(self.gamma[c]) + np.abs(self.beta[c])))

    def dx_terms(self, idx, dx64):
        """(mask, alt64, slack) at flat indices idx for check_dx."""
        idx = np.asarray(idx, dtype=np.int64)
        n = idx // (self.C * self.S)
        c = (idx // self.S) % self.C
        s = idx % self.S
        g = c // self.Cg
        with np.errstate(invalid="ignore", over="ignore"):
            xh = (as_f64(self.x[n, c, s]) - self.mean[n, g]) * self.rstd[n, g]
            pre = self.gamma[c] * xh + self.beta[c]
            mask = self._band(pre, c)
            r = self.rstd[n, g]
            step = r * self.gamma[c] * as_f64(self.dy[n, c, s])
            alt = np.where(pre > 0, dx64 - step, dx64 + step)
            slack = r * (self.dc1[n, g] + np.abs(xh) * self.dc2[n, g])
        slack = np.where(np.isfinite(slack), slack, 0.0)
        return mask, alt, slack
