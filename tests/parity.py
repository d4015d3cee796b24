"""Tolerance checks of GPU results against the fp64 oracle.

The bars (the target's tolerances, with the readings that make them well posed where a
reference value is near zero):
  mean       |d| <= 1e-5 * max(|mu|, sigma)                       (sigma = sqrt(var))
  rstd       |d| <= 1e-5 * rstd
  y (fp32)   |d| <= 1e-5 * max(|y64|, |gamma_c| + |beta_c|): relative to |y| where |y| is
             at least the channel's output scale (xhat has unit variance); near y = 0 a
             relative bar is ill-posed, since any fp32 mean is off by O(u * sigma)
  y (bf16)   within 1 bf16 ulp of the fp64 answer rounded once; elements whose fp32 terms
             cancel may instead meet the fp32 bar (counted and reported)
  dx (fp32)  |d| <= 1e-4 * max|dx64|
  dx (bf16)  |d| <= ulp_bf16(dx64) + 1e-4 * max|dx64|
  dgamma/dbeta  |d_c| <= max(1e-4 * |ref_c|, 2 * D * 2^-24 * sum|terms_c|), D the depth of
             the kernel's fp32 summation tree for the shape (the a-priori bound of fp32
             summation in that order)
NaN must match NaN (position for position) and infinities must match exactly.
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
    if y_gpu.dtype == np.uint16:
        got = as_f64(y_gpu)
        ok, why = _nan_inf_match(got, y64)
        assert ok, f"y: {why}"
        fin = np.isfinite(y64)
        ref_bits = O.round_bf16(y64)
        dist = np.abs(_ordered(y_gpu) - _ordered(ref_bits))
        bad = fin & (dist > 1)
        fallback = bad & (np.abs(got - y64) <= fp32_floor)
        hard = bad & ~fallback
        assert not hard.any(), (f"y(bf16): {hard.sum()} elements beyond 1 ulp, e.g. gpu "
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


def check_dx(dx_gpu, dx64, scale=None):
    scale = float(np.max(np.abs(dx64[np.isfinite(dx64)]))) if scale is None else scale
    got = as_f64(dx_gpu)
    ok, why = _nan_inf_match(got, dx64)
    assert ok, f"dx: {why}"
    fin = np.isfinite(dx64)
    bar = 1e-4 * scale + (bf16_ulp(dx64) if dx_gpu.dtype == np.uint16 else 0.0)
    d = np.abs(got - dx64)
    over = fin & (d > bar)
    assert not over.any(), (f"dx: {over.sum()} elements over the bar; worst "
                            f"{np.max((d / bar)[fin]):.3g}")
    return {"dx_of_bar": float(np.max((d / bar)[fin])) if fin.any() else 0.0}


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


def check_param(name, got, ref, abs_terms, depth):
    got = got.astype(np.float64)
    bar = np.maximum(1e-4 * np.abs(ref), 2 * depth * U32 * abs_terms)
    d = np.abs(got - ref)
    ok, why = _nan_inf_match(got, ref)
    assert ok, f"{name}: {why}"
    fin = np.isfinite(ref)
    assert (d[fin] <= bar[fin]).all(), f"{name}: worst {np.max(d[fin] / bar[fin]):.3g} of the bar"
    return {f"{name}_of_bar": float(np.max(d[fin] / bar[fin])) if fin.any() else 0.0}
