"""Pins for the fp64 CPU oracle, each against something other than the oracle itself.

- closed forms of the GroupNorm definition (zero mean and var/(var+eps) variance of
  the normalized output, constant input -> beta, single element groups);
- an independent library: torch's CPU float64 group_norm, instance_norm (G = C),
  layer_norm (G = 1) and autograd;
- exact rational brute force on an 8-element group;
- central finite differences of L = sum(y * dy) for dx, dgamma, dbeta;
- the bf16 rounding helper against torch's fp32 -> bf16 conversion and hand-built
  ties, double-rounding traps and special values.
"""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads
from oracle import oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


def _f64(t):
    return t.detach().to(torch.float64)


def _tiny():
    return workloads.make(workloads.TINY, "cpu")


# ----------------------------------------------------------------------------- closed forms

def test_closed_form_mean_zero_and_variance_ratio():
    """gamma = 1, beta = 0: per group mean(y) = 0 and var(y) = var / (var + eps)."""
    inp = _tiny()
    x, G, eps = inp["x"], inp["G"], inp["eps"]
    out = O.forward(x, G, eps=eps)
    N, C = x.shape[:2]
    y = out["y"].reshape(N, G, -1)
    var = out["var"]
    eps64 = float(np.float32(eps))
    for n in range(N):
        for g in range(G):
            yg = y[n, g]
            assert abs(yg.mean()) < 1e-12
            # the oracle's var is checked by an independent numpy computation too
            xg = x.numpy().astype(np.float64).reshape(N, G, -1)[n, g]
            assert var[n, g] == pytest.approx(np.var(xg), rel=1e-12)
            expect = var[n, g] / (var[n, g] + eps64)
            assert np.var(yg) == pytest.approx(expect, rel=1e-12)
            # and the "variance 1" phrasing differs from the exact form by eps/(var+eps)
            assert abs(np.var(yg) - 1.0) == pytest.approx(eps64 / (var[n, g] + eps64), rel=1e-6)


@pytest.mark.parametrize("const", [0.3, 100.0, -7.25, 0.0])
def test_constant_input_maps_to_beta_exactly(const):
    N, C, G, S = 2, 6, 3, 50
    x = np.full((N, C, S), const, dtype=np.float32)
    gamma = np.linspace(0.5, 1.5, C).astype(np.float32)
    beta = np.linspace(-0.2, 0.3, C).astype(np.float32)
    out = O.forward(x, G, gamma, beta, eps=1e-5)
    expect = np.broadcast_to(beta.astype(np.float64)[None, :, None], (N, C, S))
    assert np.array_equal(out["y"], expect)
    assert np.all(out["var"] == 0.0)
    assert np.all(out["rstd"] == 1.0 / math.sqrt(float(np.float32(1e-5))))


def test_single_element_groups_match_printed_rstd():
    """M = 1: rstd = 1/sqrt(eps) (printed as 316), y = beta, dx = 0 exactly."""
    ref = GOLDEN["single_element_group"]
    rng = np.random.default_rng(5)
    N, C, G = 2, 4, 4
    x = rng.normal(size=(N, C, 1)).astype(np.float32)
    dy = rng.normal(size=(N, C, 1)).astype(np.float32)
    gamma = rng.normal(1, 0.1, C).astype(np.float32)
    beta = rng.normal(0, 0.1, C).astype(np.float32)
    out = O.forward(x, G, gamma, beta, eps=ref["eps"])
    assert np.all(np.round(out["rstd"]) == ref["rstd_printed"])
    # eps reaches the kernels as an fp32 value; the oracle widens that value exactly
    assert np.all(out["rstd"] == 1.0 / math.sqrt(float(np.float32(ref["eps"]))))
    assert np.array_equal(out["y"], np.broadcast_to(beta.astype(np.float64)[None, :, None], x.shape))
    b = O.backward(dy, x, G, gamma, eps=ref["eps"])
    assert np.all(b["dx"] == ref["dx_exact"])
    assert np.allclose(b["dbeta"], dy.astype(np.float64).sum(axis=(0, 2)), rtol=1e-15)
    assert np.all(b["dgamma"] == 0.0)


def test_nan_and_inf_stay_in_their_group():
    rng = np.random.default_rng(9)
    N, C, G, S = 2, 8, 4, 30
    x = rng.normal(size=(N, C, S)).astype(np.float32)
    x[0, 2, 7] = np.nan   # group (0, 1)
    x[1, 6, 3] = np.inf   # group (1, 3)
    out = O.forward(x, G, eps=1e-5)
    y = out["y"].reshape(N, G, -1)
    bad = {(0, 1), (1, 3)}
    for n in range(N):
        for g in range(G):
            if (n, g) in bad:
                assert np.all(np.isnan(y[n, g])) and np.isnan(out["rstd"][n, g])
            else:
                assert np.all(np.isfinite(y[n, g]))


# ----------------------------------------------------------------------------- independent library

def _torch_ref(x64, G, gamma, beta, eps, dy64=None):
    x64 = x64.clone().requires_grad_(dy64 is not None)
    g = torch.from_numpy(np.asarray(gamma, dtype=np.float32)).to(torch.float64).requires_grad_(dy64 is not None)
    b = torch.from_numpy(np.asarray(beta, dtype=np.float32)).to(torch.float64).requires_grad_(dy64 is not None)
    y = F.group_norm(x64, G, g, b, float(np.float32(eps)))
    if dy64 is None:
        return y.detach(), None
    y.backward(dy64)
    return y.detach(), (x64.grad, g.grad, b.grad)


@pytest.mark.parametrize("case", ["tiny", "deep", "ragged", "f16"])
def test_against_torch_float64_group_norm(case):
    if case == "tiny":
        inp = _tiny()
    elif case == "deep":
        inp = workloads.make(workloads.DEEP, "cpu")
    elif case == "f16":
        inp = workloads.make(workloads.custom(2, 8, 4, (6, 7, 5), torch.float16, dist="unet", seed=6), "cpu")
    else:
        inp = workloads.make(workloads.custom(3, 6, 2, (5, 7, 3), torch.bfloat16, dist="unet", seed=3), "cpu")
    x, dy, G, eps = inp["x"], inp["dy"], inp["G"], inp["eps"]
    gamma, beta = inp["gamma"].numpy(), inp["beta"].numpy()
    out = O.forward(x, G, gamma, beta, eps=eps)
    y_t, grads = _torch_ref(_f64(x), G, gamma, beta, eps, _f64(dy))
    scale = np.abs(y_t.numpy()).max()
    assert np.abs(out["y"] - y_t.numpy()).max() <= 1e-12 * scale
    b = O.backward(dy, x, G, gamma, eps=eps)
    dx_t, dg_t, db_t = (t.numpy() for t in grads)
    assert np.abs(b["dx"] - dx_t).max() <= 1e-10 * np.abs(dx_t).max()
    assert np.abs(b["dgamma"] - dg_t).max() <= 1e-10 * np.abs(dg_t).max()
    assert np.abs(b["dbeta"] - db_t).max() <= 1e-10 * np.abs(db_t).max()


def test_special_cases_instance_norm_and_layer_norm():
    rng = np.random.default_rng(11)
    N, C, D, H, W = 2, 6, 3, 4, 5
    x = (rng.normal(size=(N, C, D, H, W)) * 1.7 + 0.4).astype(np.float32)
    eps = 1e-5
    x64 = torch.from_numpy(x).to(torch.float64)
    # G = C is instance normalization
    out = O.forward(x, C, eps=eps)
    ref = F.instance_norm(x64, eps=float(np.float32(eps)))
    assert np.abs(out["y"] - ref.numpy()).max() < 1e-12
    # G = 1 is layer normalization over (C, D, H, W)
    out = O.forward(x, 1, eps=eps)
    ref = F.layer_norm(x64, (C, D, H, W), eps=float(np.float32(eps)))
    assert np.abs(out["y"] - ref.numpy()).max() < 1e-12


# ----------------------------------------------------------------------------- exact brute force

def test_exact_rational_brute_force_on_eight_elements():
    getcontext().prec = 60
    vals = [0.75, -1.5, 2.25, 0.125, 3.0, -0.625, 1.0, 0.5]  # dyadic: exact in fp32 and fp64
    x = np.array(vals, dtype=np.float32).reshape(1, 2, 4)     # C=2, G=1 -> M = 8
    gamma = np.array([1.25, -0.5], dtype=np.float32)
    beta = np.array([0.25, 0.125], dtype=np.float32)
    eps32 = np.float32(1e-5)
    out = O.forward(x, 1, gamma, beta, eps=float(eps32))
    fx = [Fraction(v) for v in vals]
    mu = sum(fx) / 8
    var = sum((v - mu) ** 2 for v in fx) / 8
    assert Fraction(out["mean"][0, 0]) == mu                           # dyadic, exact
    assert abs(Fraction(out["var"][0, 0]) - var) <= var * Fraction(2, 2 ** 52)
    rstd = 1 / (Decimal(var.numerator) / Decimal(var.denominator) + Decimal(float(eps32))).sqrt()
    assert abs(Decimal(out["rstd"][0, 0]) - rstd) <= rstd * Decimal(2) ** -50
    for i, v in enumerate(fx):
        c = i // 4
        xm = v - mu
        exact = (Decimal(xm.numerator) / Decimal(xm.denominator)) * rstd * Decimal(float(gamma[c])) \
            + Decimal(float(beta[c]))
        assert abs(Decimal(out["y"].ravel()[i]) - exact) <= Decimal(2) ** -48 * (abs(exact) + 1)


# ----------------------------------------------------------------------------- finite differences

def _loss(x64, G, gamma, beta, eps, w):
    return float((O.forward(x64, G, gamma, beta, eps=eps, tag="f64")["y"] * w).sum())


def test_backward_against_central_differences_all_elements():
    rng = np.random.default_rng(21)
    N, C, G, S = 2, 4, 2, 60
    x = rng.normal(0.3, 1.2, size=(N, C, S))
    w = rng.normal(size=(N, C, S))
    gamma = rng.normal(1, 0.1, C).astype(np.float32)
    beta = rng.normal(0, 0.1, C).astype(np.float32)
    eps = 1e-5
    b = O.backward(w, x, G, gamma, eps=eps, dy_tag="f64", x_tag="f64")
    h = 1e-5
    fd = np.empty_like(x)
    flat, fdf = x.reshape(-1), fd.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + h; lp = _loss(x, G, gamma, beta, eps, w)
        flat[i] = old - h; lm = _loss(x, G, gamma, beta, eps, w)
        flat[i] = old
        fdf[i] = (lp - lm) / (2 * h)
    assert np.abs(b["dx"] - fd).max() <= 1e-6 * np.abs(fd).max()


def test_param_gradients_and_sampled_dx_against_central_differences_tiny():
    inp = _tiny()
    x = inp["x"].numpy().astype(np.float64)
    w = inp["dy"].numpy().astype(np.float64)
    gamma, beta, G, eps = inp["gamma"].numpy(), inp["beta"].numpy(), inp["G"], inp["eps"]
    b = O.backward(w, x, G, gamma, eps=eps, dy_tag="f64", x_tag="f64")
    # dgamma, dbeta: L is linear in gamma and beta, so central differences are exact up to rounding.
    # gamma/beta are fp32 at the oracle's boundary: step by an fp32-exact amount.
    for c in range(x.shape[1]):
        for name, vec, grad in (("gamma", gamma, b["dgamma"]), ("beta", beta, b["dbeta"])):
            h = np.float32(2.0 ** -10)
            vp = vec.copy(); vp[c] += h
            vm = vec.copy(); vm[c] -= h
            hp, hm = float(vp[c]) - float(vec[c]), float(vec[c]) - float(vm[c])
            if name == "gamma":
                lp, lm = _loss(x, G, vp, beta, eps, w), _loss(x, G, vm, beta, eps, w)
            else:
                lp, lm = _loss(x, G, gamma, vp, eps, w), _loss(x, G, gamma, vm, eps, w)
            fd = (lp - lm) / (hp + hm)
            assert grad[c] == pytest.approx(fd, rel=1e-8, abs=1e-9 * np.abs(w).sum())
    rng = np.random.default_rng(1)
    flat = x.reshape(-1)
    idx = rng.choice(flat.size, 48, replace=False)
    h = 1e-5
    scale = np.abs(b["dx"]).max()
    for i in idx:
        old = flat[i]
        flat[i] = old + h; lp = _loss(x, G, gamma, beta, eps, w)
        flat[i] = old - h; lm = _loss(x, G, gamma, beta, eps, w)
        flat[i] = old
        assert b["dx"].reshape(-1)[i] == pytest.approx((lp - lm) / (2 * h), abs=1e-6 * scale)


def test_backward_closed_forms():
    """sum over a group of dx is 0 for any gamma; sum of dx*xhat = rstd*M*c2*eps/(var+eps); dbeta = sum dy."""
    inp = workloads.make(workloads.custom(2, 8, 4, (6, 5, 4), torch.float32, dist="tiny", seed=8), "cpu")
    x, dy, G, eps = inp["x"], inp["dy"], inp["G"], inp["eps"]
    gamma = inp["gamma"].numpy()
    b = O.backward(dy, x, G, gamma, eps=eps)
    f = O.forward(x, G, eps=eps)  # gamma=1, beta=0: y is xhat
    N, C = x.shape[:2]
    dx = b["dx"].reshape(N, G, -1)
    xhat = f["y"].reshape(N, G, -1)
    M = dx.shape[-1]
    eps64 = float(np.float32(eps))
    for n in range(N):
        for g in range(G):
            scale = np.abs(dx[n, g]).sum()
            assert abs(dx[n, g].sum()) <= 1e-13 * scale
            lhs = (dx[n, g] * xhat[n, g]).sum()
            rhs = b["rstd"][n, g] * M * b["c2"][n, g] * eps64 / (f["var"][n, g] + eps64)
            assert lhs == pytest.approx(rhs, rel=1e-6, abs=1e-13 * scale)
    assert np.allclose(b["dbeta"], dy.numpy().astype(np.float64).sum(axis=(0, 2, 3, 4)), rtol=1e-13)


def test_sampled_entry_points_agree_with_full():
    inp = _tiny()
    x, dy, G, eps = inp["x"], inp["dy"], inp["G"], inp["eps"]
    gamma, beta = inp["gamma"], inp["beta"]
    f = O.forward(x, G, gamma, beta, eps=eps)
    b = O.backward(dy, x, G, gamma, eps=eps)
    idx = np.arange(0, x.numel(), 37, dtype=np.int64)
    assert np.array_equal(O.forward_at(x, G, idx, f["mean"], f["rstd"], gamma, beta), f["y"].reshape(-1)[idx])
    assert np.array_equal(O.backward_at(dy, x, G, idx, b["mean"], b["rstd"], b["c1"], b["c2"], gamma),
                          b["dx"].reshape(-1)[idx])


# ----------------------------------------------------------------------------- rounding helper

def test_round_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(2)
    v32 = np.concatenate([
        rng.normal(size=20000).astype(np.float32),
        (rng.normal(size=2000) * 1e30).astype(np.float32),
        (rng.normal(size=2000) * 1e-38).astype(np.float32),   # fp32 subnormals
        np.array([3.3895e38, -3.3895e38, 3.4e38, 1e-45, -0.0, 0.0], dtype=np.float32),
    ])
    ours = O.round_bf16(v32.astype(np.float64))
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_round_bf16_ties_double_rounding_and_specials():
    r = O._load().gno_round_bf16
    assert r(1.0 + 2.0 ** -8) == 0x3F80            # tie -> even (1.0)
    assert r(1.0 + 3 * 2.0 ** -8) == 0x3F82        # tie -> even (1 + 2^-6)
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # just above the tie: up (fp32 first would tie to 1.0)
    assert r(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == 0xBF81
    assert r(float("inf")) == 0x7F80 and r(float("-inf")) == 0xFF80
    assert r(float("nan")) == 0x7FC0
    assert r(2.0 ** 128 * (1 - 2.0 ** -9)) == 0x7F80  # rounds up past the largest finite bf16
    assert r((2 - 2.0 ** -7) * 2.0 ** 127) == 0x7F7F  # largest finite
    assert r(2.0 ** -133) == 0x0001 and r(2.0 ** -134) == 0x0000 and r(2.0 ** -134 * 1.5) == 0x0001
    assert r(-0.0) == 0x8000
    assert np.array_equal(O.round_f32(np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24])),
                          np.array([1.0, 1.0 + 2.0 ** -22], dtype=np.float32))


def test_f16_decode_exhaustive_against_numpy():
    """The oracle's binary16 decoder, written from the format's definition, on all 65536
    bit patterns against numpy's float16."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = O.f16_bits_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(ours, ref, equal_nan=True)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))


def test_round_f16_against_numpy_ties_and_specials():
    """Rounding fp64 -> fp16 once, nearest-even: random values across the whole range
    (subnormals and the overflow edge included) against numpy's direct conversion, every
    exact midpoint between consecutive finite fp16 values, and hand-built cases."""
    rng = np.random.default_rng(8)
    v = np.concatenate([rng.normal(size=50000) * 10.0 ** rng.integers(-9, 5, 50000),
                        rng.uniform(65000, 66000, 5000), -rng.uniform(0, 2.0 ** -14, 5000)])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(O.round_f16(v), ref)
    # exact midpoints: ties go to the even neighbour (even fraction bit)
    lo = np.arange(0, 0x7BFF, dtype=np.uint16)            # finite positives with a finite successor
    a, b = lo.view(np.float16).astype(np.float64), (lo + 1).view(np.float16).astype(np.float64)
    mid = (a + b) / 2                                     # exact in fp64
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    assert np.array_equal(O.round_f16(mid), want)
    assert np.array_equal(O.round_f16(-mid), want | np.uint16(0x8000))
    r = O._load().gno_round_f16
    assert r(65504.0) == 0x7BFF and r(65519.99) == 0x7BFF and r(65520.0) == 0x7C00  # tie past the max -> inf
    assert r(2.0 ** -24) == 0x0001 and r(2.0 ** -25) == 0x0000 and r(1.5 * 2.0 ** -25) == 0x0001
    assert r(1.0 + 2.0 ** -11 + 2.0 ** -40) == 0x3C01   # just above a tie: up
    assert r(float("inf")) == 0x7C00 and r(float("-inf")) == 0xFC00 and r(-0.0) == 0x8000
    assert (r(float("nan")) & 0x7C00) == 0x7C00 and (r(float("nan")) & 0x3FF) != 0


# ----------------------------------------------------------------------------- negative control

def test_naive_variance_formula_fails_where_the_oracle_does_not():
    """At mu/sigma = 1e5 an fp32 E[x^2] - E[x]^2 loses the variance; the oracle keeps it."""
    ratio = GOLDEN["naive_variance_breaks"]["mu_over_sigma"]
    rng = np.random.default_rng(4)
    sigma = 1.0
    x = (ratio * sigma + rng.normal(0, sigma, 8192)).reshape(1, 1, -1)
    out = O.forward(x, 1, eps=1e-5, tag="f64")
    true_var = np.var(x.astype(np.float64))
    assert out["var"][0, 0] == pytest.approx(true_var, rel=1e-9)
    x32 = x.astype(np.float32).astype(np.float64)
    naive = np.float32(np.mean(x32.astype(np.float32) ** 2, dtype=np.float32)) - \
        np.float32(np.mean(x32.astype(np.float32), dtype=np.float32)) ** 2
    assert abs(float(naive) - true_var) > 0.5 * true_var


# ----------------------------------------------------------------------------- fused relu option

def _torch_relu_ref(x64, G, gamma, beta, eps, dy64):
    x64 = x64.clone().requires_grad_(True)
    g = torch.from_numpy(np.asarray(gamma, dtype=np.float32)).to(torch.float64).requires_grad_(True)
    b = torch.from_numpy(np.asarray(beta, dtype=np.float32)).to(torch.float64).requires_grad_(True)
    y = torch.relu(F.group_norm(x64, G, g, b, float(np.float32(eps))))
    y.backward(dy64)
    return y.detach().numpy(), x64.grad.numpy(), g.grad.numpy(), b.grad.numpy()


def test_relu_option_against_torch_autograd():
    """relu(GroupNorm(x)) and its gradients ("Optimize GroupNorm", fused-ReLU paragraphs)."""
    inp = workloads.make(workloads.custom(2, 8, 4, (6, 5, 7), torch.float32, dist="tiny", seed=41), "cpu")
    x, dy, G, eps = inp["x"], inp["dy"], inp["G"], inp["eps"]
    gamma, beta = inp["gamma"].numpy(), inp["beta"].numpy()
    f = O.forward(x, G, gamma, beta, eps=eps, relu=True)
    b = O.backward(dy, x, G, gamma, eps=eps, beta=beta, relu=True)
    y_t, dx_t, dg_t, db_t = _torch_relu_ref(_f64(x), G, gamma, beta, eps, _f64(dy))
    assert np.abs(f["y"] - y_t).max() <= 1e-12 * np.abs(y_t).max()
    assert (f["y"] >= 0).all() and (f["y"] == 0).mean() > 0.3   # the relu did something
    assert np.abs(b["dx"] - dx_t).max() <= 1e-10 * np.abs(dx_t).max()
    assert np.abs(b["dgamma"] - dg_t).max() <= 1e-10 * np.abs(dg_t).max()
    assert np.abs(b["dbeta"] - db_t).max() <= 1e-10 * np.abs(db_t).max()
    idx = np.arange(0, x.numel(), 7, dtype=np.int64)
    assert np.array_equal(O.forward_at(x, G, idx, f["mean"], f["rstd"], gamma, beta, relu=True),
                          f["y"].reshape(-1)[idx])
    assert np.array_equal(O.backward_at(dy, x, G, idx, b["mean"], b["rstd"], b["c1"], b["c2"], gamma,
                                        beta=beta, relu=True), b["dx"].reshape(-1)[idx])


def test_relu_keeps_negative_zero_and_nan_group_gradient():
    """The relu and its gate on special values against torch's F.relu and its autograd; then a
    NaN group, whose gradient passes the gate ("Optimize GroupNorm", NaN-correct ReLU paragraph)."""
    lib = O._load()
    vals = [-0.0, 0.0, float("nan"), float("inf"), float("-inf"), -1.5, 2.5, 1e-300, -1e-300]
    t = torch.tensor(vals, dtype=torch.float64, requires_grad=True)
    r = torch.relu(t)
    r.backward(torch.full_like(t, 3.0))
    for i, v in enumerate(vals):
        ours = lib.gno_relu_value(v)
        ref = float(r[i])
        assert (math.isnan(ours) and math.isnan(ref)) or (ours == ref and math.copysign(1, ours) == math.copysign(1, ref))
        assert lib.gno_gate_value(ours, 3.0) == float(t.grad[i])
    rng = np.random.default_rng(2)
    x = rng.normal(size=(2, 4, 12)).astype(np.float32)
    x[1, 2, 5] = np.nan
    dy = rng.normal(size=x.shape).astype(np.float32)
    gamma, beta = np.ones(4, np.float32), np.full(4, 0.1, np.float32)
    b = O.backward(dy, x, 2, gamma, eps=1e-5, beta=beta, relu=True)
    _, dx_t, dg_t, db_t = _torch_relu_ref(torch.from_numpy(x).to(torch.float64), 2, gamma, beta, 1e-5,
                                          torch.from_numpy(dy).to(torch.float64))
    assert np.isfinite(db_t).all() and np.allclose(b["dbeta"], db_t, rtol=1e-12)
    assert np.array_equal(np.isnan(b["dx"]), np.isnan(dx_t))
    assert np.array_equal(np.isnan(b["dgamma"]), np.isnan(dg_t))


# ----------------------------------------------------------------------------- gradient magnitudes

def _abs_sums_torch(x, dy, G, gamma, beta, eps, relu):
    """sum |g| and sum |g * xhat| per channel, entirely in torch float64: the statistics from
    torch's mean and biased var, and with relu the gradient that reaches the affine output
    taken from torch's autograd through relu."""
    N, C = x.shape[:2]
    x64, dy64 = x.to(torch.float64), dy.to(torch.float64)
    xg = x64.reshape(N, G, -1)
    mean = xg.mean(-1)
    rstd = 1.0 / torch.sqrt(xg.var(-1, unbiased=False) + float(np.float32(eps)))
    xhat = ((xg - mean[..., None]) * rstd[..., None]).reshape(x.shape)
    bshape = (1, C) + (1,) * (x.dim() - 2)
    g = dy64
    if relu:
        pre = (xhat * gamma.to(torch.float64).view(bshape) + beta.to(torch.float64).view(bshape))
        pre.requires_grad_(True)
        (g,) = torch.autograd.grad(torch.relu(pre), pre, dy64)
    dims = (0,) + tuple(range(2, x.dim()))
    return (g.abs().sum(dims).numpy(), (g * xhat).abs().sum(dims).numpy(), mean.numpy(), rstd.numpy(),
            float((g == 0).double().mean()))


@pytest.mark.parametrize("relu", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_channel_abs_sums_against_torch_autograd(dtype, relu):
    """The magnitudes that scale every dgamma/dbeta tolerance: per channel sum |g| and
    sum |g * xhat| over the samples and voxels, g = dy or the relu-gated dy. Checked against
    torch float64 with its own statistics (passed to the oracle as its mean/rstd inputs) and,
    with relu, torch autograd's gate; channels of one group and samples all differ."""
    case = workloads.custom(3, 12, 4, (5, 6, 7), dtype, dist="tiny", seed=77)
    inp = workloads.make(case, "cpu")
    x, dy, G, eps = inp["x"], inp["dy"], inp["G"], inp["eps"]
    gamma, beta = inp["gamma"], inp["beta"]
    ea, eb, mean, rstd, zero_frac = _abs_sums_torch(x, dy, G, gamma, beta, eps, relu)
    a, b = O.channel_abs_sums(dy, x, G, mean, rstd, gamma=gamma, beta=beta, relu=relu)
    assert a.shape == b.shape == (12,)
    assert np.allclose(a, ea, rtol=1e-12, atol=0.0)
    assert np.allclose(b, eb, rtol=1e-12, atol=0.0)
    # the gate did something, and every channel's magnitude is distinct
    assert (zero_frac > 0.2) if relu else (zero_frac == 0.0)
    assert len(set(np.round(a, 9))) == 12 and len(set(np.round(b, 9))) == 12
