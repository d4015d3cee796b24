"""Seeded synthetic GroupNorm inputs shaped like the UNet sites of the pages.

This module only draws numbers: it holds none of GroupNorm's arithmetic, and both
the GPU path and the CPU oracle receive exactly the tensors it returns.

Recipes (per-channel parameters are drawn first, then gamma, then beta with a numpy
PCG64 stream; the two volumes, x then dy, are drawn with a torch generator on the
requested device so that 256^3 volumes are generated in place):

- ``tiny``: N=1, C=8, G=4, 16^3, fp32. x = mu_c + sigma_c * z with
  mu_c ~ U(-2, 2), sigma_c ~ U(0.5, 2). dy ~ N(0, 1) fp32.
- ``unet`` (the 128^3 and 256^3 top-level sites): x = s_c * z + o_c with
  s_c ~ U(0.5, 2), o_c ~ U(-1, 1), rounded to bf16; dy ~ N(0, sigma=1e-2) bf16.
- ``deep``: x = 100 + z in bf16 (large offset, unit spread: the cancellation case);
  dy ~ N(0, 1) bf16.
- ``normal``: z ~ N(0, 1) for both x and dy (the whole-UNet census sites).

dy has zero mean in every recipe above, so each channel's sums of dy and dy * xhat
cancel to about sqrt(S) of their terms' size. A case with ``dy_mode="offset"`` instead
draws dy = sigma * (u_c + z' + v_c * z), with per-channel u_c ~ U(1, 2) and v_c ~ U(4, 6)
drawn after beta, z' a fresh N(0, 1) draw and z the standard normal draw that x was made
from. Both channel sums then grow with S instead of cancelling: dbeta_c ~ sigma * u_c * S,
and dgamma_c ~ sigma * S * (v_c * s_c + u_c * (o_c - mu_g)) / sigma_g, where v_c * s_c >= 2
outweighs the channel offset term (|o_c - mu_g| < 2); so the parameter gradients can be
held to a relative bar that means something.

In every recipe gamma ~ N(1, 0.1), beta ~ N(0, 0.1) in fp32 and eps = 1e-5.
Values are drawn in fp32 and rounded once (nearest-even) to bf16 or fp16 where the
case asks for a 16-bit dtype. The pages' real activations come from a trained UNet on a fractal
dataset that is not available here; these draws stand in for them.
"""
from dataclasses import dataclass, field
from typing import Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Case:
    name: str
    N: int
    C: int
    G: int
    spatial: Tuple[int, ...]
    x_dtype: torch.dtype
    dy_dtype: torch.dtype
    dist: str
    seed: int
    out_dtype: torch.dtype = None  # None: the input's dtype
    eps: float = 1e-5
    tags: Tuple[str, ...] = field(default_factory=tuple)
    dy_mode: str = "zero_mean"  # or "offset": channel sums of dy and dy * xhat that do not cancel

    @property
    def S(self) -> int:
        return int(np.prod(self.spatial))

    @property
    def numel(self) -> int:
        return self.N * self.C * self.S

    @property
    def shape(self):
        return (self.N, self.C) + tuple(self.spatial)


BF16, F16, F32 = torch.bfloat16, torch.float16, torch.float32

# The workloads named by the pages' UNet (sizes and distributions as listed above).
TINY = Case("tiny_fp32_16cube", 1, 8, 4, (16, 16, 16), F32, F32, "tiny", 1001)
SCALE7 = Case("scale7_128cube_c32_g8", 1, 32, 8, (128, 128, 128), BF16, BF16, "unet", 1007)
SCALE8 = Case("scale8_256cube_c32_g8", 1, 32, 8, (256, 256, 256), BF16, BF16, "unet", 1008)
DEEP = Case("deep_n4_c512_g32_8cube", 4, 512, 32, (8, 8, 8), BF16, BF16, "deep", 1004)
# The 128^3 site with fp16 activations (the pages list fp16 among the input dtypes).
SCALE7_F16 = Case("scale7_128cube_c32_g8_fp16", 1, 32, 8, (128, 128, 128), F16, F16, "unet", 1017)
# The two top-level sites with a dy whose channel sums do not cancel (dy_mode "offset").
SCALE7_DY_OFFSET = Case("scale7_128cube_c32_g8_dy_offset", 1, 32, 8, (128, 128, 128), BF16, BF16, "unet", 1027,
                        dy_mode="offset")
SCALE8_DY_OFFSET = Case("scale8_256cube_c32_g8_dy_offset", 1, 32, 8, (256, 256, 256), BF16, BF16, "unet", 1028,
                        dy_mode="offset")
# fp32-output mode: y in fp32, dy arrives in fp32 (holding bf16-representable values).
DEEP_F32OUT = Case("deep_n4_c512_g32_8cube_f32out", 4, 512, 32, (8, 8, 8), BF16, F32, "deep", 1004,
                   out_dtype=F32)


def census_cases():
    """The 18 GroupNorm sites of a 5-level scale-7 UNet.

    Two sites per encoder level and two per decoder level at levels 1-4, two at the
    bottom level 5. GroupNorm follows each convolution, so a decoder site normalizes
    the level's own channel count (the 2x concatenated channels are the
    convolution's input, not GroupNorm's).
    """
    levels = [(32, 8, 128, 4), (64, 8, 64, 4), (128, 16, 32, 4), (256, 32, 16, 4), (512, 32, 8, 2)]
    out, site = [], 0
    for C, G, d, count in levels:
        for _ in range(count):
            out.append(Case(f"census_site{site:02d}_c{C}_g{G}_{d}cube", 1, C, G, (d, d, d),
                            BF16, BF16, "normal", 1100 + site))
            site += 1
    return out


def _channel_params(rng: np.random.Generator, case: Case):
    C = case.C
    if case.dist == "tiny":
        mu = rng.uniform(-2.0, 2.0, C)
        sigma = rng.uniform(0.5, 2.0, C)
        return sigma, mu
    if case.dist == "unet":
        s = rng.uniform(0.5, 2.0, C)
        o = rng.uniform(-1.0, 1.0, C)
        return s, o
    if case.dist == "deep":
        return np.ones(C), np.full(C, 100.0)
    if case.dist == "normal":
        return np.ones(C), np.zeros(C)
    raise ValueError(case.dist)


def _dy_sigma(case: Case) -> float:
    return 1e-2 if case.dist == "unet" else 1.0


def make(case: Case, device="cpu", with_dy=True):
    """Returns dict(x, gamma, beta, dy, G, eps, out_dtype) with x/dy on ``device``."""
    rng = np.random.Generator(np.random.PCG64(case.seed))
    scale, offset = _channel_params(rng, case)
    gamma = rng.normal(1.0, 0.1, case.C).astype(np.float32)
    beta = rng.normal(0.0, 0.1, case.C).astype(np.float32)
    if case.dy_mode not in ("zero_mean", "offset"):
        raise ValueError(case.dy_mode)
    if case.dy_mode == "offset":
        u = rng.uniform(1.0, 2.0, case.C)
        v = rng.uniform(4.0, 6.0, case.C)

    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(case.seed)
    shape = case.shape
    bshape = (1, case.C) + (1,) * len(case.spatial)
    sc = torch.tensor(scale, dtype=torch.float32, device=dev).view(bshape)
    of = torch.tensor(offset, dtype=torch.float32, device=dev).view(bshape)
    z = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
    x = (z * sc).add_(of).to(case.x_dtype)
    dy = None
    if with_dy:
        dy = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
        if case.dy_mode == "offset":
            uc = torch.tensor(u, dtype=torch.float32, device=dev).view(bshape)
            vc = torch.tensor(v, dtype=torch.float32, device=dev).view(bshape)
            dy.add_(uc).add_(z.mul_(vc))
        del z
        dy.mul_(_dy_sigma(case))
        # dy carries the output's values; in the fp32-output mode it holds values of x's
        # 16-bit dtype stored as fp32, so that both dy dtypes describe the same numbers.
        dy = dy.to(case.x_dtype if case.x_dtype in (BF16, F16) else F32).to(case.dy_dtype)
    return {
        "x": x,
        "gamma": torch.from_numpy(gamma).to(dev),
        "beta": torch.from_numpy(beta).to(dev),
        "dy": dy,
        "G": case.G,
        "eps": case.eps,
        "out_dtype": case.out_dtype or case.x_dtype,
    }


def custom(N, C, G, spatial, x_dtype=BF16, dy_dtype=None, dist="normal", seed=0, out_dtype=None,
           dy_mode="zero_mean"):
    """A Case for an arbitrary test shape (ragged sizes, edge cases)."""
    return Case(f"custom_n{N}_c{C}_g{G}_{'x'.join(map(str, spatial))}", N, C, G, tuple(spatial),
                x_dtype, dy_dtype or (out_dtype or x_dtype), dist, seed, out_dtype=out_dtype, dy_mode=dy_mode)
