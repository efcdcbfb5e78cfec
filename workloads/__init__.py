"""Seeded synthetic inputs for the guided denoising step.

This module draws random numbers and nothing else: no part of the method's
arithmetic (schedules, bucket tables, area slices, feathering, the stand-in
denoiser, guidance, blending, sampler updates, storage rounding) lives here.
Both the CPU oracle and the HIP path are fed from it.

Workload shapes follow the five synthetic configurations of the task: a tiny
smoke case, a mixed-bucket batch, a bf16 Heun throughput batch, a regional +
inpaint batch and a large bf16 batch.  The latent geometry (4 channels,
128x128) is the SDXL-style 1024x1024 image divided by a VAE factor of 8, the
example the sampling page of the ComfyUI guide gives when it says the latent is
the pixel size divided by the VAE scale ("one step's data shapes").

Draw order per spec (fixed, so a seed reproduces every array):
  noise -> mu_uncond -> mu_cond -> start_step -> override sample set ->
  region fractions -> region strengths -> region means -> ellipse -> x_orig
Every draw is float64 from numpy's PCG64 ``default_rng(seed)`` and is rounded
to float32 once.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Spec", "Inputs", "CONFIGS", "config", "make_inputs", "small_spec"]


@dataclass(frozen=True)
class Curve:
    """Guidance curve description: kind in {"const", "linear", "front_high", "mid_peak"}.

    const:      value = p0
    linear:     from p0 at progress 0 to p1 at progress 1
    front_high: p0 for the first ``p2`` fraction of progress, p1 after
    mid_peak:   p0 at both ends, p1 at progress ``p2``
    """
    kind: str
    p0: float
    p1: float = 0.0
    p2: float = 0.0


@dataclass(frozen=True)
class Spec:
    name: str
    n: int
    C: int
    H: int
    W: int
    dtype: str                 # "f32" or "bf16" storage
    sampler: str               # "euler" or "heun"
    steps: int                 # sampler steps actually taken
    num_buckets: int
    curve: Curve
    sigma_max: float = 14.6
    sigma_min: float = 0.03
    denoise: float = 1.0
    s2: float = 0.25           # stand-in data variance s^2 (s = 0.5)
    mixed_start: bool = False  # per-sample uniform start step in [0, steps)
    shared_mu: bool = False    # one [C] row of means shared by every sample
    skip_frac: float = 0.0     # fraction of samples with a cfg override of 1.0
    regions: int = 0           # regional conds per sample
    feather: int = 8
    region_lo: float = 0.2     # box side as a fraction of the latent side
    region_hi: float = 0.8
    inpaint: bool = False      # ellipse denoise mask + original latent
    seed: int = 0
    bucket_interp: bool = False  # scale interpolated within each bucket
    region_ranges: bool = False  # each regional cond valid over a range of progress only


@dataclass
class Inputs:
    spec: Spec
    noise: np.ndarray                 # f32 [n,C,H,W]
    mu_uncond: np.ndarray             # f32 [n,C]
    mu_cond: np.ndarray               # f32 [n,C]
    start_step: np.ndarray            # i32 [n]
    cfg_override: np.ndarray          # f32 [n], NaN = no override
    region_count: np.ndarray          # i32 [n]
    region_frac: np.ndarray           # f64 [n,R,4] (fy, fx, fh, fw), R = max(regions, 1)
    region_strength: np.ndarray       # f32 [n,R]
    mu_region: np.ndarray             # f32 [n,R,C]
    mask: np.ndarray | None           # f32 [n,1,H,W] binary, or None
    x_orig: np.ndarray | None         # f32 [n,C,H,W], or None
    region_range: np.ndarray | None = None  # f64 [n,R,2] (start, end) progress, or None

    def subset(self, idx) -> "Inputs":
        """Inputs restricted to the samples ``idx`` (per-sample independence)."""
        idx = np.asarray(idx, dtype=np.int64)
        sp = dataclasses.replace(self.spec, n=int(idx.size))
        take = lambda a: None if a is None else np.ascontiguousarray(a[idx])
        return Inputs(sp, take(self.noise), take(self.mu_uncond), take(self.mu_cond),
                      take(self.start_step), take(self.cfg_override),
                      take(self.region_count), take(self.region_frac),
                      take(self.region_strength), take(self.mu_region),
                      take(self.mask), take(self.x_orig), take(self.region_range))


def _f32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def make_inputs(spec: Spec, samples=None) -> Inputs:
    """Draw every input of ``spec`` from ``default_rng(spec.seed)``.

    ``samples`` (optional) keeps only those sample indices; the draws are made
    for the whole batch first so a subset is bit-identical to the same rows of
    the full batch.
    """
    n, C, H, W = spec.n, spec.C, spec.H, spec.W
    rng = np.random.default_rng(spec.seed)
    noise = _f32(rng.standard_normal((n, C, H, W)))
    if spec.shared_mu:
        mu_u = np.broadcast_to(_f32(rng.standard_normal(C)), (n, C)).copy()
        mu_c = np.broadcast_to(_f32(rng.standard_normal(C)), (n, C)).copy()
    else:
        mu_u = _f32(rng.standard_normal((n, C)))
        mu_c = _f32(rng.standard_normal((n, C)))
    if spec.mixed_start:
        start = rng.integers(0, spec.steps, size=n).astype(np.int32)
    else:
        start = np.zeros(n, np.int32)
    override = np.full(n, np.nan, np.float32)
    k = int(round(spec.skip_frac * n))
    if k > 0:
        override[rng.permutation(n)[:k]] = 1.0
    R = max(spec.regions, 1)
    frac = np.zeros((n, R, 4), np.float64)
    strength = np.zeros((n, R), np.float32)
    mu_r = np.zeros((n, R, C), np.float32)
    count = np.full(n, spec.regions, np.int32)
    if spec.regions > 0:
        fh = rng.uniform(spec.region_lo, spec.region_hi, size=(n, R))
        fw = rng.uniform(spec.region_lo, spec.region_hi, size=(n, R))
        fy = rng.uniform(0.0, 1.0, size=(n, R)) * (1.0 - fh)
        fx = rng.uniform(0.0, 1.0, size=(n, R)) * (1.0 - fw)
        frac = np.stack([fy, fx, fh, fw], axis=-1)
        strength = _f32(rng.uniform(0.5, 1.5, size=(n, R)))
        mu_r = _f32(rng.standard_normal((n, R, C)))
    mask = x_orig = None
    if spec.inpaint:
        cy = rng.uniform(0.25, 0.75, size=n) * H
        cx = rng.uniform(0.25, 0.75, size=n) * W
        ay = rng.uniform(0.15, 0.35, size=n) * H
        ax = rng.uniform(0.15, 0.35, size=n) * W
        yy = np.arange(H, dtype=np.float64)[None, :, None] + 0.5
        xx = np.arange(W, dtype=np.float64)[None, None, :] + 0.5
        inside = (((yy - cy[:, None, None]) / ay[:, None, None]) ** 2
                  + ((xx - cx[:, None, None]) / ax[:, None, None]) ** 2) <= 1.0
        mask = inside.astype(np.float32)[:, None, :, :]
        x_orig = _f32(rng.standard_normal((n, C, H, W)))
    rng_ = None
    if spec.region_ranges and spec.regions > 0:  # drawn last: the other inputs do not change
        lo = rng.uniform(0.0, 0.6, size=(n, R))
        rng_ = np.stack([lo, lo + rng.uniform(0.2, 1.0, size=(n, R))], axis=-1)
    inp = Inputs(spec, noise, mu_u, mu_c, start, override, count, frac, strength,
                 mu_r, mask, x_orig, rng_)
    return inp if samples is None else inp.subset(samples)


def _cfgs():
    lin = Curve("linear", 2.0, 1.2)
    return {
        "tiny": Spec("tiny", 2, 4, 32, 32, "f32", "euler", 10, 1, Curve("const", 7.0),
                     shared_mu=True, seed=20261201),
        "mixed_bucket": Spec("mixed_bucket", 8, 4, 128, 128, "f32", "euler", 50, 8, lin,
                             mixed_start=True, seed=20261202),
        "throughput_bf16_heun": Spec("throughput_bf16_heun", 64, 4, 128, 128, "bf16", "heun",
                                     30, 16, Curve("front_high", 2.0, 1.2, 0.2),
                                     skip_frac=0.25, seed=20261203),
        "regional_inpaint": Spec("regional_inpaint", 16, 4, 128, 128, "f32", "euler", 20, 8,
                                 lin, denoise=0.6, regions=3, inpaint=True, seed=20261204),
        "large_bf16": Spec("large_bf16", 256, 16, 128, 128, "bf16", "euler", 50, 8, lin,
                           mixed_start=True, regions=2, seed=20261205),
    }


CONFIGS = _cfgs()
CONFIG_ORDER = ["tiny", "mixed_bucket", "throughput_bf16_heun", "regional_inpaint", "large_bf16"]


def config(name: str) -> Spec:
    return CONFIGS[name]


def small_spec(name="small", *, n=3, C=3, H=17, W=40, dtype="f32", sampler="euler",
               steps=6, num_buckets=3, curve=None, regions=0, inpaint=False,
               mixed_start=True, skip_frac=0.34, feather=3, denoise=1.0, seed=7,
               region_lo=0.2, region_hi=0.8, shared_mu=False, bucket_interp=False,
               region_ranges=False) -> Spec:
    """A small shape for parity tests (several tiles, ragged tails)."""
    return Spec(name, n, C, H, W, dtype, sampler, steps, num_buckets,
                curve or Curve("linear", 2.0, 1.2), denoise=denoise,
                mixed_start=mixed_start, skip_frac=skip_frac, regions=regions,
                feather=feather, inpaint=inpaint, seed=seed, region_lo=region_lo,
                region_hi=region_hi, shared_mu=shared_mu, bucket_interp=bucket_interp,
                region_ranges=region_ranges)
