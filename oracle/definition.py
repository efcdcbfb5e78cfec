"""Mode D: the guided denoising step written out as its definition, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).  Plain, slow and meant to
be checked by eye against the pages.  Pages cited:

* "12 · Samplers, schedulers and CFG" (ComfyUI guide, sampling chapter) --
  sections "sigma sequence", "denoise below 1", "core of CFG", "the cfg = 1
  optimisation", "calc_cond_batch()", "inpaint and mask", "data shapes of one
  sampling step".
* "10 · ModelPatcher and weight views" (ComfyUI guide, model-patcher chapter)
  -- section "strength_model and strength_patch" (the affine form
  W' = strength_model*W + strength_patch*dW, used here as an identity pin).
* The SGLang diffusion BCG write-up (zwxr.cn news 258547) -- sections 2 "BCG
  core mechanism" (bucket assignment snippet), 3 "bucket construction under
  tensor parallelism" (BucketPlan, split/combine, [uncond... | cond...]
  layout), 4 "debug chain" (scale 0 / 1 checks, norm logging, fp32 guidance),
  5 "performance and edge cases" (guidance curve shapes).

Readings taken where the pages are silent are stated at each function.  Pins
(tests/test_oracle_pins.py) tie every function here to closed forms, brute
force, special cases the pages fix or library routines.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

# --------------------------------------------------------------------------
# Storage rounding
# --------------------------------------------------------------------------


def round_bf16(x):
    """Round to the nearest bfloat16 value, ties to even, returned as float64.

    bfloat16 keeps 8 significant bits.  Writing x = m * 2**e with
    0.5 <= |m| < 1 (frexp), the nearest 8-bit significand is rint(m * 256)
    (numpy's rint rounds halves to even), so the rounded value is
    rint(m*256)/256 * 2**e.  Valid in bfloat16's normal range (every value of
    this path is far inside it); NaN and infinities pass through.
    The half-precision guidance passage (SGLang write-up section 4, stage 4:
    compute in fp32, cast back to the storage dtype) fixes the order: the
    state is computed wide and rounded on store.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def to_storage(x, dtype: str):
    """Value of ``x`` after a store in the storage dtype ("f32" or "bf16")."""
    if dtype == "f32":
        return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f64":
        return np.asarray(x, np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# a1: sigma schedule ("12 · Samplers...", sections "sigma sequence" and
# "denoise below 1")
# --------------------------------------------------------------------------


def base_steps(steps: int, denoise: float) -> int:
    """Length of the base schedule built for ``denoise`` < 1.

    The page says a longer base step count is built and its tail taken, but
    gives no formula.  Reading: the smallest N with N*denoise >= steps,
    i.e. ceil(steps/denoise) evaluated in float64; denoise = 1 gives steps.
    (The regional + inpaint workload fixes 34 base steps for 20 kept at 0.6,
    which a truncating int() would miss.)
    """
    if denoise >= 1.0:
        return steps
    return int(math.ceil(steps / denoise))


def sigma_schedule(sigma_max: float, sigma_min: float, steps: int,
                   denoise: float = 1.0):
    """Descending log-linear sigmas, a terminal 0, and the denoise tail.

    Base schedule of N = base_steps(steps, denoise) points, evenly spaced in
    log(sigma) from sigma_max to sigma_min (both endpoints exact), then 0.
    Keep the last steps+1 values.  Returned as float32 (the schedule is stored
    in float32), plus N.  Computed point by point with the C library's
    exp/log through ``math``.
    """
    N = base_steps(steps, denoise)
    la, lb = math.log(sigma_max), math.log(sigma_min)
    base = []
    for i in range(N):
        if i == 0:
            s = sigma_max
        elif i == N - 1:
            s = sigma_min
        else:
            s = math.exp(la + (lb - la) * (i / (N - 1)))
        base.append(s)
    base.append(0.0)
    sig = np.array(base[N - steps:], dtype=np.float64).astype(np.float32)
    return sig, N


def crop_sigmas(sig, start_step: int, last_step=None, force_full_denoise: bool = False):
    """Staged sampling on a schedule ("12 · Samplers...", section "denoise
    below 1": start_step and last_step crop the sequence further; section
    "force_full_denoise": when the cropped sequence does not end at 0, the
    option sets its last sigma to 0 so the output is fully denoised).

    Reading: steps start_step .. last_step-1 are kept, i.e. the sigmas at
    indices start_step .. last_step (last_step None, negative or beyond the
    end: to the end); the cropped sequence is the schedule from then on.
    """
    sig = np.asarray(sig, np.float32)
    end = len(sig) - 1
    last = end if last_step is None or last_step < 0 or last_step > end else int(last_step)
    if not 0 <= start_step <= last:
        raise ValueError((start_step, last))
    out = sig[start_step:last + 1].copy()
    if force_full_denoise and out[-1] != 0:
        out[-1] = np.float32(0.0)
    return out


# --------------------------------------------------------------------------
# a2: bucket plan (SGLang write-up sections 2 and 3)
# --------------------------------------------------------------------------


def bucket_id(t: int, steps: int, nb: int) -> int:
    """progress = t/steps; bucket = min(int(progress*nb), nb-1), in integers.

    The page writes the progress as a float; its floor is taken here exactly
    as floor(t*nb/steps) so the id is the one brute-force enumeration gives
    (a float64 product misplaces some (t, steps, nb), e.g. t=3, steps=11,
    nb=55).
    """
    return min((t * nb) // steps, nb - 1)


def bucket_id_bruteforce(t: int, steps: int, nb: int) -> int:
    """The unique b with b*steps <= t*nb < (b+1)*steps, clipped to nb-1."""
    for b in range(nb + t * nb // max(steps, 1) + 2):
        if b * steps <= t * nb < (b + 1) * steps:
            return min(b, nb - 1)
    raise AssertionError("no bucket")


def curve_value(kind: str, p0: float, p1: float, p2: float, u: float) -> float:
    """The continuous guidance curve at progress u in [0, 1] (float64).

    Section 5 of the write-up names three shapes: linear decay (e.g. 2.0 ->
    1.2), front-high (strong for the first 20% of progress, weak after) and
    mid-peak (guidance raised in the middle stage).  Reading for mid-peak,
    which the pages give no formula for: a triangle, p0 at both ends and p1
    at u = p2, linear on each side.
    """
    if kind == "const":
        return p0
    if kind == "linear":
        return p0 + (p1 - p0) * u
    if kind == "front_high":
        return p0 if u < p2 else p1
    if kind == "mid_peak":
        if not 0.0 < p2 < 1.0:
            raise ValueError(p2)
        return p0 + (p1 - p0) * (u / p2 if u <= p2 else (1.0 - u) / (1.0 - p2))
    raise ValueError(kind)


def bucket_table(kind: str, p0: float, p1: float, p2: float, nb: int):
    """Scale per bucket from a continuous guidance curve (float32 table).

    Section 2 of the write-up discretises a continuous curve into buckets,
    constant within a bucket.  Reading: bucket b samples the curve at
    u = b/(nb-1) (u = 0 when nb = 1), so a linear curve hits both end values
    exactly.
    """
    out = [curve_value(kind, p0, p1, p2, 0.0 if nb == 1 else b / (nb - 1)) for b in range(nb)]
    return np.array(out, dtype=np.float64).astype(np.float32)


def bucket_bounds(kind: str, p0: float, p1: float, p2: float, nb: int):
    """The curve at the edges of each bucket (float32 tables lo, hi).

    Section 2 of the write-up cuts the continuous curve at the bucket
    boundaries and, within a bucket, uses a constant or a simple linear
    interpolation.  Bucket b covers progress [b/nb, (b+1)/nb) (that is what
    bucket_id assigns), so its interpolation runs from the curve at b/nb to
    the curve at (b+1)/nb.
    """
    lo = [curve_value(kind, p0, p1, p2, b / nb) for b in range(nb)]
    hi = [curve_value(kind, p0, p1, p2, (b + 1) / nb) for b in range(nb)]
    return (np.array(lo, np.float64).astype(np.float32), np.array(hi, np.float64).astype(np.float32))


def interp_scale(t: int, steps: int, nb: int, lo, hi):
    """Within-bucket linear interpolation (write-up section 2): the fraction of
    the way through bucket b, f = (t*nb - b*steps)/steps, in float64, then
    lo[b] + (hi[b] - lo[b]) * f rounded to float32."""
    b = bucket_id(t, steps, nb)
    f = (t * nb - b * steps) / steps
    lo_b, hi_b = float(np.float32(lo[b])), float(np.float32(hi[b]))
    return np.float32(lo_b + (hi_b - lo_b) * f)


def area_box(frac, H: int, W: int):
    """Area fractions (fy, fx, fh, fw) -> half-open latent slice (y0, y1, x0, x1).

    "12 · Samplers...", calc_cond_batch(): area percentages are turned into
    latent slices.  The rounding is not stated.  Reading: each coordinate is
    the integer nearest to the exact product of the float64 fraction and the
    extent, a tie (an exact half) going to the larger integer; then the side
    is clamped to [1, extent] and the offset so that the box stays inside.
    The product is taken exactly (a float64 fraction is a dyadic rational), so
    the rule does not depend on how a float64 product would round.
    """
    def nearest_up(f, n):
        v = Fraction(float(f)) * n
        return math.floor(v + Fraction(1, 2))

    fy, fx, fh, fw = frac
    h = min(max(nearest_up(fh, H), 1), H)
    w = min(max(nearest_up(fw, W), 1), W)
    y0 = min(max(nearest_up(fy, H), 0), H - h)
    x0 = min(max(nearest_up(fx, W), 0), W - w)
    return (y0, y0 + h, x0, x0 + w)


def covers_frame(boxes, strengths, H: int, W: int) -> bool:
    """True when the boxes with positive strength cover every latent pixel."""
    cov = np.zeros((H, W), bool)
    for (y0, y1, x0, x1), s in zip(boxes, strengths):
        if s > 0:
            cov[y0:y1, x0:x1] = True
    return bool(cov.all())


def build_plan(t, steps: int, nb: int, table, override=None, covered=None, table_end=None):
    """Bucket plan of one step: ids, scales, skip set, layout and offsets.

    * bucket id per active sample (t in [0, steps)), scale = its override if
      given (not NaN) else table[bucket], or with ``table_end`` the
      within-bucket interpolation from table[bucket] to table_end[bucket]
      -- write-up sections 2, 4 (stage 1: re-bucketing each step with
      update_guidance_scales).
    * the uncond branch is skipped when the scale is exactly 1 and nothing
      forces it ("12 · Samplers...", section "the cfg = 1 optimisation");
      a sample whose regional conds leave pixels uncovered is forced to keep
      it (those pixels take the uncond prediction, see regional_cond).
    * layout [uncond rows | cond rows] (write-up section 3, layout fix).
      Reading: cond rows are the active samples stably ordered by
      (bucket, sample id); the uncond half is the same order with skipped
      samples removed (compacted).  bucket_offset / uncond_offset are the
      exclusive prefix sums of per-bucket row counts in each half
      (BucketPlan.bucket_offset).  Inactive samples get no rows.
    """
    t = np.asarray(t, np.int64)
    n = t.size
    table = np.asarray(table, np.float32)
    if override is None:
        override = np.full(n, np.nan, np.float32)
    override = np.asarray(override, np.float32)
    if covered is None:
        covered = np.ones(n, bool)
    bid = np.full(n, -1, np.int32)
    scale = np.zeros(n, np.float32)
    need_u = np.zeros(n, bool)
    active = (t >= 0) & (t < steps)
    for i in range(n):
        if not active[i]:
            continue
        b = bucket_id(int(t[i]), steps, nb)
        bid[i] = b
        if not np.isnan(override[i]):
            w = override[i]
        elif table_end is not None:
            w = interp_scale(int(t[i]), steps, nb, table, table_end)
        else:
            w = table[b]
        scale[i] = w
        need_u[i] = not (w == np.float32(1.0) and covered[i])
    order = sorted((int(bid[i]), i) for i in range(n) if active[i])
    order = np.array([i for _, i in order], np.int32)
    n_act = order.size
    uorder = np.array([i for i in order if need_u[i]], np.int32)
    m = uorder.size
    count = np.zeros(nb, np.int32)
    ucount = np.zeros(nb, np.int32)
    for i in order:
        count[bid[i]] += 1
        if need_u[i]:
            ucount[bid[i]] += 1
    offset = np.zeros(nb + 1, np.int32)
    uoffset = np.zeros(nb + 1, np.int32)
    for b in range(nb):
        offset[b + 1] = offset[b] + count[b]
        uoffset[b + 1] = uoffset[b] + ucount[b]
    cond_row = np.full(n, -1, np.int32)
    uncond_row = np.full(n, -1, np.int32)
    for pos, i in enumerate(order):
        cond_row[i] = m + pos
    for pos, i in enumerate(uorder):
        uncond_row[i] = pos
    return dict(bucket_id=bid, scale=scale, need_uncond=need_u, order=order,
                n_active=n_act, n_uncond=m, bucket_count=count,
                bucket_offset=offset, uncond_offset=uoffset,
                cond_row=cond_row, uncond_row=uncond_row)


# --------------------------------------------------------------------------
# a3: stand-in denoiser (closed form; the pages fix no network)
# --------------------------------------------------------------------------


def denoise(x, sigma: float, mu, s2: float):
    """Posterior mean of Gaussian data N(mu_c, s^2) seen through noise sigma.

    D(x, sigma) = (s^2 x + sigma^2 mu_c) / (s^2 + sigma^2), mu per channel
    (x is [C,H,W], mu is [C]).  This replaces model.apply_model
    ("12 · Samplers...", calc_cond_batch()).
    """
    x = np.asarray(x, np.float64)
    mu = np.asarray(mu, np.float64)[:, None, None]
    return (s2 * x + sigma * sigma * mu) / (s2 + sigma * sigma)


# --------------------------------------------------------------------------
# a4: regional conds ("12 · Samplers...", calc_cond_batch())
# --------------------------------------------------------------------------


def feather_1d(d, L: int, F: int):
    """Linear edge ramp of F pixels along one axis of a box of length L.

    The page lists mask and feathering handling per cond without the ramp
    shape.  Reading: weight (d+1)/F at the first
    pixel, rising by 1/F per pixel until it reaches 1, on both ends; 0 outside
    the box; F <= 0 means no feathering.
    """
    d = np.asarray(d, np.float64)
    inside = (d >= 0) & (d < L)
    if F <= 0:
        return inside.astype(np.float64)
    g = np.minimum(1.0, (d + 1.0) / F) * np.minimum(1.0, (L - d) / F)
    return np.where(inside, g, 0.0)


def region_weight(box, strength: float, H: int, W: int, F: int):
    """strength * feathered box mask, [H,W] float64 (separable in y and x)."""
    y0, y1, x0, x1 = box
    gy = feather_1d(np.arange(H) - y0, y1 - y0, F)
    gx = feather_1d(np.arange(W) - x0, x1 - x0, F)
    return float(strength) * gy[:, None] * gx[None, :]


def regional_cond(preds, weights, uncond):
    """Accumulate region predictions by weight and normalise by the weight sum.

    C(p) = sum_r w_r(p) * D_r(p) / sum_r w_r(p), summed in ascending r.
    Where no region has weight the pages leave the value open.  Reading:
    there is no conditional signal there, so the cond prediction is the
    uncond prediction (zero guidance at that pixel).
    """
    num = np.zeros_like(uncond, dtype=np.float64)
    den = np.zeros(uncond.shape[1:], np.float64)
    for P, w in zip(preds, weights):
        num = num + w[None] * P
        den = den + w
    safe = np.where(den > 0, den, 1.0)
    return np.where(den[None] > 0, num / safe[None], uncond)


# --------------------------------------------------------------------------
# a5, a6: guidance combine and inpaint blend
# --------------------------------------------------------------------------


def cfg_combine(u, c, w: float):
    """pred = uncond + cfg * (cond - uncond) ("12 · Samplers...", core of CFG).

    With cfg = 1 the result is the cond prediction itself (section "the cfg = 1
    optimisation"), returned exactly rather than through u + (c - u).
    """
    if w == 1.0:
        return np.array(c, np.float64, copy=True)
    return u + w * (c - u)


def inpaint_blend(pred, x_orig, mask):
    """mask*pred + (1-mask)*x_orig, mask [H,W] broadcast over channels.

    "12 · Samplers...", section "inpaint and mask": each step the unmasked
    region is blended with the original latent.  Reading: the blend is applied
    to the denoised prediction before the sampler update, at every model
    evaluation; mask 1 means "regenerate".
    """
    m = np.asarray(mask, np.float64)[None]
    return m * pred + (1.0 - m) * x_orig


# --------------------------------------------------------------------------
# a3-a7 for one sample
# --------------------------------------------------------------------------


class SampleParams:
    """Per-sample constants of the path (everything except x and t).
    ``regional``: the sample's cond is regional (default: it has regions);
    a regional sample none of whose regions is valid at a step keeps the
    regional rule, C = U everywhere."""

    def __init__(self, mu_u, mu_c, s2, regions=(), feather=0, H=0, W=0,
                 mask=None, x_orig=None, regional=None):
        self.mu_u = np.asarray(mu_u, np.float64)
        self.mu_c = np.asarray(mu_c, np.float64)
        self.s2 = float(s2)
        # regions: list of (box, strength, mu_r[C])
        self.regions = list(regions)
        self.regional = bool(self.regions) if regional is None else bool(regional)
        self.weights = [region_weight(b, s, H, W, feather) for b, s, _ in self.regions]
        self.mask = None if mask is None else np.asarray(mask, np.float64)
        self.x_orig = None if x_orig is None else np.asarray(x_orig, np.float64)


def guided_pred(x, sigma: float, w: float, prm: SampleParams):
    """The guided, blended prediction P(x, sigma) the sampler steps with."""
    u = denoise(x, sigma, prm.mu_u, prm.s2)
    if prm.regional:
        preds = [denoise(x, sigma, mu_r, prm.s2) for _, _, mu_r in prm.regions]
        c = regional_cond(preds, prm.weights, u)
    else:
        c = denoise(x, sigma, prm.mu_c, prm.s2)
    pred = cfg_combine(u, c, w)
    if prm.mask is not None:
        pred = inpaint_blend(pred, prm.x_orig, prm.mask)
    return pred


def step(x, sigma: float, sigma_next: float, w: float, prm: SampleParams,
         sampler: str):
    """One sampler step from sigma to sigma_next (float64).

    The pages give no update formula (they leave the update between
    neighbouring sigmas to the sampler, and note that some samplers evaluate
    the model more than once per step).  Euler and Heun are taken from Karras et al. 2022 (EDM), Alg. 1:
      d  = (x - P(x, sigma)) / sigma,  x' = x + (sigma' - sigma) d
      Heun: x~ = x + h d, d' = (x~ - P(x~, sigma')) / sigma',
            x' = x + h (d + d') / 2, with h = sigma' - sigma.
    The step to sigma' = 0 is the Euler step, which lands on P(x, sigma)
    exactly.
    """
    x = np.asarray(x, np.float64)
    sigma = float(sigma)
    sigma_next = float(sigma_next)
    P = guided_pred(x, sigma, w, prm)
    if sigma_next == 0.0:
        return P
    h = sigma_next - sigma
    d = (x - P) / sigma
    if sampler == "euler":
        return x + h * d
    if sampler == "heun":
        xt = x + h * d
        P2 = guided_pred(xt, sigma_next, w, prm)
        d2 = (xt - P2) / sigma_next
        return x + h * (d + d2) / 2.0
    raise ValueError(sampler)


# --------------------------------------------------------------------------
# Materialised branches: the model's outputs given as rows of the plan layout
# --------------------------------------------------------------------------


def rows_pred(rows, plan, i: int, w: float, x_orig=None, mask=None):
    """The guided, blended prediction of sample i from materialised branch
    outputs.

    ``rows`` is one model evaluation's output in the layout the plan defines
    (write-up section 3, [uncond_0..uncond_m | cond_0..cond_n]): sample i's
    cond prediction is row cond_row[i], its uncond prediction row
    uncond_row[i] (absent when the uncond branch was skipped).  Reading: the
    cond row already holds the regionally accumulated cond ("12 ·
    Samplers...", "calc_cond_batch()"; area_accumulate builds it, with the
    uncond prediction where no region has weight), so with w == 1 the
    prediction is that row itself and no uncond row is used (section "the
    cfg = 1 optimisation").
    """
    c = np.asarray(rows[plan["cond_row"][i]], np.float64)
    if w == 1.0:
        pred = c.copy()
    else:
        pred = cfg_combine(np.asarray(rows[plan["uncond_row"][i]], np.float64), c, w)
    if mask is not None:
        pred = inpaint_blend(pred, x_orig, mask)
    return pred


def euler_from_pred(x, P, sigma: float, sigma_next: float):
    """Euler step given the prediction P at (x, sigma) (Karras et al. 2022,
    Alg. 1); the step to sigma' = 0 lands on P."""
    if sigma_next == 0.0:
        return np.array(P, np.float64, copy=True)
    return x + (sigma_next - sigma) * (x - P) / sigma


def heun_predict(x, P, sigma: float, sigma_next: float):
    """First call of a Heun step whose model evaluations are materialised:
    returns (d, x~) with d = (x - P)/sigma and x~ = x + h d, the point the
    model is evaluated at next.  On the last step (sigma' = 0) the step is
    Euler's and lands on P: returns (None, P)."""
    if sigma_next == 0.0:
        return None, np.array(P, np.float64, copy=True)
    d = (x - P) / sigma
    return d, x + (sigma_next - sigma) * d


def heun_correct(x, d, P2, sigma: float, sigma_next: float):
    """Second call: with P2 the prediction at (x~, sigma'), the slopes are
    averaged, x' = x + h (d + d')/2, d' = (x~ - P2)/sigma'."""
    h = sigma_next - sigma
    xt = x + h * d
    d2 = (xt - P2) / sigma_next
    return x + h * (d + d2) / 2.0


def norm_stats(x, sigma: float, w: float, prm: SampleParams, need_uncond: bool):
    """Per-sample norm check before/after guidance.

    SGLang write-up section 4 logs hidden_states.norm(dim=-1).mean() before and
    after apply_guidance.  Reading: per sample, the mean over (channel, row)
    of the L2 norm over the last (width) axis, for the cond prediction C, the
    uncond prediction U (0 when its branch is skipped) and the guided pred
    (before the inpaint blend), from the evaluation at (x, sigma).
    """
    u = denoise(x, sigma, prm.mu_u, prm.s2)
    if prm.regional:
        preds = [denoise(x, sigma, mu_r, prm.s2) for _, _, mu_r in prm.regions]
        c = regional_cond(preds, prm.weights, u)
    else:
        c = denoise(x, sigma, prm.mu_c, prm.s2)
    pred = cfg_combine(u, c, w)
    nrm = lambda v: float(np.sqrt((v * v).sum(axis=-1)).mean())
    return np.array([nrm(c), nrm(u) if need_uncond else 0.0, nrm(pred)])


# --------------------------------------------------------------------------
# Whole trajectory
# --------------------------------------------------------------------------


def region_valid(rng, t: int, steps: int) -> bool:
    """Whether a regional cond takes part in step t ("12 · Samplers...",
    "calc_cond_batch()": each cond entry is checked for the current timestep
    being valid).  Reading: a cond carries a range [start, end) of sampling
    progress, the progress of step t being t/steps (float64, as for the
    buckets); outside its range the cond contributes nothing."""
    if rng is None:
        return True
    p = t / steps
    return bool(rng[0] <= p < rng[1])


def valid_regions(inp, i: int, t=None):
    """Indices of sample i's regions that take part in step t (all if t is None)."""
    k = int(inp.region_count[i])
    if t is None or inp.region_range is None:
        return list(range(k))
    return [r for r in range(k) if region_valid(inp.region_range[i, r], int(t), inp.spec.steps)]


def sample_params(inp, i: int, t=None):
    """SampleParams of sample i from a ``workloads.Inputs`` (at step t when the
    regions have validity ranges)."""
    sp = inp.spec
    regions = []
    for r in valid_regions(inp, i, t):
        box = area_box(inp.region_frac[i, r], sp.H, sp.W)
        regions.append((box, float(inp.region_strength[i, r]), inp.mu_region[i, r]))
    return SampleParams(inp.mu_uncond[i], inp.mu_cond[i], sp.s2, regions,
                        sp.feather, sp.H, sp.W,
                        None if inp.mask is None else inp.mask[i, 0],
                        None if inp.x_orig is None else stored_orig(inp)[i],
                        regional=int(inp.region_count[i]) > 0)


def stored_orig(inp):
    """The original latent as held by the path: in the storage dtype, like every
    latent of the step (reading: the inpaint source latent is stored the same
    way as the state it is blended into)."""
    return to_storage(inp.x_orig, inp.spec.dtype)


def covered_at(inp, i: int, t=None) -> bool:
    """Whether sample i's regions valid at step t (all of them if t is None)
    cover the frame; a sample without regions is covered."""
    sp = inp.spec
    if int(inp.region_count[i]) == 0:
        return True
    rs = valid_regions(inp, i, t)
    boxes = [area_box(inp.region_frac[i, r], sp.H, sp.W) for r in rs]
    return bool(covers_frame(boxes, inp.region_strength[i, rs], sp.H, sp.W))


def coverage(inp, t=None):
    """Per-sample full-coverage flag (samples without regions are covered); with
    validity ranges, of the regions valid at each sample's step t[i]."""
    return np.array([covered_at(inp, i, None if t is None else t[i]) for i in range(inp.spec.n)], bool)


def run_setup(inp):
    """Schedule, bucket table, coverage and per-sample params of a workload.
    With within-bucket interpolation the table is the bucket-start values
    (bucket_bounds) and table_end(inp) gives the bucket-end values."""
    sp = inp.spec
    sig, _ = sigma_schedule(sp.sigma_max, sp.sigma_min, sp.steps, sp.denoise)
    c = sp.curve
    if sp.bucket_interp:
        table = bucket_bounds(c.kind, c.p0, c.p1, c.p2, sp.num_buckets)[0]
    else:
        table = bucket_table(c.kind, c.p0, c.p1, c.p2, sp.num_buckets)
    return sig, table, coverage(inp)


def table_end(inp):
    """The bucket-end values when the workload interpolates within buckets."""
    sp = inp.spec
    if not sp.bucket_interp:
        return None
    c = sp.curve
    return bucket_bounds(c.kind, c.p0, c.p1, c.p2, sp.num_buckets)[1]


def init_latent(inp, sig, storage: str):
    """x = latent + noise * sigma[start] per sample, stored in the storage dtype.

    "12 · Samplers...", section "disable_noise": a latent input still follows
    the sigma trajectory, so the start is the latent plus noise at the first
    sigma of the sample.  The latent is the original latent when inpainting,
    zero otherwise.  Reading for mixed progress: sample i joins at its own
    start step with noise at that level.
    """
    sp = inp.spec
    x = np.asarray(inp.noise, np.float64) * sig.astype(np.float64)[
        inp.start_step][:, None, None, None]
    if inp.x_orig is not None:
        x = stored_orig(inp) + x
    return to_storage(x, storage)


def trajectory(inp, storage: str | None = None, launches: int | None = None,
               samples=None, keep=False):
    """Run the sampler loop in mode D.

    Launch k moves every active sample i (t_i = start_i + k < steps) one step.
    The state is stored in the workload's storage dtype after every step
    (``storage`` overrides it, "f64" keeps it unrounded).  Returns the final
    state [n,C,H,W] (float64 values), and the list of states if ``keep``.
    """
    sp = inp.spec
    storage = storage or sp.dtype
    sig, table, cov = run_setup(inp)
    sig64 = sig.astype(np.float64)
    idx = range(sp.n) if samples is None else samples
    prms = {i: sample_params(inp, i) for i in idx}
    x = init_latent(inp, sig, storage)
    states = [x.copy()] if keep else None
    L = sp.steps if launches is None else launches
    ranged = inp.region_range is not None
    for k in range(L):
        t = inp.start_step.astype(np.int64) + k
        plan = build_plan(t, sp.steps, sp.num_buckets, table, inp.cfg_override,
                          coverage(inp, t) if ranged else cov, table_end(inp))
        for i in idx:
            if plan["bucket_id"][i] < 0:
                continue
            ti = int(t[i])
            prm = sample_params(inp, i, ti) if ranged else prms[i]
            x[i] = to_storage(step(x[i], sig64[ti], sig64[ti + 1],
                                   float(plan["scale"][i]), prm, sp.sampler),
                              storage)
        if keep:
            states.append(x.copy())
    return (x, states) if keep else x


# --------------------------------------------------------------------------
# Continuous batching: slots refilled from a queue of requests
# --------------------------------------------------------------------------


def serve_schedule(start, steps: int, n_slots: int, n_requests: int, launches: int, ring: bool = False):
    """Which request each slot of a continuously batched loop holds at each
    launch, the step it takes there, and whether it joins at that launch.

    SGLang write-up section 3 (one batch carries samples of several buckets)
    and section 4 stage 3 (the scheduler builds each step's plan; samples move
    between buckets from step to step).  The pages describe the mixed batch,
    not how it is refilled.  Reading: slots 0..n_slots-1 begin with requests
    0..n_slots-1 at their start steps (each in [0, steps)); a request takes
    one step per launch; after the launch in which a request takes its last
    step, its slot takes the next request of the queue at the next launch
    (the freed slots in index order take the queued requests in id order),
    and that request joins at step 0 from its own noise; once the queue is
    exhausted a freed slot stays empty.  With ``ring`` the queue never ends:
    request ids run modulo n_requests (a fixed pool served over and over).

    Returns int arrays req[launches, n_slots] and t[launches, n_slots] (-1 in
    both where the slot is empty) and a bool array join[launches, n_slots]
    (the request's state is initialised before its step at that launch; every
    initial request joins at launch 0).
    """
    start = np.asarray(start, np.int64)
    if n_requests < n_slots:
        raise ValueError("fewer requests than slots")
    if ((start[:n_slots] < 0) | (start[:n_slots] >= steps)).any():
        raise ValueError("initial start steps must lie in [0, steps)")
    req = np.full((launches, n_slots), -1, np.int64)
    tt = np.full((launches, n_slots), -1, np.int64)
    join = np.zeros((launches, n_slots), bool)
    cur_r = np.arange(n_slots, dtype=np.int64)
    cur_t = start[:n_slots].copy()
    cur_j = np.ones(n_slots, bool)
    nxt = n_slots
    for k in range(launches):
        if k > 0:
            for s in range(n_slots):
                if cur_r[s] < 0 or cur_t[s] >= steps:  # empty, or its request has finished
                    if ring or nxt < n_requests:
                        cur_r[s] = nxt % n_requests if ring else nxt
                        cur_t[s] = 0
                        cur_j[s] = True
                        nxt += 1
                    else:
                        cur_r[s] = -1
                        cur_t[s] = -1
        req[k], tt[k], join[k] = cur_r, cur_t, cur_j
        for s in range(n_slots):
            if cur_r[s] >= 0:
                cur_t[s] += 1
                cur_j[s] = False
    return req, tt, join


def init_sample(inp, i: int, sigma: float, storage: str):
    """Request i's state when it joins at noise level sigma: its latent (the
    original latent when inpainting, else zero) plus its noise times sigma,
    stored in the storage dtype (the rule of init_latent for one sample)."""
    x = np.asarray(inp.noise[i], np.float64) * float(sigma)
    if inp.x_orig is not None:
        x = stored_orig(inp)[i] + x
    return to_storage(x, storage)


def serve_trajectory(inp, n_slots: int, launches: int, ring: bool = False, slots=None, keep=False):
    """Mode D of a continuously batched loop over the request pool ``inp``
    (inp.spec.n requests; the first n_slots' start steps are the initial
    progress): at each launch the plan of the slots' steps (each slot with its
    request's override and coverage), then every active slot in ``slots``
    (default all) takes its step, after joining if it joins there.  Returns
    the final slot states and, with ``keep``, the state after every launch,
    plus the schedule.  With validity ranges ([S] "calc_cond_batch()": a cond
    takes part while the current timestep is in its range) a request's
    regions, and so its coverage, follow its own progress: the reading is
    that serving a request changes nothing of its own trajectory."""
    sp = inp.spec
    ranged = inp.region_range is not None
    sig, table, cov = run_setup(inp)
    sig64 = sig.astype(np.float64)
    req, tt, join = serve_schedule(inp.start_step, sp.steps, n_slots, sp.n, launches, ring)
    x = np.zeros((n_slots, sp.C, sp.H, sp.W))
    states = []
    idx = range(n_slots) if slots is None else slots
    ov = np.asarray(inp.cfg_override, np.float32)
    for k in range(launches):
        r = req[k]
        ovk = np.where(r >= 0, ov[np.maximum(r, 0)], np.float32(np.nan)).astype(np.float32)
        if ranged:
            covk = np.array([r[s] < 0 or covered_at(inp, int(r[s]), int(tt[k, s])) for s in range(n_slots)])
        else:
            covk = cov[np.maximum(r, 0)]
        plan = build_plan(tt[k], sp.steps, sp.num_buckets, table, ovk, covk, table_end(inp))
        for s in idx:
            if r[s] < 0 or plan["bucket_id"][s] < 0:
                continue
            ti = int(tt[k, s])
            if join[k, s]:
                x[s] = init_sample(inp, int(r[s]), sig64[ti], sp.dtype)
            x[s] = to_storage(step(x[s], sig64[ti], sig64[ti + 1], float(plan["scale"][s]),
                                   sample_params(inp, int(r[s]), ti if ranged else None), sp.sampler),
                              sp.dtype)
        if keep:
            states.append(x.copy())
    return x, states, (req, tt, join)


def pf_ode_exact(x, sigma: float, sigma_next: float, mean, s2: float):
    """Exact probability-flow solution for Gaussian data N(mean, s^2).

    With D(x, sigma) = (s^2 x + sigma^2 mean)/(s^2 + sigma^2) the ODE
    dx/dsigma = (x - D)/sigma = (x - mean) sigma/(s^2 + sigma^2) integrates to
    x(sigma') = mean + (x - mean) sqrt((s^2 + sigma'^2)/(s^2 + sigma^2)).
    """
    return mean + (x - mean) * math.sqrt((s2 + sigma_next ** 2) / (s2 + sigma ** 2))
