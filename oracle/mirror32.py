"""Mode M: the guided step as a fixed sequence of IEEE float32 operations.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Why this mode exists: with bf16 storage the stored state is an 8-bit
significand code chosen from a float32 result.  For |x| >= 4 one bf16 ulp is
0.03125, above the 2e-2 final-latent bound, so the expected code has to be
decided in the same precision and order as the device decides it: every
operation below is one correctly rounded float32 operation (numpy float32
arithmetic; division correctly rounded; fma(a, b, c) is IEEE 754
fusedMultiplyAdd, a*b + c rounded once, emulated exactly by ``fma32``),
evaluated in the order written.  Mode M is pinned to mode D (``definition``) by the
per-step tolerance and to the exact special cases (scale 0 -> uncond, scale 1
-> cond, mask 0 -> original latent, ...).

The evaluation order (a specification both sides implement independently).
The update is linear in x for every path: pred = alpha*x + P with P free of
x, so x' = K*x + B with K per sample (per pixel when inpainting) and B from
per-channel tables; the tables and K are built once, and each element costs
one fused multiply-add per region plus one.

per sample, from sigma = sig[t], sigma' = sig[t+1], scale w:
    v = sigma*sigma; den = s2 + v; a = s2/den; b1 = v/den
    last step (sigma' == 0), Euler or Heun:  g = 1; K = a
    Euler:  q = (sigma' - sigma)/sigma; g = -q; K = fma(q, b1, 1)
    Heun:   v' = sigma'*sigma'; den' = s2 + v'; a' = s2/den'; b2 = v'/den'
            h = sigma' - sigma; i1 = 1/sigma; i2 = 1/sigma'; hh = h*0.5; nh = -hh
            e1 = b1*i1; e2 = b2*i2
            K  = fma(hh, fma(e2, fma(h, e1, 1), e1), 1)
            c1 = (nh*i1)*fma(h, e2, 1); c2 = nh*i2
    mode A: scale != 1; mode B: scale == 1, uncond kept; mode C: uncond skipped
    (a regional sample in mode C is stepped as in mode B: where no region has
    weight the cond is the uncond, as the definition's regional sum falls back
    to it; the plan skips the uncond only where the regions cover the latent)
per channel c, at sigma (and at sigma' with v', den' for Heun):
    bu = (v*mu_u)/den
    no regions:  P = fma(w, (v*(mu_c - mu_u))/den, bu)   (mode A)
                 P = (v*mu_c)/den                        (modes B, C)
    regions:     t0 = bu, t_r = (v*(mu_r - mu_u))/den
    (a regional sample none of whose regions is valid: regions, none of them)
    tables without inpaint: T0 = g*t0, T_r = g*t_r (P: g*P)       (Euler, last)
                            T0 = fma(c1, t0, c2*t0'), T_r likewise (Heun)
per pixel (regional launches):
    f_r = float(ny_r*nx_r) * (1/F^4)  with ny = min(dy+1,F)*min(h_r-dy,F),
                                           nx likewise, 0 outside the box
    w_r = strength_r*f_r; W = ((w_0 + w_1) + w_2) ...
    covered = W > 0; iW = 1/W (0 if not covered); wh_r = w_r*iW
    om_r = (covered ? w : 0)*wh_r
per element, without inpaint:
    B = T0 (or the P table); B = fma(om_r, T_r, B) for r = 0, 1, ...
    x' = fma(K, x, B)
with inpaint (mask m, om = 1 - m, original latent xo), per pixel:
    last:  k = m*a; l1 = g*m; lo = g*om
    Euler: k = fma(q, fma(-m, a, 1), 1); l1 = g*m; lo = g*om
    Heun:  A1 = fma(-m, a, 1); A2 = fma(-m, a', 1); f1 = i1*A1;
           f2 = i2*A2; G = fma(h, f2, 1); k = fma(hh, fma(f2, fma(h, f1, 1), f1), 1)
           l1 = ((nh*i1)*G)*m; l2 = (nh*i2)*m; lo = (nh*fma(i1, G, i2))*om
    per element: B1 = t0-chain at sigma (B1 = t0; B1 = fma(om_r, t_r, B1)), or P;
           B2 likewise at sigma' (Heun)
    Euler, last: x' = fma(k, x, fma(l1, B1, lo*xo))
    Heun:        x' = fma(k, x, fma(l1, B1, fma(l2, B2, lo*xo)))
store float32, or round to bf16 (nearest, ties to even)

The two evaluations of Heun's step and the guidance combine are folded
into K and the tables exactly (in real arithmetic): x' = x + h/2 (d + d2)
with d = (x - pred(x))/sigma, xt = x + h d, d2 = (xt - pred(xt))/sigma',
pred(x) = alpha x + P, gives the coefficients above; the regional cond
sum_r wh_r (a x + b_r) uses sum_r wh_r = 1 on covered pixels.

materialised branches (rows of the plan layout, storage dtype, read as float32):
    pred = c                                 (scale == 1)
         = fma(w, c - u, u)                  (otherwise)
    pb = fma(m, pred, om*xo)  (inpaint)  else pred
    Euler: sigma' == 0: x' = pb, else x' = fma(x - pb, q, x)
    Heun, first call: d = (x - pb)*i; xt = fma(h, d, x); store d (float32) and
           xt (storage dtype); sigma' == 0: xt = pb and no d
    Heun, second call: xt = fma(h, d, x); d2 = (xt - pb2)*i'; x' = fma(d + d2, hh, x)
"""
from __future__ import annotations

import numpy as np

from . import definition as D

f32 = np.float32


def fma32(a, b, c):
    """IEEE 754 float32 fusedMultiplyAdd: a*b + c rounded once (to nearest even).

    float64 holds a*b exactly (24 + 24 significant bits).  The sum s = a*b + c
    in float64 is rounded once; TwoSum gives its exact error e.  Turning s
    into the round-to-odd value (if e != 0 and the last bit of s is even, step
    one ulp towards the exact sum) and then rounding to float32 yields the
    correctly rounded float32 sum, because float64 carries at least 24 + 2
    bits (Boldo and Melquiond, "Emulation of FMA and correctly rounded sums:
    proved algorithms using rounding to odd", IEEE Trans. Computers 2008).
    """
    a = np.asarray(a, np.float32).astype(np.float64)
    b = np.asarray(b, np.float32).astype(np.float64)
    c = np.asarray(c, np.float32).astype(np.float64)
    p = a * b
    s = p + c
    bv = s - p
    e = (p - (s - bv)) + (c - bv)
    s = np.asarray(s, np.float64)
    odd = (s.view(np.int64) & 1) == 1
    fix = (e != 0) & ~odd
    toward = np.where(e > 0, np.inf, -np.inf)
    s = np.where(fix, np.nextafter(s, toward), s)
    return s.astype(np.float32)


def _store(x, dtype):
    x = np.asarray(x, np.float32)
    if dtype == "bf16":
        return D.round_bf16(x).astype(np.float32)
    return x


def _ramp_counts(d, L, F):
    """Integer feather numerators min(d+1,F)*min(L-d,F) (0 outside [0,L))."""
    F = max(int(F), 1)
    d = np.asarray(d, np.int64)
    num = np.minimum(d + 1, F) * np.minimum(L - d, F)
    return np.where((d >= 0) & (d < L), num, 0)


def pixel_weights(boxes, strengths, H, W, F):
    """Normalised per-pixel region weights wh[R,H,W] and the covered flag."""
    Fe = max(int(F), 1)
    inv_f4 = f32(1.0) / f32(Fe * Fe * Fe * Fe)
    ws = []
    for (y0, y1, x0, x1), s in zip(boxes, strengths):
        ny = _ramp_counts(np.arange(H) - y0, y1 - y0, Fe)
        nx = _ramp_counts(np.arange(W) - x0, x1 - x0, Fe)
        f = (ny[:, None] * nx[None, :]).astype(np.float32) * inv_f4
        ws.append(f32(s) * f)
    Wsum = ws[0]
    for w in ws[1:]:
        Wsum = Wsum + w
    covered = Wsum > f32(0)
    iW = np.where(covered, f32(1.0) / np.where(covered, Wsum, f32(1)), f32(0)).astype(np.float32)
    return [w * iW for w in ws], covered, Wsum


class Params32:
    """Per-sample constants in float32."""

    def __init__(self, mu_u, mu_c, s2, boxes=(), strengths=(), mu_r=(), feather=0,
                 H=0, W=0, mask=None, x_orig=None, regional=None):
        self.mu_u = np.asarray(mu_u, np.float32)
        self.mu_c = np.asarray(mu_c, np.float32)
        self.s2 = f32(s2)
        self.mu_r = [np.asarray(m, np.float32) for m in mu_r]
        self.nr = len(self.mu_r)
        # a regional sample none of whose regions is valid at this step: C = U
        self.regional = self.nr > 0 if regional is None else bool(regional)
        if self.nr:
            self.wh, self.covered, self.wsum = pixel_weights(boxes, strengths, H, W, feather)
        self.mask = None if mask is None else np.asarray(mask, np.float32)
        self.x_orig = None if x_orig is None else np.asarray(x_orig, np.float32)


def _tables(sigma, w, mode, prm):
    """Per-channel offsets at one sigma: (t0, [t_r]) for a regional sample,
    (P, None) otherwise."""
    v = sigma * sigma
    den = prm.s2 + v
    bu = (v * prm.mu_u) / den
    if not prm.regional:
        if mode == "A":
            return fma32(w, (v * (prm.mu_c - prm.mu_u)) / den, bu), None
        return (v * prm.mu_c) / den, None
    return bu, [(v * (m - prm.mu_u)) / den for m in prm.mu_r]


def _chain(t0, tr, om):
    """B = t0; B = fma(om_r, t_r, B) over the regions, per element."""
    B = np.broadcast_to(t0[:, None, None], (t0.shape[0],) + (om[0].shape if om else (1, 1)))
    B = np.asarray(B, np.float32)
    for o, t in zip(om, tr or []):
        B = fma32(o[None], t[:, None, None], B)
    return B


def step32(x, sigma, sigma_next, w, need_uncond, prm, sampler):
    """One step in mode M.  ``x`` float32 [C,H,W]; returns float32 (unstored)."""
    x = np.asarray(x, np.float32)
    sigma, sigma_next, w = f32(sigma), f32(sigma_next), f32(w)
    mode = "C" if not need_uncond else ("B" if w == f32(1) else "A")
    one, s2 = f32(1), prm.s2
    v = sigma * sigma
    den = s2 + v
    a = s2 / den
    b1 = v / den
    last = sigma_next == f32(0)
    heun = sampler == "heun" and not last
    if last:
        g, K = one, a
    elif not heun:
        q = (sigma_next - sigma) / sigma
        g, K = -q, fma32(q, b1, one)
    else:
        v2 = sigma_next * sigma_next
        den2 = s2 + v2
        a2 = s2 / den2
        b2 = v2 / den2
        h = sigma_next - sigma
        i1 = one / sigma
        i2 = one / sigma_next
        hh = h * f32(0.5)
        nh = -hh
        e1 = b1 * i1
        e2 = b2 * i2
        K = fma32(hh, fma32(e2, fma32(h, e1, one), e1), one)
        c1 = (nh * i1) * fma32(h, e2, one)
        c2 = nh * i2
    t0, tr = _tables(sigma, w, mode, prm)
    if heun:
        t0b, trb = _tables(sigma_next, w, mode, prm)
    om = []
    if prm.regional and prm.nr:
        weff = np.where(prm.covered, w, f32(0)).astype(np.float32)
        om = [weff * wh for wh in prm.wh]
    if prm.mask is None:
        if heun:
            T0 = fma32(c1, t0, c2 * t0b)
            Tr = [fma32(c1, t, c2 * u) for t, u in zip(tr, trb)] if tr is not None else None
        else:
            T0 = g * t0
            Tr = [g * t for t in tr] if tr is not None else None
        return fma32(K, x, _chain(T0, Tr, om))
    m = prm.mask[None]
    omk = f32(1) - m
    B1 = _chain(t0, tr, om)
    xo = prm.x_orig
    if not heun:
        k = m * a if last else fma32(q, fma32(-m, a, one), one)
        return fma32(k, x, fma32(g * m, B1, (g * omk) * xo))
    A1 = fma32(-m, a, one)
    A2 = fma32(-m, a2, one)
    f1 = i1 * A1
    f2 = i2 * A2
    G = fma32(h, f2, one)
    k = fma32(hh, fma32(f2, fma32(h, f1, one), f1), one)
    l1 = ((nh * i1) * G) * m
    l2 = (nh * i2) * m
    lo = (nh * fma32(i1, G, i2)) * omk
    B2 = _chain(t0b, trb, om)
    return fma32(k, x, fma32(l1, B1, fma32(l2, B2, lo * xo)))


def params32(inp, i, t=None):
    """Params32 of sample i (at step t when the regions have validity ranges)."""
    sp = inp.spec
    rs = D.valid_regions(inp, i, t)
    boxes = [D.area_box(inp.region_frac[i, r], sp.H, sp.W) for r in rs]
    return Params32(inp.mu_uncond[i], inp.mu_cond[i], sp.s2, boxes,
                    inp.region_strength[i, rs], [inp.mu_region[i, r] for r in rs],
                    sp.feather, sp.H, sp.W,
                    None if inp.mask is None else inp.mask[i, 0],
                    None if inp.x_orig is None else _store(inp.x_orig[i], sp.dtype),
                    regional=int(inp.region_count[i]) > 0)


def init_latent32(inp, sig):
    sp = inp.spec
    z = sig[inp.start_step][:, None, None, None]
    if inp.x_orig is not None:
        x = fma32(inp.noise, z, _store(inp.x_orig, sp.dtype))
    else:
        x = inp.noise.astype(np.float32) * z
    return _store(x, sp.dtype)


def trajectory32(inp, launches=None, samples=None, keep=False):
    """The sampler loop in mode M (same plan and schedule as mode D)."""
    sp = inp.spec
    sig, table, cov = D.run_setup(inp)
    idx = range(sp.n) if samples is None else samples
    prms = {i: params32(inp, i) for i in idx}
    x = init_latent32(inp, sig)
    states = [x.copy()] if keep else None
    L = sp.steps if launches is None else launches
    for k in range(L):
        t = inp.start_step.astype(np.int64) + k
        ranged = inp.region_range is not None
        plan = D.build_plan(t, sp.steps, sp.num_buckets, table, inp.cfg_override,
                            D.coverage(inp, t) if ranged else cov, D.table_end(inp))
        for i in idx:
            if plan["bucket_id"][i] < 0:
                continue
            ti = int(t[i])
            prm = params32(inp, i, ti) if ranged else prms[i]
            x[i] = _store(step32(x[i], sig[ti], sig[ti + 1], plan["scale"][i],
                                 bool(plan["need_uncond"][i]), prm, sp.sampler),
                          sp.dtype)
        if keep:
            states.append(x.copy())
    return (x, states) if keep else x


def init_sample32(inp, i, sigma):
    """Request i's joining state in mode M (init_latent32's rule for one sample)."""
    sp = inp.spec
    z = np.float32(sigma)
    if inp.x_orig is not None:
        x = fma32(inp.noise[i], np.full(inp.noise[i].shape, z, np.float32), _store(inp.x_orig[i], sp.dtype))
    else:
        x = inp.noise[i].astype(np.float32) * z
    return _store(x, sp.dtype)


def serve_trajectory32(inp, n_slots, launches, ring=False, slots=None, keep=False):
    """The continuously batched loop in mode M (the schedule, plans and
    validity ranges of definition.serve_trajectory)."""
    sp = inp.spec
    ranged = inp.region_range is not None
    sig, table, cov = D.run_setup(inp)
    req, tt, join = D.serve_schedule(inp.start_step, sp.steps, n_slots, sp.n, launches, ring)
    x = np.zeros((n_slots, sp.C, sp.H, sp.W), np.float32)
    states = []
    idx = range(n_slots) if slots is None else slots
    ov = np.asarray(inp.cfg_override, np.float32)
    prms = {}
    for k in range(launches):
        r = req[k]
        ovk = np.where(r >= 0, ov[np.maximum(r, 0)], np.float32(np.nan)).astype(np.float32)
        if ranged:
            covk = np.array([r[s] < 0 or D.covered_at(inp, int(r[s]), int(tt[k, s])) for s in range(n_slots)])
        else:
            covk = cov[np.maximum(r, 0)]
        plan = D.build_plan(tt[k], sp.steps, sp.num_buckets, table, ovk, covk, D.table_end(inp))
        for s in idx:
            if r[s] < 0 or plan["bucket_id"][s] < 0:
                continue
            ri, ti = int(r[s]), int(tt[k, s])
            key = (ri, ti) if ranged else ri
            if key not in prms:
                prms[key] = params32(inp, ri, ti if ranged else None)
            if join[k, s]:
                x[s] = init_sample32(inp, ri, sig[ti])
            x[s] = _store(step32(x[s], sig[ti], sig[ti + 1], plan["scale"][s],
                                 bool(plan["need_uncond"][s]), prms[key], sp.sampler), sp.dtype)
        if keep:
            states.append(x.copy())
    return x, states, (req, tt, join)


def area_accumulate32(crops, boxes, strengths, H, W, F, fallback=None):
    """Standalone regional accumulation in mode M.

    ``crops[r]`` is the [C, h_r, w_r] prediction of region r.  Returns the
    normalised cond prediction [C,H,W] (fallback, else 0, where no region has
    weight) and the weight sum [H,W].  Terms of regions that do not contain a
    pixel are left out of its sum (they are exact zeros in the fused step).
    """
    wh, covered, wsum = pixel_weights(boxes, strengths, H, W, F)
    C = crops[0].shape[0]
    acc = np.zeros((C, H, W), np.float32)
    started = np.zeros((H, W), bool)
    for r, (y0, y1, x0, x1) in enumerate(boxes):
        full = np.zeros((C, H, W), np.float32)
        full[:, y0:y1, x0:x1] = crops[r]
        inb = np.zeros((H, W), bool)
        inb[y0:y1, x0:x1] = True
        acc = np.where(inb[None], np.where(started[None], fma32(wh[r][None], full, acc),
                                           wh[r][None] * full), acc)
        started |= inb
    if fallback is not None:
        acc = np.where(covered[None], acc, np.asarray(fallback, np.float32))
    else:
        acc = np.where(covered[None], acc, f32(0))
    return acc.astype(np.float32), wsum


def mask_blend32(a, b, mask, dtype):
    """out = m*a + (1-m)*b in float32, mask [.,1,H,W] broadcast over channels."""
    m = np.asarray(mask, np.float32)
    om = f32(1) - m
    return _store(fma32(m, np.asarray(a, np.float32), om * np.asarray(b, np.float32)), dtype)


def rows_pred32(c, u, w, mask=None, x_orig=None):
    """Mode M prediction from materialised cond/uncond rows (float32 values)."""
    c = np.asarray(c, np.float32)
    w = f32(w)
    if w == f32(1):
        pred = c.copy()
    else:
        u = np.asarray(u, np.float32)
        pred = fma32(w, c - u, u)
    if mask is not None:
        m = np.asarray(mask, np.float32)[None]
        om = f32(1) - m
        pred = fma32(m, pred, om * np.asarray(x_orig, np.float32))
    return np.asarray(pred, np.float32)


def rows_euler32(x, pb, sigma, sigma_next):
    x = np.asarray(x, np.float32)
    sigma, sigma_next = f32(sigma), f32(sigma_next)
    if sigma_next == f32(0):
        return np.asarray(pb, np.float32).copy()
    q = (sigma_next - sigma) / sigma
    return fma32(x - pb, q, x)


def rows_heun_predict32(x, pb, sigma, sigma_next):
    """Returns (d float32 or None, x~ float32, unstored)."""
    x = np.asarray(x, np.float32)
    sigma, sigma_next = f32(sigma), f32(sigma_next)
    if sigma_next == f32(0):
        return None, np.asarray(pb, np.float32).copy()
    h = sigma_next - sigma
    d = (x - pb) * (f32(1) / sigma)
    return d.astype(np.float32), fma32(h, d, x)


def rows_heun_correct32(x, d, pb2, sigma, sigma_next):
    x = np.asarray(x, np.float32)
    sigma, sigma_next = f32(sigma), f32(sigma_next)
    h = sigma_next - sigma
    i2 = f32(1) / sigma_next
    hh = h * f32(0.5)
    xt = fma32(h, d, x)
    d2 = (xt - pb2) * i2
    return fma32(d + d2, hh, x)
