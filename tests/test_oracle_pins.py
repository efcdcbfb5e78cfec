"""Pins of the CPU oracle to facts fixed outside itself (no GPU needed).

Each test ties an oracle function to a closed form, brute force, a special
case the pages fix, or a library routine -- chosen so that a dropped term, a
wrong sign or index, or a transposed operand fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W
from oracle import definition as D
from oracle import mirror32 as M


# ---------------------------------------------------------------- bf16 store

def test_round_bf16_matches_library_rne():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    # exact ties: a bf16 value plus half an ulp, both parities of the last bit
    base = torch.from_numpy(x[:2000]).to(torch.bfloat16).to(torch.float32).numpy()
    bits = base.view(np.uint32) | np.uint32(0x8000)
    ties = bits.view(np.float32)
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1.0, -1.0, 3.0e38])])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = D.round_bf16(x).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_round_bf16_nan_inf_pass_through():
    v = D.round_bf16(np.array([np.nan, np.inf, -np.inf]))
    assert np.isnan(v[0]) and v[1] == np.inf and v[2] == -np.inf


# ---------------------------------------------------------------- schedule

@pytest.mark.parametrize("steps,denoise", [(10, 1.0), (50, 1.0), (30, 1.0), (20, 0.6), (7, 0.35)])
def test_sigma_schedule_closed_form(steps, denoise):
    sig, N = D.sigma_schedule(14.6, 0.03, steps, denoise)
    assert sig.dtype == np.float32 and sig.size == steps + 1
    assert sig[-1] == 0.0
    assert sig[-2] == np.float32(0.03)
    assert N * denoise >= steps and (N - 1) * denoise < steps
    # independent closed form: the power form sigma_max*(min/max)**(i/(N-1))
    i = np.arange(N - steps, N)
    pw = 14.6 * (0.03 / 14.6) ** (i / (N - 1))
    np.testing.assert_allclose(sig[:-1], pw, rtol=2e-7)
    # log-equal spacing (constant ratio)
    r = np.log(sig[1:-1].astype(np.float64)) - np.log(sig[:-2].astype(np.float64))
    np.testing.assert_allclose(r, math.log(0.03 / 14.6) / (N - 1), atol=3e-7)
    if denoise == 1.0:
        assert sig[0] == np.float32(14.6) and N == steps


def test_denoise_tail_of_regional_workload():
    # 20 steps at denoise 0.6 are taken from a 34-step base schedule.
    sig, N = D.sigma_schedule(14.6, 0.03, 20, 0.6)
    assert N == 34
    assert abs(float(sig[0]) - 14.6 * (0.03 / 14.6) ** (14 / 33)) < 2e-7
    full, _ = D.sigma_schedule(14.6, 0.03, 34, 1.0)
    assert np.array_equal(full[14:], sig)


# ---------------------------------------------------------------- buckets

def test_bucket_id_bruteforce_enumeration():
    for steps in range(1, 61):
        for nb in range(1, 21):
            for t in range(steps):
                assert D.bucket_id(t, steps, nb) == D.bucket_id_bruteforce(t, steps, nb)


def test_bucket_id_matches_page_formula_on_workloads():
    # the write-up's float formula min(int(t/steps*nb), nb-1) for every
    # (steps, nb) pair the workloads use
    for steps, nb in [(10, 1), (50, 8), (30, 16), (20, 8)]:
        for t in range(steps):
            assert D.bucket_id(t, steps, nb) == min(int(t / steps * nb), nb - 1)


def test_bucket_id_exact_where_float_product_fails():
    assert min(int(3 / 11 * 55), 54) == 14        # float64 rounding below 15
    assert D.bucket_id(3, 11, 55) == 15           # 3*55 = 165 = 15*11


def test_bucket_tables():
    lin = D.bucket_table("linear", 2.0, 1.2, 0.0, 8)
    assert lin[0] == np.float32(2.0) and lin[-1] == np.float32(1.2)
    assert np.all(np.diff(lin) < 0)
    np.testing.assert_allclose(lin, np.linspace(2.0, 1.2, 8), rtol=1e-7)
    assert np.array_equal(D.bucket_table("const", 7.0, 0, 0, 1), np.float32([7.0]))
    fh = D.bucket_table("front_high", 2.0, 1.2, 0.2, 16)
    # front-high at 30 steps: exactly the first 20% (6 steps) are strong
    per_step = [fh[D.bucket_id(t, 30, 16)] for t in range(30)]
    assert per_step[:6] == [np.float32(2.0)] * 6
    assert per_step[6:] == [np.float32(1.2)] * 24


# ---------------------------------------------------------------- plan

def _brute_plan_checks(t, steps, nb, table, override, covered, plan):
    n = len(t)
    act = [i for i in range(n) if 0 <= t[i] < steps]
    assert plan["n_active"] == len(act)
    assert sorted(plan["order"].tolist()) == act
    # stable (bucket, id) order
    keys = [(int(plan["bucket_id"][i]), i) for i in plan["order"]]
    assert keys == sorted(keys)
    for b in range(nb):
        cnt = sum(1 for i in act if D.bucket_id(t[i], steps, nb) == b)
        assert plan["bucket_count"][b] == cnt
        assert plan["bucket_offset"][b + 1] - plan["bucket_offset"][b] == cnt
        ucnt = sum(1 for i in act if D.bucket_id(t[i], steps, nb) == b and plan["need_uncond"][i])
        assert plan["uncond_offset"][b + 1] - plan["uncond_offset"][b] == ucnt
    m = plan["n_uncond"]
    for i in range(n):
        if i not in act:
            assert plan["bucket_id"][i] == -1 and plan["cond_row"][i] == -1
            assert plan["uncond_row"][i] == -1
            continue
        w = override[i] if not np.isnan(override[i]) else table[plan["bucket_id"][i]]
        assert plan["scale"][i] == w
        assert plan["need_uncond"][i] == (not (w == 1.0 and covered[i]))
        # rows: cond rows follow the uncond half; within each half samples of
        # bucket b sit inside [offset[b], offset[b+1])
        b = plan["bucket_id"][i]
        r = plan["cond_row"][i] - m
        assert plan["bucket_offset"][b] <= r < plan["bucket_offset"][b + 1]
        if plan["need_uncond"][i]:
            u = plan["uncond_row"][i]
            assert plan["uncond_offset"][b] <= u < plan["uncond_offset"][b + 1]
        else:
            assert plan["uncond_row"][i] == -1
    assert sorted(plan["cond_row"][plan["cond_row"] >= 0].tolist()) == list(range(m, m + len(act)))
    assert sorted(plan["uncond_row"][plan["uncond_row"] >= 0].tolist()) == list(range(m))


def test_plan_bruteforce_random():
    rng = np.random.default_rng(3)
    for _ in range(300):
        n = int(rng.integers(1, 40))
        steps = int(rng.integers(1, 60))
        nb = int(rng.integers(1, 17))
        t = rng.integers(-3, steps + 3, size=n)
        table = D.bucket_table("linear", 2.0, 1.0, 0, nb)
        ov = np.where(rng.random(n) < 0.3, 1.0, np.nan).astype(np.float32)
        cov = rng.random(n) < 0.8
        plan = D.build_plan(t, steps, nb, table, ov, cov)
        _brute_plan_checks(t, steps, nb, table, ov, cov, plan)


def test_plan_layout_scale_one_samples_skip():
    # throughput workload: a quarter of the samples carry cfg 1 and lose
    # their uncond row; the rest keep it
    inp = W.make_inputs(W.config("throughput_bf16_heun"))
    sig, table, cov = D.run_setup(inp)
    plan = D.build_plan(np.zeros(64, np.int64), 30, 16, table, inp.cfg_override, cov)
    assert plan["n_active"] == 64 and plan["n_uncond"] == 48
    assert set(np.nonzero(~plan["need_uncond"])[0]) == set(np.nonzero(inp.cfg_override == 1.0)[0])


# ---------------------------------------------------------------- areas

def test_area_box_bounds_and_sizes():
    inp = W.make_inputs(W.config("regional_inpaint"))
    for i in range(16):
        for r in range(3):
            y0, y1, x0, x1 = D.area_box(inp.region_frac[i, r], 128, 128)
            assert 0 <= y0 < y1 <= 128 and 0 <= x0 < x1 <= 128
            assert round(0.2 * 128) - 1 <= y1 - y0 <= round(0.8 * 128) + 1
    assert D.area_box((0, 0, 1, 1), 40, 72) == (0, 40, 0, 72)
    assert D.area_box((0.5, 0.25, 0.5, 0.5), 8, 8) == (4, 8, 2, 6)
    assert D.area_box((0.99, 0.99, 0.001, 0.001), 8, 8) == (7, 8, 7, 8)


def test_feather_dyadic_values_and_symmetry():
    wgt = D.region_weight((10, 40, 20, 60), 1.0, 64, 80, 8)
    assert wgt[25, 40] == 1.0                 # interior
    assert wgt[10, 40] == 1 / 8               # top edge
    assert wgt[39, 40] == 1 / 8               # bottom edge
    assert wgt[10, 20] == 1 / 64              # corner
    assert wgt[13, 40] == 4 / 8
    assert wgt[9, 40] == 0 and wgt[40, 40] == 0 and wgt[25, 19] == 0 and wgt[25, 60] == 0
    # separable and mirror-symmetric inside the box
    box = wgt[10:40, 20:60]
    assert np.array_equal(box, box[::-1, :]) and np.array_equal(box, box[:, ::-1])
    assert np.allclose(box, np.outer(box[:, 20], box[15, :]))
    # no feathering: the box indicator
    w0 = D.region_weight((1, 3, 2, 5), 2.0, 4, 6, 0)
    ind = np.zeros((4, 6)); ind[1:3, 2:5] = 2.0
    assert np.array_equal(w0, ind)


def test_feather_integer_form_equals_ramp_product():
    # the mirror's integer numerators over F^4 are the same dyadic weights
    for F in (1, 2, 3, 8):
        for L in (1, 2, 5, 17, 30):
            ny = M._ramp_counts(np.arange(-2, L + 2), L, F)
            g = D.feather_1d(np.arange(-2, L + 2), L, F)
            np.testing.assert_allclose(ny / F ** 2, g, rtol=1e-15)


# ---------------------------------------------------------------- denoiser

def test_denoiser_is_gaussian_posterior_mean_by_quadrature():
    # E[y | x] for y ~ N(mu, s^2), x = y + sigma*eps, by direct numerical
    # integration over y (independent of the closed form).
    s2, mu = 0.25, np.array([0.7])
    y = np.linspace(-12, 12, 400001)
    for sigma in (0.03, 0.5, 3.0, 14.6):
        for x in (-4.0, 0.2, 9.0):
            p = np.exp(-(y - mu[0]) ** 2 / (2 * s2) - (x - y) ** 2 / (2 * sigma ** 2))
            want = (y * p).sum() / p.sum()
            got = D.denoise(np.full((1, 1, 1), x), sigma, mu, s2)[0, 0, 0]
            assert abs(got - want) < 1e-7 * max(1.0, abs(want))


def test_denoiser_limits():
    x = np.random.default_rng(0).standard_normal((2, 3, 3))
    mu = np.array([0.3, -1.0])
    assert np.array_equal(D.denoise(x, 0.0, mu, 0.25), x)
    np.testing.assert_allclose(D.denoise(x, 1e8, mu, 0.25), np.broadcast_to(mu[:, None, None], x.shape), atol=1e-12)


# ---------------------------------------------------------------- regions

def _region_setup(seed=0, H=20, W=24, F=3):
    rng = np.random.default_rng(seed)
    C = 2
    x = rng.standard_normal((C, H, W))
    mus = [rng.standard_normal(C) for _ in range(3)]
    boxes = [(0, 12, 0, 15), (5, 20, 8, 24), (3, 9, 2, 7)]
    strengths = [0.7, 1.3, 0.9]
    wts = [D.region_weight(b, s, H, W, F) for b, s in zip(boxes, strengths)]
    return x, mus, boxes, strengths, wts


def test_regional_cond_closed_form_mean():
    x, mus, boxes, strengths, wts = _region_setup()
    sigma, s2 = 1.7, 0.25
    u = D.denoise(x, sigma, np.array([0.1, 0.2]), s2)
    preds = [D.denoise(x, sigma, m, s2) for m in mus]
    c = D.regional_cond(preds, wts, u)
    wsum = sum(wts)
    cov = wsum > 0
    mbar = sum(w[None] * m[:, None, None] for w, m in zip(wts, mus)) / np.where(cov, wsum, 1)[None]
    closed = (s2 * x + sigma ** 2 * mbar) / (s2 + sigma ** 2)
    np.testing.assert_allclose(c[:, cov], closed[:, cov], rtol=1e-13, atol=1e-13)
    assert np.array_equal(c[:, ~cov], u[:, ~cov])
    assert (~cov).any()


def test_regional_cond_invariances():
    x, mus, boxes, strengths, wts = _region_setup(1)
    u = D.denoise(x, 2.0, np.zeros(2), 0.25)
    preds = [D.denoise(x, 2.0, m, 0.25) for m in mus]
    c = D.regional_cond(preds, wts, u)
    np.testing.assert_allclose(D.regional_cond(preds, [3.5 * w for w in wts], u), c, rtol=1e-13, atol=1e-15)
    zero = [0 * wts[0]]
    np.testing.assert_allclose(D.regional_cond(preds + [preds[0] * 9], wts + zero, u), c, rtol=0, atol=0)
    # one full-frame region reproduces its own prediction
    full = [D.region_weight((0, 20, 0, 24), 0.8, 20, 24, 0)]
    np.testing.assert_allclose(D.regional_cond(preds[:1], full, u), preds[0], rtol=1e-15)


# ---------------------------------------------------------------- combine / blend

def test_cfg_combine_special_cases_and_affine_form():
    rng = np.random.default_rng(5)
    u, c = rng.standard_normal((2, 3, 4, 5))
    assert np.array_equal(D.cfg_combine(u, c, 0.0), u)          # scale 0 -> uncond
    assert np.array_equal(D.cfg_combine(u, c, 1.0), c)          # scale 1 -> cond
    for w in (0.3, 1.2, 2.0, 7.0):
        # W' = sm*W + sp*dW with W = u, dW = c - u, sm = 1, sp = w, and the
        # equivalent (1-w) u + w c
        np.testing.assert_allclose(D.cfg_combine(u, c, w), (1 - w) * u + w * c, rtol=1e-13, atol=1e-13)
        u2, c2 = rng.standard_normal((2, 3, 4, 5))
        lhs = D.cfg_combine(2 * u - 0.5 * u2, 2 * c - 0.5 * c2, w)
        rhs = 2 * D.cfg_combine(u, c, w) - 0.5 * D.cfg_combine(u2, c2, w)
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_inpaint_blend_extremes():
    rng = np.random.default_rng(6)
    p, xo = rng.standard_normal((2, 2, 3, 4))
    assert np.array_equal(D.inpaint_blend(p, xo, np.ones((3, 4))), p)
    assert np.array_equal(D.inpaint_blend(p, xo, np.zeros((3, 4))), xo)


# ---------------------------------------------------------------- sampler

def _tiny_prm():
    rng = np.random.default_rng(11)
    return D.SampleParams(rng.standard_normal(2), rng.standard_normal(2), 0.25), rng


@pytest.mark.parametrize("sampler,order", [("euler", 1), ("heun", 2)])
def test_sampler_converges_to_probability_flow(sampler, order):
    prm, rng = _tiny_prm()
    w = 7.0
    x0 = 14.6 * rng.standard_normal((2, 3, 3))
    mean = (prm.mu_u + w * (prm.mu_c - prm.mu_u))[:, None, None]
    exact = D.pf_ode_exact(x0, 14.6, 0.03, mean, 0.25)
    errs = []
    for N in (10, 20, 40, 80, 160):
        sig = [14.6 * (0.03 / 14.6) ** (i / (N - 1)) for i in range(N)]
        x = x0.copy()
        for k in range(N - 1):
            x = D.step(x, sig[k], sig[k + 1], w, prm, sampler)
        errs.append(np.abs(x - exact).max())
    ratios = [errs[i] / errs[i + 1] for i in range(len(errs) - 1)]
    target = 2.0 ** order
    assert all(abs(r - target) < 0.25 * target for r in ratios[1:]), ratios
    assert errs[-1] < (0.05 if order == 1 else 0.01)


def test_final_step_lands_on_prediction():
    prm, rng = _tiny_prm()
    x = rng.standard_normal((2, 3, 3))
    for s in ("euler", "heun"):
        assert np.array_equal(D.step(x, 0.03, 0.0, 2.0, prm, s), D.guided_pred(x, 0.03, 2.0, prm))


def test_unmasked_region_follows_original_plus_noise():
    sp = W.small_spec(n=2, C=2, H=10, W=12, inpaint=True, regions=0, steps=8,
                      mixed_start=False, skip_frac=0.0)
    inp = W.make_inputs(sp)
    inp.mask[:, :, :, :6] = 0.0
    sig, _ = D.sigma_schedule(sp.sigma_max, sp.sigma_min, sp.steps)
    _, states = D.trajectory(inp, storage="f64", keep=True)
    for k in range(sp.steps):
        want = (inp.x_orig[:, :, :, :6].astype(np.float64)
                + inp.noise[:, :, :, :6].astype(np.float64) * float(sig[k]))
        np.testing.assert_allclose(states[k][:, :, :, :6], want, atol=1e-11)
    assert np.array_equal(states[-1][:, :, :, :6], inp.x_orig[:, :, :, :6])
    # mask 1 everywhere is the plain run
    inp1 = W.make_inputs(sp); inp1.mask[:] = 1.0
    plain = W.make_inputs(dataclasses_replace(sp, inpaint=False))
    plain.x_orig = inp1.x_orig  # same starting latent
    x_mask1 = D.trajectory(inp1, storage="f64")
    x_plain = D.trajectory(plain, storage="f64")
    assert np.array_equal(x_mask1, x_plain)


def dataclasses_replace(sp, **kw):
    import dataclasses
    return dataclasses.replace(sp, **kw)


def test_scale_one_skip_ignores_uncond_and_scale_zero_ignores_cond():
    sp = W.small_spec(n=3, C=2, H=6, W=8, steps=5, mixed_start=False, skip_frac=0.0,
                      curve=W.Curve("const", 1.0), num_buckets=1)
    inp = W.make_inputs(sp)
    a = D.trajectory(inp, storage="f64")
    inp.mu_uncond[:] = 99.0
    assert np.array_equal(D.trajectory(inp, storage="f64"), a)
    sp0 = dataclasses_replace(sp, curve=W.Curve("const", 0.0))
    inp0 = W.make_inputs(sp0)
    b = D.trajectory(inp0, storage="f64")
    inp0.mu_cond[:] = -42.0
    assert np.array_equal(D.trajectory(inp0, storage="f64"), b)


def test_per_sample_independence():
    sp = W.small_spec(n=5, C=2, H=9, W=11, regions=2, inpaint=True, steps=6)
    inp = W.make_inputs(sp)
    full = D.trajectory(inp)
    sub = D.trajectory(inp.subset([1, 3]))
    assert np.array_equal(sub, full[[1, 3]])


def test_bucket_count_invariance():
    # equal scales in every bucket -> identical trajectories for 1/4/8/16 buckets
    base = W.small_spec(n=3, C=2, H=6, W=8, steps=16, curve=W.Curve("const", 1.7))
    outs = [D.trajectory(W.make_inputs(dataclasses_replace(base, num_buckets=nb)))
            for nb in (1, 4, 8, 16)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


# ---------------------------------------------------------------- mode M vs mode D

@pytest.mark.parametrize("kw", [
    dict(dtype="f32", sampler="euler"),
    dict(dtype="f32", sampler="heun", regions=3, inpaint=True),
    dict(dtype="bf16", sampler="heun"),
    dict(dtype="bf16", sampler="euler", regions=2),
    dict(dtype="f32", sampler="heun", regions=3, region_ranges=True),
    dict(dtype="f32", sampler="euler", regions=2, inpaint=True),
    dict(dtype="bf16", sampler="euler", inpaint=True),
    dict(dtype="f32", sampler="heun", inpaint=True),
])
def test_mirror_per_step_within_tolerance_of_definition(kw):
    sp = W.small_spec(n=4, C=3, H=12, W=16, steps=7, **kw)
    inp = W.make_inputs(sp)
    sig, table, cov = D.run_setup(inp)
    x = D.init_latent(inp, sig, "f32")
    for k in range(sp.steps):
        t = inp.start_step.astype(np.int64) + k
        plan = D.build_plan(t, sp.steps, sp.num_buckets, table, inp.cfg_override,
                            D.coverage(inp, t))
        for i in range(sp.n):
            if plan["bucket_id"][i] < 0:
                continue
            ti = int(t[i])
            ref = D.step(x[i], float(sig[ti]), float(sig[ti + 1]), float(plan["scale"][i]),
                         D.sample_params(inp, i, ti), sp.sampler)
            got = M.step32(x[i].astype(np.float32), sig[ti], sig[ti + 1], plan["scale"][i],
                           bool(plan["need_uncond"][i]), M.params32(inp, i, ti), sp.sampler)
            assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()
            x[i] = ref.astype(np.float32)


@pytest.mark.parametrize("sampler", ["euler", "heun"])
@pytest.mark.parametrize("inpaint", [False, True])
def test_mirror_scale_one_within_tolerance_of_definition(sampler, inpaint):
    """Scale 1, uncond skipped and kept, where one region covers the latent
    and where coverage is partial, against the definition at w = 1, at an
    interior step and at the last one (where no region has weight the cond
    is the uncond in both)."""
    sp = W.small_spec(n=2, C=3, H=12, W=16, steps=5, regions=2, inpaint=inpaint, sampler=sampler)
    inp = W.make_inputs(sp)
    inp.region_frac[0, 0] = (0.0, 0.0, 1.0, 1.0)
    rng = np.random.default_rng(5)
    for i, need_uncond in ((0, False), (1, True), (1, False)):
        prmD, prmM = D.sample_params(inp, i), M.params32(inp, i)
        if i == 0:
            assert prmM.covered.all()
        else:
            assert not prmM.covered.all()
        x = (3.0 * rng.standard_normal((sp.C, sp.H, sp.W))).astype(np.float32)
        for s0, s1 in ((3.0, 2.0), (0.4, 0.0)):
            ref = D.step(x, s0, s1, 1.0, prmD, sampler)
            got = M.step32(x, s0, s1, 1.0, need_uncond, prmM, sampler)
            assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()


def test_mirror_exact_special_cases():
    sp = W.small_spec(n=2, C=2, H=6, W=8, steps=4, inpaint=True, mixed_start=False)
    inp = W.make_inputs(sp)
    inp.mask[:] = 0.0
    xf = M.trajectory32(inp)
    assert np.array_equal(xf, inp.x_orig)
    prm = M.Params32(np.float32([0.5, -1]), np.float32([2, 3]), 0.25)
    x = np.random.default_rng(2).standard_normal((2, 3, 3)).astype(np.float32)
    # scale 1, uncond skipped: uncond means play no part
    a = M.step32(x, 3.0, 2.0, 1.0, False, prm, "heun")
    prm2 = M.Params32(np.float32([7, 7]), np.float32([2, 3]), 0.25)
    assert np.array_equal(a, M.step32(x, 3.0, 2.0, 1.0, False, prm2, "heun"))
    # scale 0: cond means play no part
    b = M.step32(x, 3.0, 2.0, 0.0, True, prm, "euler")
    prm3 = M.Params32(np.float32([0.5, -1]), np.float32([-9, 9]), 0.25)
    assert np.array_equal(b, M.step32(x, 3.0, 2.0, 0.0, True, prm3, "euler"))


def test_norm_stats_special_cases():
    prm, rng = _tiny_prm()
    x = rng.standard_normal((2, 3, 4))
    s0 = D.norm_stats(x, 1.3, 0.0, prm, True)
    s1 = D.norm_stats(x, 1.3, 1.0, prm, False)
    assert s0[2] == s0[1] and s1[2] == s1[0] and s1[1] == 0.0
    v = D.denoise(x, 1.3, prm.mu_c, prm.s2)
    assert abs(s1[0] - np.mean([np.linalg.norm(v[c, h]) for c in range(2) for h in range(3)])) < 1e-12


# ---------------------------------------------------------------- exact fp32 fused multiply-add

def _rn_f32(q):
    """Exact round-to-nearest-even of a rational to float32 (normal range)."""
    from fractions import Fraction
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    scale = Fraction(2) ** (e - 23)
    m = q / scale
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return np.float32(float(sign * fl * scale))


def test_fma32_matches_exact_rational_rounding():
    from fractions import Fraction
    rng = np.random.default_rng(21)
    a = (rng.standard_normal(3000) * np.exp(rng.uniform(-8, 8, 3000))).astype(np.float32)
    b = (rng.standard_normal(3000) * np.exp(rng.uniform(-8, 8, 3000))).astype(np.float32)
    c = (rng.standard_normal(3000) * np.exp(rng.uniform(-16, 16, 3000))).astype(np.float32)
    c[:1000] = -(a[:1000].astype(np.float64) * b[:1000]).astype(np.float32)  # heavy cancellation
    got = M.fma32(a, b, c)
    for k in range(a.size):
        want = _rn_f32(Fraction(float(a[k])) * Fraction(float(b[k])) + Fraction(float(c[k])))
        assert got[k] == want, (a[k], b[k], c[k], got[k], want)


def test_fma32_double_rounding_trap():
    # a*b = 1 + 2^-11 + 2^-24 sits exactly halfway between two float32 values;
    # a tiny c breaks the tie upwards.  Rounding a*b + c to float64 first would
    # lose c and then round the tie to even (downwards).
    a = np.float32(1 + 2.0 ** -12)
    c = np.float32(2.0 ** -70)
    naive = np.float32(np.float64(a) * np.float64(a) + np.float64(c))
    assert naive == np.float32(1 + 2.0 ** -11)
    assert M.fma32(a, a, c) == np.float32(1 + 2.0 ** -11 + 2.0 ** -23)
    assert M.fma32(a, a, -c) == np.float32(1 + 2.0 ** -11)
    # the exact residual of a rounded product is representable and recovered
    p = np.float32(np.float64(a) * np.float64(a))
    assert M.fma32(a, a, -p) == np.float32(2.0 ** -24)


def test_fma32_identities():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(1000).astype(np.float32)
    y = rng.standard_normal(1000).astype(np.float32)
    assert np.array_equal(M.fma32(np.float32(0), x, y), y)
    assert np.array_equal(M.fma32(np.float32(1), x, np.float32(0)), x)
    assert np.array_equal(M.fma32(x, np.float32(2), np.float32(0)), x * np.float32(2))


# ---------------------------------------------------------------- materialised branches

def _rows_case(sampler="euler", seed=3):
    sp = W.small_spec(n=5, C=3, H=12, W=20, regions=2, inpaint=True, steps=6, num_buckets=3,
                      sampler=sampler, feather=3, seed=seed)
    inp = W.make_inputs(sp)
    inp.cfg_override[:] = [np.nan, 1.0, 0.0, 1.0, np.nan]
    inp.region_count[3] = 0  # a sample without regions
    sig, table, cov = D.run_setup(inp)
    x = D.init_latent(inp, sig, "f32").astype(np.float64)
    return inp, sig, table, cov, x


def _stand_in_rows(inp, plan, xs, sigmas):
    """One evaluation of the stand-in per branch, laid out as the plan says:
    uncond rows (kept samples) then cond rows; sample i at xs[i], sigmas[i]."""
    n = inp.spec.n
    rows = np.full((plan["n_uncond"] + plan["n_active"],) + xs.shape[1:], np.nan)
    for i in range(n):
        if plan["bucket_id"][i] < 0:
            continue
        prm = D.sample_params(inp, i)
        u = D.denoise(xs[i], sigmas[i], prm.mu_u, prm.s2)
        if prm.regions:
            preds = [D.denoise(xs[i], sigmas[i], mr, prm.s2) for _, _, mr in prm.regions]
            c = D.regional_cond(preds, prm.weights, u)
        else:
            c = D.denoise(xs[i], sigmas[i], prm.mu_c, prm.s2)
        rows[plan["cond_row"][i]] = c
        if plan["uncond_row"][i] >= 0:
            rows[plan["uncond_row"][i]] = u
    return rows


@pytest.mark.parametrize("k", [0, 3, 5])
def test_rows_euler_equals_inline_step(k):
    """Branch outputs laid out as the plan says, then combine + blend + Euler,
    equal the inline definition of the step (a different code path)."""
    inp, sig, table, cov, x = _rows_case("euler")
    sp = inp.spec
    t = inp.start_step.astype(np.int64) + k
    plan = D.build_plan(t, sp.steps, sp.num_buckets, table, inp.cfg_override, cov)
    act = [i for i in range(sp.n) if plan["bucket_id"][i] >= 0]
    assert act
    if k == 0:
        assert plan["n_uncond"] < plan["n_active"]  # some uncond rows are compacted away
    rows = _stand_in_rows(inp, plan, x, {i: float(sig[t[i]]) for i in act})
    for i in act:
        prm = D.sample_params(inp, i)
        s0, s1 = float(sig[t[i]]), float(sig[t[i] + 1])
        P = D.rows_pred(rows, plan, i, float(plan["scale"][i]), prm.x_orig, prm.mask)
        got = D.euler_from_pred(x[i], P, s0, s1)
        want = D.step(x[i], s0, s1, float(plan["scale"][i]), prm, "euler")
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12), i


@pytest.mark.parametrize("k", [0, 2, 5])
def test_rows_heun_two_calls_equal_inline_step(k):
    """Heun as two calls (predictor stores d and x~; the model runs at x~;
    corrector) equals the inline Heun step, including the last step."""
    inp, sig, table, cov, x = _rows_case("heun")
    sp = inp.spec
    t = inp.start_step.astype(np.int64) + k
    plan = D.build_plan(t, sp.steps, sp.num_buckets, table, inp.cfg_override, cov)
    act = [i for i in range(sp.n) if plan["bucket_id"][i] >= 0]
    rows = _stand_in_rows(inp, plan, x, {i: float(sig[t[i]]) for i in act})
    xt = x.copy()
    ds = {}
    for i in act:
        prm = D.sample_params(inp, i)
        P = D.rows_pred(rows, plan, i, float(plan["scale"][i]), prm.x_orig, prm.mask)
        ds[i], xt[i] = D.heun_predict(x[i], P, float(sig[t[i]]), float(sig[t[i] + 1]))
    rows2 = _stand_in_rows(inp, plan, xt, {i: float(sig[t[i] + 1]) for i in act})
    for i in act:
        prm = D.sample_params(inp, i)
        s0, s1 = float(sig[t[i]]), float(sig[t[i] + 1])
        want = D.step(x[i], s0, s1, float(plan["scale"][i]), prm, "heun")
        if ds[i] is None:
            got = xt[i]  # last step: the predictor's output is final
            assert s1 == 0.0
        else:
            P2 = D.rows_pred(rows2, plan, i, float(plan["scale"][i]), prm.x_orig, prm.mask)
            got = D.heun_correct(x[i], ds[i], P2, s0, s1)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12), i


def test_rows_scale_one_reads_no_uncond_row():
    inp, sig, table, cov, x = _rows_case("euler")
    sp = inp.spec
    plan = D.build_plan(inp.start_step.astype(np.int64), sp.steps, sp.num_buckets, table,
                        inp.cfg_override, cov)
    rows = _stand_in_rows(inp, plan, x, {i: float(sig[inp.start_step[i]]) for i in range(sp.n)})
    for i in range(sp.n):
        if plan["bucket_id"][i] < 0 or plan["scale"][i] != np.float32(1):
            continue
        poisoned = rows.copy()
        poisoned[:plan["n_uncond"]] = np.nan  # every uncond row
        got = D.rows_pred(poisoned, plan, i, 1.0)
        assert np.array_equal(got, rows[plan["cond_row"][i]])


def test_rows_mirror_within_tolerance_and_exact_cases():
    rng = np.random.default_rng(11)
    C, H, Wd = 3, 8, 16
    for trial in range(20):
        x = rng.standard_normal((C, H, Wd)).astype(np.float32) * 3
        c = rng.standard_normal((C, H, Wd)).astype(np.float32)
        u = rng.standard_normal((C, H, Wd)).astype(np.float32)
        xo = rng.standard_normal((C, H, Wd)).astype(np.float32)
        m = (rng.random((H, Wd)) < 0.5).astype(np.float32)
        w = [0.0, 1.0, 2.5, 7.0][trial % 4]
        s0, s1 = np.float32(rng.uniform(0.5, 10)), np.float32(rng.uniform(0.05, 0.4))
        pm = M.rows_pred32(c, u, w, m, xo)
        pd = D.inpaint_blend(D.cfg_combine(u.astype(np.float64), c.astype(np.float64), w), xo, m)
        assert np.allclose(pm, pd, rtol=0, atol=1e-5 * max(1.0, np.abs(pd).max()))
        e_m = M.rows_euler32(x, pm, s0, s1)
        e_d = D.euler_from_pred(x.astype(np.float64), pm.astype(np.float64), float(s0), float(s1))
        assert np.abs(e_m - e_d).max() <= 1e-5 * np.abs(e_d).max()
        d_m, xt_m = M.rows_heun_predict32(x, pm, s0, s1)
        d_d, xt_d = D.heun_predict(x.astype(np.float64), pm.astype(np.float64), float(s0), float(s1))
        assert np.abs(xt_m - xt_d).max() <= 1e-5 * np.abs(xt_d).max()
        h_m = M.rows_heun_correct32(x, d_m, c, s0, s1)
        h_d = D.heun_correct(x.astype(np.float64), d_d, c.astype(np.float64), float(s0), float(s1))
        assert np.abs(h_m - h_d).max() <= 1e-5 * np.abs(h_d).max()
    # exact cases: scale 1 takes c itself, mask 0 takes the original latent,
    # sigma' = 0 lands on the prediction
    assert np.array_equal(M.rows_pred32(c, u * np.nan, 1.0), c)
    assert np.array_equal(M.rows_pred32(c, u, 3.0, np.zeros((H, Wd), np.float32), xo), xo)
    assert np.array_equal(M.rows_euler32(x, c, s0, 0.0), c)
    assert M.rows_heun_predict32(x, c, s0, 0.0)[0] is None


# ---------------------------------------------------------------- schedule and curve variants

@pytest.mark.parametrize("p2", [0.5, 0.3, 0.8])
def test_mid_peak_curve_is_the_triangle(p2):
    """p0 at both ends, p1 at the peak, linear between: numpy's piecewise-linear
    interpolation through (0, p0), (p2, p1), (1, p0)."""
    for nb in (1, 2, 5, 11, 16):
        u = np.array([0.0]) if nb == 1 else np.arange(nb) / (nb - 1)
        want = np.interp(u, [0.0, p2, 1.0], [1.2, 2.0, 1.2]).astype(np.float32)
        got = D.bucket_table("mid_peak", 1.2, 2.0, p2, nb)
        assert np.allclose(got, want, rtol=0, atol=2e-7), nb
    t = D.bucket_table("mid_peak", 1.2, 2.0, 0.5, 11)
    assert t[0] == t[-1] == np.float32(1.2) and t[5] == np.float32(2.0)
    assert np.array_equal(t, t[::-1])
    with pytest.raises(ValueError):
        D.curve_value("mid_peak", 1.2, 2.0, 1.0, 0.5)


def test_crop_sigmas_stages_compose_and_force():
    full, _ = D.sigma_schedule(14.6, 0.03, 30)
    assert np.array_equal(D.crop_sigmas(full, 0), full)
    assert np.array_equal(D.crop_sigmas(full, 0, 99), full)
    for k in (1, 7, 29):
        a, b = D.crop_sigmas(full, 0, k), D.crop_sigmas(full, k)
        assert a.size == k + 1 and b.size == 31 - k
        assert a[-1] == b[0]                                  # the stages meet
        assert np.array_equal(np.concatenate([a[:-1], b]), full)
        f = D.crop_sigmas(full, 0, k, force_full_denoise=True)
        assert np.array_equal(f[:-1], a[:-1]) and f[-1] == 0  # only the end changes
    assert np.array_equal(D.crop_sigmas(full, 12, force_full_denoise=True), full[12:])  # already ends at 0
    assert D.crop_sigmas(full, 30).size == 1                  # nothing left to run
    with pytest.raises(ValueError):
        D.crop_sigmas(full, 8, 5)


def test_within_bucket_interpolation_follows_the_curve():
    """A linear curve interpolated within buckets is the continuous curve
    itself: scale(t) = g(t/steps) for any bucket count (up to float32)."""
    for steps, nb in ((50, 8), (30, 16), (20, 8), (7, 3), (12, 1), (10, 64)):
        lo, hi = D.bucket_bounds("linear", 2.0, 1.2, 0.0, nb)
        assert np.array_equal(lo[1:], hi[:-1])  # neighbouring buckets meet
        plan = D.build_plan(np.arange(steps), steps, nb, lo, table_end=hi)
        g = 2.0 + (1.2 - 2.0) * (np.arange(steps) / steps)
        assert np.allclose(plan["scale"], g, rtol=0, atol=4e-7), (steps, nb)
        for t in range(steps):  # at a bucket's first step the scale is its start value
            b = D.bucket_id(t, steps, nb)
            if t * nb == b * steps:
                assert plan["scale"][t] == lo[b]


def test_within_bucket_interpolation_of_a_step_curve_ramps_inside_one_bucket():
    # front-high 2.0 -> 1.2 at 20%: with 4 buckets of 25%, the edge at 20%
    # falls inside bucket 0, whose scale ramps from 2.0 to 1.2
    lo, hi = D.bucket_bounds("front_high", 2.0, 1.2, 0.2, 4)
    assert list(lo) == [np.float32(2.0)] + [np.float32(1.2)] * 3
    assert list(hi) == [np.float32(1.2)] * 4
    plan = D.build_plan(np.arange(20), 20, 4, lo, table_end=hi)
    assert np.allclose(plan["scale"][:5], 2.0 - 0.8 * np.arange(5) / 5, atol=1e-7)
    assert (plan["scale"][5:] == np.float32(1.2)).all()



# ---------------------------------------------------------------- per-cond validity ranges

def test_region_validity_boundaries_by_enumeration():
    # [0.25, 0.5) of 20 steps: progress 5/20 .. 9/20 exactly
    assert [t for t in range(20) if D.region_valid((0.25, 0.5), t, 20)] == [5, 6, 7, 8, 9]
    assert all(D.region_valid(None, t, 20) for t in range(20))
    assert not any(D.region_valid((1.0, 2.0), t, 20) for t in range(20))
    assert [t for t in range(7) if D.region_valid((0.0, 1.0), t, 7)] == list(range(7))


def test_full_ranges_change_nothing_and_an_unused_region_is_absent():
    base = W.small_spec(n=4, C=2, H=12, W=16, steps=6, regions=2, region_ranges=True, seed=9)
    inp = W.make_inputs(base)
    plain = W.make_inputs(dataclasses_replace(base, region_ranges=False))
    inp.region_range[:] = (0.0, 1.5)
    assert np.array_equal(D.trajectory(inp), D.trajectory(plain))
    # region 1 never valid == the samples with region 1 removed
    inp.region_range[:, 1] = (2.0, 3.0)
    one = W.make_inputs(dataclasses_replace(base, region_ranges=False))
    one.region_count[:] = np.minimum(one.region_count, 1)
    assert np.array_equal(D.trajectory(inp), D.trajectory(one))


def test_no_valid_region_means_no_guidance():
    """A regional sample with none of its regions valid: C = U everywhere, so
    the prediction is the uncond prediction whatever the scale."""
    base = W.small_spec(n=1, C=3, H=10, W=12, steps=5, regions=2, region_ranges=True,
                        inpaint=False, seed=4)
    inp = W.make_inputs(base)
    inp.region_range[:] = (0.9, 1.0)  # not valid at step 0
    prm = D.sample_params(inp, 0, 0)
    assert prm.regional and not prm.regions
    x = np.random.default_rng(2).standard_normal((3, 10, 12))
    u = D.denoise(x, 3.0, prm.mu_u, prm.s2)
    for w in (0.0, 1.0, 7.5):
        assert np.array_equal(D.guided_pred(x, 3.0, w, prm), u)
    assert not D.coverage(inp, np.array([0]))[0]  # the uncond branch is then needed


def test_area_box_rounds_exact_products_ties_up():
    # Every tie (k + 1/2)/n of every extent n <= 256, and the float64 values on
    # either side of it: the offset and the side are the integer nearest to the
    # exact product, found by search, then clamped.  The other plausible rules
    # each give a different slice somewhere in this set.
    from area_cases import near_tie_fractions, nearest_by_search
    alt = {"floor": lambda f, n: math.floor(f * n),
           "half_even": lambda f, n: round(Fraction(f) * n),
           "float64_half_up": lambda f, n: math.floor(f * n + 0.5)}
    caught = dict.fromkeys(alt, 0)
    cases = 0
    for n in range(1, 257):
        for f in near_tie_fractions(n):
            m = nearest_by_search(f, n)
            y0, y1, x0, x1 = D.area_box((f, 0.0, 0.0, f), n, n)
            assert (y0, y1) == (min(max(m, 0), n - 1), min(max(m, 0), n - 1) + 1), (n, f)
            assert (x0, x1) == (0, min(max(m, 1), n)), (n, f)
            cases += 1
            for name, rule in alt.items():
                a = rule(f, n)
                if min(max(a, 0), n - 1) != y0 or min(max(a, 1), n) != x1 - x0:
                    caught[name] += 1
    assert cases == 3 * sum(range(1, 257))
    assert all(v > 0 for v in caught.values()), caught


def test_bf16_flip_carried_to_the_end_pins_the_final_bar():
    # The Heun bf16 workload's one final element whose fp32 order (mode M,
    # which the GPU reproduces bit for bit) and float64 definition (mode D)
    # differ by more than max(2e-2, 1 bf16 ulp): sample 44, element
    # (3, 26, 60).  The two trajectories take neighbouring bf16 codes at an
    # early step while |x| is large (a one-ulp flip of a state of magnitude
    # >= 4); the later steps carry it to the end, where it is 4 ulps of the
    # final value and inside the carried-flip bound.
    from gpu_helpers import bf16_ulp, storage_flip_bound
    inp = W.make_inputs(W.config("throughput_bf16_heun"))
    sub = inp.subset([44])
    q = (0, 3, 26, 60)
    xm, ms = M.trajectory32(sub, keep=True)
    xd, ds = D.trajectory(sub, keep=True)
    err = abs(float(xm[q]) - float(xd[q]))
    assert (float(xd[q]), float(xm[q])) == (-1.46875, -1.5)
    assert err > max(2e-2, float(bf16_ulp(xd[q])))
    assert err <= storage_flip_bound(inp, 44)[q[1:]]
    first = next(k for k in range(len(ms)) if ms[k][q] != ds[k][q])
    assert abs(float(ds[first][q])) >= 4.0
    assert abs(float(ms[first][q]) - float(ds[first][q])) == float(bf16_ulp(ds[first][q]))
    # every other element of the sample is inside max(2e-2, 1 ulp), and all inside the bound
    e = np.abs(xm.astype(np.float64) - xd)[0]
    assert int((e > np.maximum(2e-2, bf16_ulp(xd[0]))).sum()) == 1
    assert np.all(e <= storage_flip_bound(inp, 44))


# ---------------------------------------------------------------- continuous batching

def _schedule_by_events(start, steps, n, Q, L, ring):
    """The same schedule from events: a heap of (launch at which a slot is free
    again, slot); each event takes the next request for `steps` launches."""
    import heapq
    req = np.full((L, n), -1, np.int64)
    tt = np.full((L, n), -1, np.int64)
    join = np.zeros((L, n), bool)
    spans = [(s, s, 0, int(start[s])) for s in range(n)]
    heap = [(steps - int(start[s]), s) for s in range(n)]
    heapq.heapify(heap)
    nxt = n
    while heap:
        k, s = heapq.heappop(heap)
        if k >= L or (not ring and nxt >= Q):
            continue
        spans.append((s, nxt % Q if ring else nxt, k, 0))
        nxt += 1
        heapq.heappush(heap, (k + steps, s))
    for s, r, k0, t0 in spans:
        for j in range(steps - t0):
            if k0 + j < L:
                req[k0 + j, s], tt[k0 + j, s], join[k0 + j, s] = r, t0 + j, j == 0
    return req, tt, join


def test_serve_schedule_matches_event_simulation():
    rng = np.random.default_rng(77)
    for _ in range(300):
        n = int(rng.integers(1, 6))
        Q = int(rng.integers(n, 3 * n + 2))
        steps = int(rng.integers(1, 7))
        L = int(rng.integers(1, 4 * steps + 6))
        ring = bool(rng.integers(0, 2))
        start = rng.integers(0, steps, n)
        got = D.serve_schedule(start, steps, n, Q, L, ring)
        want = _schedule_by_events(start, steps, n, Q, L, ring)
        for g, w in zip(got, want):
            assert np.array_equal(g, w), (n, Q, steps, L, ring, start)
    # a drained queue: every request served once, for steps - start launches
    start = np.array([2, 0, 3])
    req, tt, join = D.serve_schedule(start, 4, 3, 8, 20)
    served = {int(r): int((req == r).sum()) for r in np.unique(req[req >= 0])}
    assert sorted(served) == list(range(8))
    assert all(served[r] == (4 - start[r] if r < 3 else 4) for r in served)
    assert (req[-1] == -1).all() and int(join.sum()) == 8


@pytest.mark.parametrize("kw", [dict(dtype="f32", regions=2, inpaint=True),
                                dict(dtype="bf16", sampler="heun", regions=1),
                                # validity ranges follow each request's own progress
                                dict(dtype="f32", regions=2, region_ranges=True, inpaint=True),
                                dict(dtype="bf16", sampler="heun", regions=2, region_ranges=True,
                                     bucket_interp=True, curve=W.Curve("mid_peak", 1.2, 3.0, 0.4))])
def test_served_requests_equal_their_solo_runs(kw):
    # Per-request independence through the queue: each request's state after
    # its last step equals its own trajectory run alone (from its start step,
    # or 0 when it came from the queue), bit for bit, in both modes.
    sp = W.small_spec(n=7, C=2, H=8, W=16, steps=4, num_buckets=3, feather=2, **kw)
    inp = W.make_inputs(sp)
    n_slots, L = 3, 12
    xd, dstates, (req, tt, join) = D.serve_trajectory(inp, n_slots, L, keep=True)
    xm, mstates, _ = M.serve_trajectory32(inp, n_slots, L, keep=True)
    for r in range(sp.n):
        where = np.argwhere((req == r) & (tt == sp.steps - 1))
        assert len(where) == 1, r
        k, s = (int(v) for v in where[0])
        solo = inp.subset([r])
        solo.start_step[:] = inp.start_step[r] if r < n_slots else 0
        left = sp.steps - int(solo.start_step[0])
        assert np.array_equal(dstates[k][s], D.trajectory(solo, launches=left)[0]), r
        assert np.array_equal(mstates[k][s], M.trajectory32(solo, launches=left)[0]), r
