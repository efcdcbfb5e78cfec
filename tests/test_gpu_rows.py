"""guided_step_rows (branch predictions materialised by a model, in the bucket
plan's [uncond (compacted) | cond] layout) against the oracle.

Bit for bit against the float32 mirror (mode M) and within the per-step bound
of the float64 definition (mode D), for Euler and for the two Heun calls, with
skipped uncond rows, scale-1 samples whose uncond rows hold NaN (never read),
last steps, inactive samples and the scalar path.
"""
import numpy as np
import pytest
import torch

from oracle import definition as D
from oracle import mirror32 as M

from gpu_helpers import bf16_ulp, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bucketed_classifier_free_amd
    bucketed_classifier_free_amd.load()  # fails loudly without libbcg.so


TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _dev(a, dtype="f32"):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(TDT[dtype])


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


class Case:
    """Seeded inputs of one materialised step: state, plan, rows, mask."""

    def __init__(self, n=7, C=3, H=16, W=24, dtype="f32", inpaint=False, steps=6, seed=0,
                 rows_scale=1.0):
        from bucketed_classifier_free_amd import api
        rng = np.random.default_rng(seed)
        self.n, self.C, self.H, self.W, self.dtype, self.steps = n, C, H, W, dtype, steps
        st = lambda a: M._store(np.asarray(a, np.float32), dtype)
        self.sig, _ = D.sigma_schedule(14.6, 0.03, steps, 1.0)
        self.t = rng.integers(0, steps, n).astype(np.int32)
        self.t[0] = steps - 1                      # a last step
        if n > 3:
            self.t[1], self.t[2] = -1, steps        # inactive
        table = api.bucket_table("linear", 2.0, 1.0, 0.0, 3)
        ov = np.full(n, np.nan, np.float32)
        ov[3::3] = 1.0
        ov[4::5] = 0.0
        self.covered = (rng.random(n) < 0.6).astype(np.uint8)
        self.plan = api.bcg_plan_build(self.t, steps, table, covered=self.covered, cfg_override=ov)
        p = self.plan
        self.rows = p.n_uncond + p.n_active
        self.x = st(rng.standard_normal((n, C, H, W)) * 4)
        self.xo = st(rng.standard_normal((n, C, H, W))) if inpaint else None
        self.mask = (rng.random((n, 1, H, W)) < 0.5).astype(np.float32) if inpaint else None
        self.pred = self.make_rows(rng, rows_scale)

    def make_rows(self, rng, scale=1.0):
        p = self.plan
        rows = M._store(rng.standard_normal((self.rows, self.C, self.H, self.W)) * scale, self.dtype)
        for i in range(self.n):  # scale-1 samples must not read their (kept) uncond rows
            if p.bucket_id[i] >= 0 and p.scale[i] == np.float32(1) and p.uncond_row[i] >= 0:
                rows[p.uncond_row[i]] = np.nan
        return rows

    def device(self):
        p = self.plan
        self.d_plan = dict(order=_i32(p.order), step_idx=_i32(self.t),
                           scale=torch.from_numpy(p.scale).cuda(), uncond_row=_i32(p.uncond_row),
                           cond_row=_i32(p.cond_row))
        self.d_sig = torch.from_numpy(self.sig).cuda()
        return self

    def active(self):
        return [i for i in range(self.n) if self.plan.bucket_id[i] >= 0]

    def pb32(self, rows, i):
        p = self.plan
        c = rows[p.cond_row[i]]
        u = rows[p.uncond_row[i]] if p.uncond_row[i] >= 0 else None
        return M.rows_pred32(c, u, p.scale[i], None if self.mask is None else self.mask[i, 0],
                             None if self.xo is None else self.xo[i])

    def pbD(self, rows, i):
        plan = dict(cond_row=self.plan.cond_row, uncond_row=self.plan.uncond_row)
        return D.rows_pred(rows.astype(np.float64), plan, i, float(self.plan.scale[i]),
                           None if self.xo is None else self.xo[i].astype(np.float64),
                           None if self.mask is None else self.mask[i, 0])

    def call(self, phase, x, out, rows, d=None, x_tilde=None, cache_hint=0, launch_vpt=0):
        from bucketed_classifier_free_amd import api
        api.guided_step_rows(x, out, _dev(rows, self.dtype), self.d_sig, n_active=self.plan.n_active,
                             phase=phase, d=d, x_tilde=x_tilde,
                             x_orig=None if self.xo is None else _dev(self.xo, self.dtype),
                             mask=None if self.mask is None else _dev(self.mask),
                             cache_hint=cache_hint, launch_vpt=launch_vpt, **self.d_plan)


def _check_D(case, got, ref, tag):
    scale = max(np.abs(ref).max(), 1e-30)
    err = np.abs(got.astype(np.float64) - ref)
    if case.dtype == "f32":
        assert err.max() <= 1e-5 * scale, f"{tag}: {err.max() / scale:.3g} rel"
    else:
        assert np.all(err <= 0.5 * bf16_ulp(ref) + 1e-5 * scale), tag


KW = [dict(dtype="f32"), dict(dtype="bf16"), dict(dtype="f32", inpaint=True),
      dict(dtype="bf16", inpaint=True), dict(dtype="f32", H=13, W=21),
      dict(dtype="bf16", H=13, W=21, inpaint=True), dict(dtype="bf16", n=3, C=1, H=1, W=8)]


# The walk is a ring of four single-channel stages: channel counts that are not
# a multiple of four end on a partial pass (C = 5, 6, 7, 9), with both cache
# hints; lanes forced to take two or three vectors (ragged last pass).
RING = [dict(dtype="f32", C=5), dict(dtype="bf16", C=6, inpaint=True, hint=1),
        dict(dtype="f32", C=7, inpaint=True), dict(dtype="bf16", C=9, hint=1),
        dict(dtype="bf16", C=5, inpaint=True, hint=1), dict(dtype="f32", C=9, inpaint=True, hint=1),
        dict(dtype="bf16", C=7), dict(dtype="f32", C=6),
        dict(dtype="bf16", C=16, H=40, W=64, vpt=2, hint=1), dict(dtype="f32", C=5, H=40, W=64, vpt=3),
        dict(dtype="bf16", C=6, H=40, W=64, vpt=3, inpaint=True, hint=1)]


def _opts(kw):
    kw = dict(kw)
    return kw.pop("hint", 0), kw.pop("vpt", 0), kw


@pytest.mark.parametrize("kw", KW + RING)
def test_rows_euler_matches_oracle(kw):
    hint, vpt, kw = _opts(kw)
    case = Case(**kw).device()
    x = _dev(case.x, case.dtype)
    out = torch.full_like(x, float("nan"))
    case.call("euler", x, out, case.pred, cache_hint=hint, launch_vpt=vpt)
    torch.cuda.synchronize()
    got = to_np(out)
    for i in range(case.n):
        if i not in case.active():
            assert np.isnan(got[i]).all(), f"inactive sample {i} written"
            continue
        s0, s1 = case.sig[case.t[i]], case.sig[case.t[i] + 1]
        ref_m = M._store(M.rows_euler32(case.x[i], case.pb32(case.pred, i), s0, s1), case.dtype)
        assert np.array_equal(got[i], ref_m), f"sample {i} differs from mode M"
        ref_d = D.euler_from_pred(case.x[i].astype(np.float64), case.pbD(case.pred, i), float(s0), float(s1))
        _check_D(case, got[i], ref_d, f"sample {i}")


@pytest.mark.parametrize("kw", KW + RING)
def test_rows_heun_two_calls_match_oracle(kw):
    hint, vpt, kw = _opts(kw)
    case = Case(**kw).device()
    rng = np.random.default_rng(99)
    x = _dev(case.x, case.dtype)
    xt = torch.full_like(x, float("nan"))
    d = torch.full(x.shape, float("nan"), dtype=torch.float32, device="cuda")
    case.call("heun_predict", x, xt, case.pred, d=d, cache_hint=hint, launch_vpt=vpt)
    rows2 = case.make_rows(rng)
    out = torch.full_like(x, float("nan"))
    case.call("heun_correct", x, out, rows2, d=d, x_tilde=xt, cache_hint=hint, launch_vpt=vpt)
    torch.cuda.synchronize()
    g_xt, g_d, got = to_np(xt), d.cpu().numpy(), to_np(out)
    for i in range(case.n):
        if i not in case.active():
            assert np.isnan(got[i]).all() and np.isnan(g_xt[i]).all()
            continue
        s0, s1 = case.sig[case.t[i]], case.sig[case.t[i] + 1]
        d_m, xt_m = M.rows_heun_predict32(case.x[i], case.pb32(case.pred, i), s0, s1)
        assert np.array_equal(g_xt[i], M._store(xt_m, case.dtype)), f"x~ of sample {i}"
        if d_m is None:  # last step: P, and the corrector copies it
            assert np.isnan(g_d[i]).all()
            assert np.array_equal(got[i], g_xt[i])
            continue
        assert np.array_equal(g_d[i], d_m), f"d of sample {i}"
        ref_m = M._store(M.rows_heun_correct32(case.x[i], d_m, case.pb32(rows2, i), s0, s1), case.dtype)
        assert np.array_equal(got[i], ref_m), f"sample {i} differs from mode M"
        dd, _ = D.heun_predict(case.x[i].astype(np.float64), case.pbD(case.pred, i), float(s0), float(s1))
        ref_d = D.heun_correct(case.x[i].astype(np.float64), dd, case.pbD(rows2, i), float(s0), float(s1))
        _check_D(case, got[i], ref_d, f"sample {i}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rows_in_place_and_streaming_hint_identical(dtype):
    case = Case(n=9, C=4, H=16, W=32, dtype=dtype, inpaint=True, seed=5).device()
    x = _dev(case.x, dtype)
    a = x.clone()
    case.call("euler", x, a, case.pred)
    b = x.clone()
    case.call("euler", b, b, case.pred)  # in place
    c = x.clone()
    case.call("euler", x, c, case.pred, cache_hint=1)  # nontemporal streams
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_rows_large_shape_sampled():
    """The large workload's shape (256 x 16x128x128 bf16, 8 buckets), every
    slot active, streaming hint: sampled samples against the mirror."""
    case = Case(n=256, C=16, H=128, W=128, dtype="bf16", steps=50, seed=8).device()
    x = _dev(case.x, "bf16")
    out = torch.full_like(x, float("nan"))
    case.call("euler", x, out, case.pred, cache_hint=1)
    torch.cuda.synchronize()
    idx = [0, 3, 37, 101, 255]
    got = to_np(out[idx])
    for k, i in enumerate(idx):
        if i not in case.active():
            assert np.isnan(got[k]).all()
            continue
        s0, s1 = case.sig[case.t[i]], case.sig[case.t[i] + 1]
        ref = M._store(M.rows_euler32(case.x[i], case.pb32(case.pred, i), s0, s1), "bf16")
        assert np.array_equal(got[k], ref), i


@pytest.mark.parametrize("kw", [dict(dtype="f32"), dict(dtype="bf16", inpaint=True),
                                dict(dtype="bf16", n=40, C=4, H=32, W=32),
                                dict(dtype="bf16", n=256, C=16, H=128, W=128, steps=50, hint=1)])
def test_rows_dplan_equals_plan_then_update(kw):
    """guided_step_rows_dplan = bcg_plan_device (the next step's plan) followed by
    guided_step_rows: the update and every plan output bit for bit.  The last
    case is the large workload's shape with the streaming hint: a grid of
    several resident rounds, whose launch sizes its dynamic LDS to bound the
    waves per CU, with the plan workgroup in it."""
    from bucketed_classifier_free_amd import api
    kw = dict(kw)
    hint = kw.pop("hint", 0)
    case = Case(**kw).device()
    n = case.n
    table = torch.from_numpy(api.bucket_table("linear", 2.0, 1.0, 0.0, 3)).cuda()
    rng = np.random.default_rng(11)
    t_next = _i32(rng.integers(-1, case.steps + 1, n))          # some inactive, some past the end
    ov = torch.from_numpy(np.where(rng.random(n) < 0.3, np.float32(1.0), np.float32(np.nan))).cuda()
    cov = _i32(rng.random(n) < 0.7)

    def plan_into():
        out = api.device_plan_arrays(n, 3)
        for v in out.values():
            v.fill_(-7)
        so = torch.full((n,), -7, dtype=torch.int32, device="cuda")
        return out, so

    opt = dict(x_orig=None if case.xo is None else _dev(case.xo, case.dtype),
               mask=None if case.mask is None else _dev(case.mask))
    rows = _dev(case.pred, case.dtype)
    x = _dev(case.x, case.dtype)

    ref_plan, ref_so = plan_into()
    api.bcg_plan_device(case.steps, table, t_next, step_out=ref_so, cfg_override=ov, covered=cov,
                        wrap=True, out=ref_plan)
    ref = x.clone()
    api.guided_step_rows(x, ref, rows, case.d_sig, n_active=case.plan.n_active, phase="euler",
                         cache_hint=hint, **case.d_plan, **opt)

    got_plan, got_so = plan_into()
    pl = api.device_plan(case.steps, table, t_next, step_out=got_so, cfg_override=ov, covered=cov,
                         wrap=True, out=got_plan)
    got = x.clone()
    api.guided_step_rows_dplan(x, got, rows, case.d_sig, n_active=case.plan.n_active, plan=pl,
                               phase="euler", cache_hint=hint, **case.d_plan, **opt)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16 if case.dtype == "bf16" else torch.int32),
                       ref.view(torch.int16 if case.dtype == "bf16" else torch.int32))
    assert torch.equal(got_so, ref_so)
    for k in ref_plan:
        g, r = got_plan[k], ref_plan[k]
        if g.dtype == torch.float32:
            g, r = g.view(torch.int32), r.view(torch.int32)
        assert torch.equal(g, r), k
