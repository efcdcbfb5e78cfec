"""Schedule and guidance variants on the GPU: staged sampling (sigma_crop),
force_full_denoise and the mid-peak curve, against the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import definition as D
from oracle import mirror32 as M

from gpu_helpers import to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bucketed_classifier_free_amd
    bucketed_classifier_free_amd.load()  # fails loudly without libbcg.so


def _sampler(inp, **kw):
    from bucketed_classifier_free_amd import GuidedSampler
    return GuidedSampler.from_inputs(inp, **kw)


def _staged_spec(sampler):
    # one bucket and a common start: the guidance of a step does not depend on
    # where the schedule was cut
    return W.small_spec(n=4, C=3, H=16, W=24, regions=2, inpaint=True, steps=12, num_buckets=1,
                        curve=W.Curve("const", 3.0), mixed_start=False, skip_frac=0.0,
                        sampler=sampler, feather=3)


@pytest.mark.parametrize("sampler", ["euler", "heun"])
@pytest.mark.parametrize("cut", [1, 5, 11])
def test_staged_sampling_equals_full_run(sampler, cut):
    inp = W.make_inputs(_staged_spec(sampler))
    full = _sampler(inp).run()
    x = _sampler(inp, sigma_last=cut).run()
    _sampler(inp, sigma_start=cut).run(x)
    torch.cuda.synchronize()
    assert torch.equal(x, full)


@pytest.mark.parametrize("sampler", ["euler", "heun"])
def test_force_full_denoise_ends_on_prediction(sampler):
    inp = W.make_inputs(_staged_spec(sampler))
    cut = 5
    a = _sampler(inp, sigma_last=cut, force_full_denoise=True)
    assert a.sigmas[-1] == 0 and a.steps == cut
    x = a.run()
    y = _sampler(inp, sigma_last=cut - 1).run()
    torch.cuda.synchronize()
    sig = a.sigmas
    plan = a.plan(cut - 1)  # the last step of the forced schedule
    got, before = to_np(x), to_np(y)
    for i in range(inp.spec.n):
        ref = M.step32(before[i], sig[cut - 1], np.float32(0), plan.scale[i], plan.uncond_row[i] >= 0,
                       M.params32(inp, i), sampler)
        assert np.array_equal(got[i], M._store(ref, inp.spec.dtype)), i
    assert not torch.equal(x, _sampler(inp, sigma_last=cut).run())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mid_peak_curve_trajectory_matches_mirror(dtype):
    sp = W.small_spec(n=5, C=2, H=16, W=16, steps=10, num_buckets=8, dtype=dtype,
                      curve=W.Curve("mid_peak", 1.2, 3.0, 0.4), regions=1)
    inp = W.make_inputs(sp)
    s = _sampler(inp)
    assert np.array_equal(s.table, D.bucket_table("mid_peak", 1.2, 3.0, 0.4, 8))
    x = s.run()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(x), M.trajectory32(inp))


@pytest.mark.parametrize("dtype,curve", [("f32", W.Curve("front_high", 2.0, 1.2, 0.2)),
                                         ("bf16", W.Curve("mid_peak", 1.2, 3.0, 0.4)),
                                         ("f32", W.Curve("linear", 2.0, 1.0))])
def test_interpolated_scale_trajectory_matches_mirror(dtype, curve):
    sp = W.small_spec(n=6, C=2, H=16, W=16, steps=12, num_buckets=4, dtype=dtype, curve=curve,
                      regions=1, bucket_interp=True)
    inp = W.make_inputs(sp)
    s = _sampler(inp)
    lo, hi = D.bucket_bounds(curve.kind, curve.p0, curve.p1, curve.p2, 4)
    assert np.array_equal(s.table, lo) and np.array_equal(s.table_end, hi)
    x = s.run()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(x), M.trajectory32(inp))


def test_interpolated_scale_device_plan_matches_oracle_and_host_path():
    from bucketed_classifier_free_amd import api
    sp = W.small_spec(n=9, C=2, H=16, W=24, steps=20, num_buckets=3, regions=2,
                      curve=W.Curve("linear", 2.0, 1.0), bucket_interp=True)
    inp = W.make_inputs(sp)
    sig, table, cov = D.run_setup(inp)
    s = _sampler(inp)
    xh = s.run()
    x = s.init_state()
    t0 = s.step_indices(0)
    bufs = [torch.from_numpy(t0).cuda(), torch.empty(sp.n, dtype=torch.int32, device="cuda")]
    out = api.device_plan_arrays(sp.n, sp.num_buckets)
    for k in range(sp.steps):
        s.dplan_step(x, bufs[k & 1], bufs[(k + 1) & 1], plan_out=out)
        torch.cuda.synchronize()
        ref = D.build_plan(s.step_indices(k), sp.steps, sp.num_buckets, table, inp.cfg_override, cov,
                           D.table_end(inp))
        assert np.array_equal(out["scale"].cpu().numpy().view(np.uint32), ref["scale"].view(np.uint32)), k
        assert np.array_equal(out["uncond_row"].cpu().numpy(), ref["uncond_row"]), k
    assert torch.equal(x, xh)


@pytest.mark.parametrize("dtype,sampler", [("f32", "euler"), ("bf16", "heun"), ("f32", "heun")])
def test_region_validity_ranges_trajectory_matches_mirror(dtype, sampler):
    sp = W.small_spec(n=7, C=3, H=16, W=24, steps=10, num_buckets=3, dtype=dtype, sampler=sampler,
                      regions=3, region_ranges=True, inpaint=(sampler == "heun"), skip_frac=0.5,
                      curve=W.Curve("linear", 2.0, 1.0), feather=3)
    inp = W.make_inputs(sp)
    inp.region_range[0] = (0.95, 1.0)  # sample 0: no region valid for most steps
    s = _sampler(inp)
    x = s.run()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(x), M.trajectory32(inp))


def test_region_validity_ranges_device_plan_and_loop_equal_host_path():
    from bucketed_classifier_free_amd import api
    sp = W.small_spec(n=9, C=2, H=16, W=24, steps=12, num_buckets=4, regions=2,
                      region_ranges=True, skip_frac=0.5, curve=W.Curve("linear", 2.0, 1.0))
    inp = W.make_inputs(sp)
    s = _sampler(inp)
    xh = s.run()
    # fused device-plan steps reading the records their plans write
    x = s.init_state()
    t0 = s.step_indices(0)
    steps = [torch.from_numpy(t0).cuda(), torch.empty(sp.n, dtype=torch.int32, device="cuda")]
    recs = [torch.from_numpy(s.records(0)).cuda(), torch.zeros((sp.n, 4), device="cuda")]
    for k in range(sp.steps):
        s.dplan_step(x, steps[k & 1], steps[(k + 1) & 1], record_in=recs[k & 1], record_out=recs[(k + 1) & 1])
        torch.cuda.synchronize()
        got = recs[(k + 1) & 1].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), s.records(k + 1).view(np.uint32)), k
    assert torch.equal(x, xh)
    # the native loop, host plans and device plans
    for dev in (False, True):
        y = s.init_state()
        loop = s.native_loop(y, upload_batch=2, device_plan=dev)
        loop.run(0, sp.steps)
        torch.cuda.synchronize()
        loop.close()
        assert torch.equal(y, xh), dev
