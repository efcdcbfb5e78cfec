"""Plans built on the device: bcg_plan_device, guided_step_dplan and the
native loop's device-plan mode.

Integer plan outputs are compared bit for bit with the oracle's build_plan
(SGLang BCG write-up, sections 2 and 3); latents bit for bit with the
host-plan path and with the oracle's fp32 mirror, which pin the same step.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import definition as D
from oracle import mirror32 as M

from gpu_helpers import to_dev, to_np

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


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def _next(t, steps, wrap):
    nt = t.astype(np.int64) + 1
    if wrap:
        nt = np.where(nt >= 0, nt % steps, nt)
    return nt.astype(np.int32)


def _check_plan(got, ref, n, tag=""):
    """Device plan outputs (torch) vs the oracle's plan (numpy), bit for bit."""
    g = {k: v.cpu().numpy() for k, v in got.items()}
    assert np.array_equal(g["bucket_id"], ref["bucket_id"]), tag
    assert np.array_equal(g["scale"].view(np.uint32), ref["scale"].view(np.uint32)), tag
    na, m = ref["n_active"], ref["n_uncond"]
    assert tuple(g["totals"]) == (na, m), tag
    assert np.array_equal(g["order"][:na], ref["order"]), tag
    assert (g["order"][na:] == -1).all(), tag
    assert np.array_equal(g["bucket_count"], ref["bucket_count"]), tag
    assert np.array_equal(g["bucket_offset"], ref["bucket_offset"]), tag
    assert np.array_equal(g["uncond_offset"], ref["uncond_offset"]), tag
    cond_row = np.full(n, -1, np.int32)
    cond_row[ref["order"]] = m + np.arange(na, dtype=np.int32)
    assert np.array_equal(g["cond_row"], cond_row), tag
    unc = np.full(n, -1, np.int32)
    uo = ref["order"][ref["need_uncond"][ref["order"]]]
    unc[uo] = np.arange(uo.size, dtype=np.int32)
    assert np.array_equal(g["uncond_row"], unc), tag


@pytest.mark.parametrize("n,nb,steps", [(1, 1, 10), (3, 8, 50), (64, 16, 30), (65, 8, 20),
                                        (700, 1024, 1000), (5000, 37, 53), (257, 64, 7)])
@pytest.mark.parametrize("wrap", [False, True])
def test_device_plan_matches_oracle(n, nb, steps, wrap):
    from bucketed_classifier_free_amd import api
    rng = np.random.default_rng(n * 31 + nb)
    table = api.bucket_table("linear", 2.0, 1.0, 0.0, nb)  # the last bucket is exactly 1.0
    override = np.where(rng.random(n) < 0.3, np.float32(1.0), np.float32(np.nan)).astype(np.float32)
    override[rng.random(n) < 0.1] = 3.5
    covered = rng.random(n) < 0.7
    out = api.device_plan_arrays(n, nb)
    d_table, d_ov, d_cov = (torch.from_numpy(table).cuda(), torch.from_numpy(override).cuda(),
                            _i32(covered))
    for rep in range(3):
        t = rng.integers(-3, steps + 3, n).astype(np.int32)
        if rep == 0:
            t[:] = np.arange(n) % steps  # every sample active
        step_in, step_out = _i32(t), torch.full((n,), -77, dtype=torch.int32, device="cuda")
        api.bcg_plan_device(steps, d_table, step_in, step_out=step_out, cfg_override=d_ov,
                            covered=d_cov, wrap=wrap, out=out)
        torch.cuda.synchronize()
        ref = D.build_plan(t, steps, nb, table, override, covered)
        _check_plan(out, ref, n, f"n={n} nb={nb} rep={rep}")
        assert np.array_equal(step_out.cpu().numpy(), _next(t, steps, wrap))
        assert np.array_equal(step_in.cpu().numpy(), t)  # input untouched


def test_device_plan_step_advance_only_and_defaults():
    from bucketed_classifier_free_amd import api
    n, steps = 300, 12
    t = np.arange(-5, n - 5).astype(np.int32) % 40 - 10
    table = torch.tensor([2.5, 1.0], dtype=torch.float32, device="cuda")
    step_in, step_out = _i32(t), torch.empty(n, dtype=torch.int32, device="cuda")
    api.bcg_plan_device(steps, table, step_in, step_out=step_out, wrap=True)
    out = api.device_plan_arrays(n, 2)
    api.bcg_plan_device(steps, table, step_in, out=out)  # no override, all covered
    torch.cuda.synchronize()
    assert np.array_equal(step_out.cpu().numpy(), _next(t, steps, True))
    _check_plan(out, D.build_plan(t, steps, 2, np.float32([2.5, 1.0])), n)


def _dplan_trajectory(s, x, launches, check_plans=None):
    """Launches 0..launches-1 with device plans, alternating step buffers."""
    from bucketed_classifier_free_amd import api
    t0 = s.step_indices(0)
    bufs = [_i32(t0), torch.empty_like(_i32(t0))]
    out = api.device_plan_arrays(s.n, s.nb)
    for k in range(launches):
        s.dplan_step(x, bufs[k & 1], bufs[(k + 1) & 1], plan_out=out)
        if check_plans is not None:
            torch.cuda.synchronize()
            check_plans(k, out, bufs[(k + 1) & 1])
    torch.cuda.synchronize()
    return x


@pytest.mark.parametrize("name", ["tiny", "mixed_bucket", "throughput_bf16_heun", "regional_inpaint"])
def test_dplan_trajectory_equals_host_plan_and_mirror(name):
    inp = W.make_inputs(W.config(name))
    sp = inp.spec
    sig, table, cov = D.run_setup(inp)
    s = _sampler(inp)
    xh = s.run()
    torch.cuda.synchronize()

    def check(k, out, nxt):
        t = s.step_indices(k)
        ref = D.build_plan(t, sp.steps, sp.num_buckets, table, inp.cfg_override, cov)
        _check_plan(out, ref, sp.n, f"{name} k={k}")
        assert np.array_equal(nxt.cpu().numpy(), s.step_indices(k + 1))

    xd = _dplan_trajectory(s, s.init_state(), sp.steps, check)
    assert torch.equal(xd, xh)
    idx = list(range(min(sp.n, 4)))
    xm = M.trajectory32(inp, samples=idx)
    assert np.array_equal(to_np(xd)[idx], xm[idx])


def test_dplan_inactive_samples_untouched_and_out_of_place():
    sp = W.small_spec(n=6, C=3, H=16, W=24, regions=2, inpaint=True, steps=8, feather=3)
    inp = W.make_inputs(sp)
    inp.start_step[:] = [0, -2, 3, 9, 7, -20]  # two not joined, one finished
    s = _sampler(inp)
    x = s.init_state()
    x0 = x.clone()
    y = torch.full_like(x, float("nan"))
    s.dplan_step(x, _i32(s.step_indices(0)), None, x_out=y)
    y_ref = torch.full_like(x, float("nan"))
    s.step(0, x0.clone(), y_ref)
    torch.cuda.synchronize()
    assert torch.equal(x, x0)
    active = (s.step_indices(0) >= 0) & (s.step_indices(0) < sp.steps)
    yn, rn = to_np(y), to_np(y_ref)
    for i in range(sp.n):
        if active[i]:
            assert np.array_equal(yn[i], rn[i])
        else:
            assert np.isnan(yn[i]).all()


@pytest.mark.parametrize("k", [0, 17])
def test_large_full_size_dplan_step_streaming(k):
    """Full-size large workload, the bench's launch configuration (device
    plan, nontemporal streams, every slot active by wrapping): one fused
    step equals the host-plan step over the whole tensor."""
    from bucketed_classifier_free_amd import api
    from bucketed_classifier_free_amd import _lib as L
    inp = W.make_inputs(W.config("large_bf16"))
    s = _sampler(inp, wrap=True)
    x = s.init_state()
    a, b = torch.empty_like(x), torch.empty_like(x)
    p, d = s.upload_plan(k)
    s.launch(d, p.n_active, x, a, cache_hint=L.BCG_CACHE_STREAM)
    out = api.device_plan_arrays(s.n, s.nb)
    nxt = torch.empty(s.n, dtype=torch.int32, device="cuda")
    s.dplan_step(x, _i32(s.step_indices(k)), nxt, x_out=b, plan_out=out,
                 cache_hint=L.BCG_CACHE_STREAM)
    torch.cuda.synchronize()
    assert p.n_active == s.n
    assert torch.equal(a, b)
    sig, table, cov = D.run_setup(inp)
    ref = D.build_plan(s.step_indices(k), inp.spec.steps, inp.spec.num_buckets, table,
                       inp.cfg_override, cov)
    _check_plan(out, ref, s.n)
    assert np.array_equal(nxt.cpu().numpy(), s.step_indices(k + 1))


def _loop_states(inp, reps, device_plan, graph, runs, wrap):
    s = _sampler(inp, wrap=wrap)
    # samples that have not joined yet are not initialised: start them from 0
    fresh = lambda: s.init_state(torch.zeros_like(s.alloc_state()))
    x = torch.stack([fresh() for _ in range(reps)]) if reps > 1 else fresh()
    loop = s.native_loop(x, upload_batch=2, device_plan=device_plan, graph_launches=graph)
    for k0, count in runs:
        loop.run(k0, count)
    torch.cuda.synchronize()
    plan = None if loop.plan_out is None else {k: v.clone() for k, v in loop.plan_out.items()}
    loop.close()
    return x, plan, s


@pytest.mark.parametrize("reps", [1, 2])
@pytest.mark.parametrize("wrap", [False, True])
def test_native_loop_device_plan_equals_host_plan(reps, wrap):
    sp = W.small_spec(n=5, C=2, H=8, W=16, regions=2, steps=6, num_buckets=3)
    inp = W.make_inputs(sp)
    inp.start_step[:] = [0, 2, -1, 5, -3]
    runs = [(0, 5), (5, 19)]  # launches 0..23; with graphs, replays start at launches 0, 5, 9, ...
    xh, _, _ = _loop_states(inp, reps, False, 0, runs, wrap)
    for graph in (0, 4 * reps):
        xd, plan, s = _loop_states(inp, reps, True, graph, runs, wrap)
        assert torch.equal(xd, xh), f"graph={graph}"
        last = 23  # the last launch advanced replica 23 % reps at its step 23 // reps
        sig, table, cov = D.run_setup(inp)
        t = s.step_indices(last // reps)
        _check_plan(plan, D.build_plan(t, sp.steps, sp.num_buckets, table, inp.cfg_override, cov),
                    sp.n)


def test_native_loop_device_plan_restart_and_continuation():
    from bucketed_classifier_free_amd import _lib as L
    sp = W.small_spec(n=3, C=2, H=8, W=16, steps=6)
    inp = W.make_inputs(sp)
    s = _sampler(inp)
    x = s.init_state()
    x0 = x.clone()
    loop = s.native_loop(x, device_plan=True, graph_launches=2)
    loop.run(0, 4)
    with pytest.raises(L.BCGError) as e:
        loop.run(7, 1)  # neither a continuation nor a restart
    assert e.value.code == L.BCG_EINVAL
    torch.cuda.synchronize()
    first = x.clone()
    x.copy_(x0)
    loop.run(0, 4)  # restart: the step indices start again from `start`
    torch.cuda.synchronize()
    loop.close()
    assert torch.equal(x, first)


def test_dplan_many_samples_plan_without_lds_copy():
    """More samples than the plan workgroup keeps in LDS (pass 3 derives the
    buckets again): plan and latents still match."""
    from bucketed_classifier_free_amd import api
    sp = W.small_spec(n=3500, C=1, H=8, W=8, steps=9, num_buckets=8, regions=1, feather=2)
    inp = W.make_inputs(sp)
    sig, table, cov = D.run_setup(inp)
    s = _sampler(inp)
    x = s.init_state()
    a, b = torch.empty_like(x), torch.empty_like(x)
    p, d = s.upload_plan(2)
    s.launch(d, p.n_active, x, a)
    out = api.device_plan_arrays(s.n, s.nb)
    s.dplan_step(x, _i32(s.step_indices(2)), None, x_out=b, plan_out=out)
    torch.cuda.synchronize()
    t = s.step_indices(2)
    act = torch.from_numpy((t >= 0) & (t < sp.steps))
    assert torch.equal(a[act], b[act])
    _check_plan(out, D.build_plan(t, sp.steps, sp.num_buckets, table, inp.cfg_override, cov), sp.n)


def test_graph_replays_match_direct_launches_each_time():
    """Each graph replay, with eager work and synchronisation in between,
    equals the same launches issued directly (state and plan)."""
    sp = W.small_spec(n=6, C=3, H=16, W=24, regions=2, inpaint=True, steps=7, num_buckets=4)
    inp = W.make_inputs(sp)
    sa, sb = _sampler(inp, wrap=True), _sampler(inp, wrap=True)
    xa, xb = sa.init_state(), sb.init_state()
    la = sa.native_loop(xa, device_plan=True, graph_launches=4)
    lb = sb.native_loop(xb, device_plan=True, graph_launches=0)
    for r in range(5):
        la.run(4 * r, 4)  # one replay
        lb.run(4 * r, 4)  # four direct launches
        junk = (xa.float() * 2).sum() + xb.float().mean()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(xa, xb), f"replay {r}"
        for k in la.plan_out:
            assert torch.equal(la.plan_out[k], lb.plan_out[k]), (r, k)
    la.close()
    lb.close()


@pytest.mark.parametrize("name", ["mixed_bucket", "regional_inpaint", "throughput_bf16_heun"])
def test_dplan_with_sample_records_equals_host_path(name):
    """Steps that read the sample records their previous plan wrote (instead of
    deriving sigma, scale and the skip from the step index) give the same
    trajectory; every record written equals the host's records of that step."""
    inp = W.make_inputs(W.config(name))
    sp = inp.spec
    s = _sampler(inp)
    xh = s.run()
    x = s.init_state()
    t0 = s.step_indices(0)
    steps = [_i32(t0), torch.empty_like(_i32(t0))]
    recs = [torch.from_numpy(s.records(0)).cuda(), torch.full((sp.n, 4), np.nan, device="cuda")]
    for k in range(sp.steps):
        s.dplan_step(x, steps[k & 1], steps[(k + 1) & 1], record_in=recs[k & 1],
                     record_out=recs[(k + 1) & 1])
        torch.cuda.synchronize()
        got = recs[(k + 1) & 1].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), s.records(k + 1).view(np.uint32)), k
    assert torch.equal(x, xh)


def test_bench_loop_large_shape_matches_mirror():
    """The bench's loop at the large workload's full size (256 x 16x128x128
    bf16, 2 regions, Euler): device plans with sample records, replays of a
    captured graph, two replicas served round robin with the streaming hint,
    starts without wrapping (the oracle's trajectory).  After every replay the
    sampled samples of both replicas equal mode M bit for bit; at the end they
    are within the mode-D bars."""
    from gpu_helpers import bf16_ulp, storage_flip_bound
    inp = W.make_inputs(W.config("large_bf16"))
    idx = [0, 37, 101, 255]
    sub = inp.subset(idx)
    _, ms = M.trajectory32(sub, launches=12, keep=True)
    s = _sampler(inp)
    x = torch.stack([s.init_state(), s.init_state()])
    loop = s.native_loop(x, device_plan=True, graph_launches=8, records=True)
    for r in range(3):
        loop.run(8 * r, 8)          # one replay: 4 steps of each replica
        assert loop.last_run() == (8, 0)
        torch.cuda.synchronize()
        for rep in range(2):
            got = to_np(x[rep, idx])
            assert np.array_equal(got, ms[4 * (r + 1)]), f"replay {r} replica {rep}"
    loop.close()
    xd = D.trajectory(sub, launches=12)
    err = np.abs(to_np(x[1, idx]).astype(np.float64) - xd)
    for q in np.argwhere(err > np.maximum(2e-2, bf16_ulp(xd))):
        assert err[tuple(q)] <= storage_flip_bound(sub, int(q[0]), 12)[tuple(q[1:])]


@pytest.mark.parametrize("name,records", [("mixed_bucket", False), ("mixed_bucket", True),
                                          ("throughput_bf16_heun", True), ("large_bf16", True)])
def test_dplan_norm_stats_inside_the_step(name, records):
    """Norm statistics of a device-plan step, computed inside the step from
    per-row-group partials (no second pass over x) and summed per sample in a
    fixed order: within 1e-5 of the float64 definition, the step's output
    unchanged, and equal bit for bit to the host-plan path's statistics (the
    same grid when every sample is active)."""
    from bucketed_classifier_free_amd import guided_step_workspace_size
    inp = W.make_inputs(W.config(name))
    sp = inp.spec
    s = _sampler(inp, wrap=True)
    sig, table, cov = D.run_setup(inp)
    x = s.init_state()
    k = 3
    t = s.step_indices(k)
    ws = torch.empty(guided_step_workspace_size(sp.n, sp.C, sp.H, sp.W) // 4 + 1, device="cuda")
    st_d = torch.full((sp.n, 3), float("nan"), device="cuda")
    st_h = torch.full((sp.n, 3), float("nan"), device="cuda")
    yd, y0, yh = (torch.full_like(x, float("nan")) for _ in range(3))
    kw = dict(record_in=torch.from_numpy(s.records(k)).cuda()) if records else {}
    s.dplan_step(x, _i32(t), None, x_out=yd, stats=st_d, workspace=ws, **kw)
    s.dplan_step(x, _i32(t), None, x_out=y0, **kw)
    p = s.step(k, x, yh, stats=st_h, workspace=ws)
    torch.cuda.synchronize()
    bits = torch.int16 if sp.dtype == "bf16" else torch.int32
    assert torch.equal(yd.view(bits), y0.view(bits)) and torch.equal(yd.view(bits), yh.view(bits))
    got = to_np(st_d)
    if p.n_active == sp.n:
        assert np.array_equal(got, to_np(st_h))
    plan = D.build_plan(t, sp.steps, sp.num_buckets, table, inp.cfg_override, cov)
    x_np = to_np(x)
    idx = range(sp.n) if sp.n <= 64 else [0, 37, 101, 255]
    for i in idx:
        if plan["bucket_id"][i] < 0:
            assert np.isnan(got[i]).all()
            continue
        ref = D.norm_stats(x_np[i].astype(np.float64), float(sig[t[i]]), float(plan["scale"][i]),
                           D.sample_params(inp, i), bool(plan["need_uncond"][i]))
        np.testing.assert_allclose(got[i], ref, rtol=1e-5, atol=1e-6)
