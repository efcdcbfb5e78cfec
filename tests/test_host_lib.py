"""Host half of libbcg against the oracle, on the CPU (no GPU calls).

Cases marked ``host`` call only the functions of bcg_host.cpp; they also run
against its sanitized host-only build (test_host_sanitized.py).

The library must load and export every function include/bcg.h declares;
sigma_schedule, bucket_table and bcg_plan_build are plain host code and are
compared with the oracle bit for bit; argument errors come back as status
codes before anything is launched.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

import bucketed_classifier_free_amd as bcg
from bucketed_classifier_free_amd import _lib as L
import workloads as W
from oracle import definition as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "bcg.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, re.M)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) == 23, names
    lib = C.CDLL(L.LIB_PATH)
    for nm in names:
        assert hasattr(lib, nm), nm
    assert sorted(L.EXPORTS) == names
    assert lib.bcg_abi_version() == L.ABI_VERSION == 9


@pytest.mark.host
@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_sigma_schedule_bit_exact_on_workloads(name):
    sp = W.config(name)
    got, nb = bcg.sigma_schedule(sp.sigma_max, sp.sigma_min, sp.steps, sp.denoise)
    want, nb2 = D.sigma_schedule(sp.sigma_max, sp.sigma_min, sp.steps, sp.denoise)
    assert nb == nb2
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.host
def test_sigma_schedule_bit_exact_random():
    rng = np.random.default_rng(8)
    for _ in range(200):
        steps = int(rng.integers(1, 400))
        den = float(rng.choice([1.0, rng.uniform(0.05, 1.0)]))
        smax = float(rng.uniform(1.0, 100.0))
        smin = float(rng.uniform(1e-3, 0.9))
        got, nb = bcg.sigma_schedule(smax, smin, steps, den)
        want, nb2 = D.sigma_schedule(smax, smin, steps, den)
        assert nb == nb2
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.host
def test_bucket_table_bit_exact():
    for kind, p in (("const", (7.0, 0, 0)), ("linear", (2.0, 1.2, 0)), ("front_high", (2.0, 1.2, 0.2)),
                    ("linear", (0.5, 9.0, 0))):
        for nb in (1, 2, 3, 8, 16, 64):
            got = bcg.bucket_table(kind, *p, num_buckets=nb)
            want = D.bucket_table(kind, *p, nb)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _compare_plan(got, want):
    for k in ("bucket_id", "uncond_row", "cond_row", "bucket_count", "bucket_offset"):
        assert np.array_equal(getattr(got, k), want[k]), k
    assert np.array_equal(got.uncond_offset, want["uncond_offset"])
    assert np.array_equal(got.scale.view(np.uint32), want["scale"].view(np.uint32))
    assert got.n_active == want["n_active"] and got.n_uncond == want["n_uncond"]
    assert np.array_equal(got.order[:got.n_active], want["order"])
    assert np.all(got.order[got.n_active:] == -1)


@pytest.mark.host
def test_plan_build_bit_exact_random():
    rng = np.random.default_rng(9)
    for _ in range(400):
        n = int(rng.integers(0, 50))
        steps = int(rng.integers(1, 80))
        nb = int(rng.integers(1, 20))
        t = rng.integers(-4, steps + 4, size=n).astype(np.int32)
        table = D.bucket_table("linear", 2.0, rng.choice([1.0, 1.2]), 0, nb)
        ov = np.where(rng.random(n) < 0.3, rng.choice([1.0, 3.5]), np.nan).astype(np.float32)
        got = bcg.bcg_plan_build(t, steps, table, cfg_override=ov)
        _compare_plan(got, D.build_plan(t, steps, nb, table, ov, None))


@pytest.mark.host
@pytest.mark.parametrize("name", ["regional_inpaint", "large_bf16"])
def test_plan_regions_bit_exact_on_workloads(name):
    inp = W.make_inputs(W.config(name))
    sp = inp.spec
    sig, table, cov = D.run_setup(inp)
    for k in (0, 7, sp.steps - 1):
        t = inp.start_step + k
        got = bcg.bcg_plan_build(t, sp.steps, table, C=sp.C, H=sp.H, W=sp.W,
                                 cfg_override=inp.cfg_override, region_count=inp.region_count,
                                 region_frac=inp.region_frac, region_strength=inp.region_strength,
                                 max_regions=sp.regions)
        _compare_plan(got, D.build_plan(t, sp.steps, sp.num_buckets, table, inp.cfg_override, cov))
    off = 0
    for i in range(sp.n):
        for r in range(sp.regions):
            box = D.area_box(inp.region_frac[i, r], sp.H, sp.W)
            assert tuple(got.region_box[i, r]) == box
            assert got.region_off[i * sp.regions + r] == off
            off += sp.C * (box[1] - box[0]) * (box[3] - box[2])
    assert got.region_off[-1] == off


@pytest.mark.host
def test_plan_coverage_forces_uncond_at_scale_one():
    # two samples at cfg 1: one fully covered by its regions, one not
    frac = np.array([[[0, 0, 1, 0.5], [0, 0.5, 1, 0.5]],
                     [[0, 0, 0.5, 0.5], [0.5, 0.5, 0.5, 0.5]]], np.float64)
    plan = bcg.bcg_plan_build(np.zeros(2, np.int32), 4, np.float32([1.0]), C=2, H=8, W=8,
                              region_count=np.int32([2, 2]), region_frac=frac,
                              region_strength=np.float32([[1, 1], [1, 1]]), max_regions=2)
    assert plan.uncond_row[0] == -1 and plan.uncond_row[1] == 0
    # a zero-strength region does not cover
    plan = bcg.bcg_plan_build(np.zeros(2, np.int32), 4, np.float32([1.0]), C=2, H=8, W=8,
                              region_count=np.int32([2, 2]), region_frac=frac,
                              region_strength=np.float32([[1, 0], [1, 1]]), max_regions=2)
    assert plan.uncond_row[0] >= 0


@pytest.mark.host
def test_plan_coverage_matches_bruteforce_random():
    rng = np.random.default_rng(12)
    for _ in range(200):
        n, R = 6, int(rng.integers(1, 5))
        H, Wd = int(rng.integers(1, 20)), int(rng.integers(1, 20))
        frac = rng.uniform(-0.2, 1.2, size=(n, R, 4))
        frac[..., 2:] = rng.uniform(0.0, 1.1, size=(n, R, 2))
        cnt = rng.integers(0, R + 1, size=n).astype(np.int32)
        st = np.where(rng.random((n, R)) < 0.2, 0.0, 1.0).astype(np.float32)
        plan = bcg.bcg_plan_build(np.zeros(n, np.int32), 3, np.float32([1.0]), C=1, H=H, W=Wd,
                                  region_count=cnt, region_frac=frac, region_strength=st,
                                  max_regions=R)
        for i in range(n):
            boxes = [D.area_box(frac[i, r], H, Wd) for r in range(cnt[i])]
            cov = True if cnt[i] == 0 else D.covers_frame(boxes, st[i, :cnt[i]], H, Wd)
            assert (plan.uncond_row[i] == -1) == cov
            for r in range(cnt[i]):
                assert tuple(plan.region_box[i, r]) == boxes[r]


@pytest.mark.host
def test_error_paths_return_codes():
    with pytest.raises(L.BCGError) as e:
        bcg.sigma_schedule(1.0, 2.0, 10)
    assert e.value.code == L.BCG_EINVAL and "sigma_max" in str(e.value)
    with pytest.raises(L.BCGError):
        bcg.sigma_schedule(14.6, 0.03, 10, denoise=0.0)
    with pytest.raises(L.BCGError):
        bcg.bucket_table("linear", 2.0, 1.2, 0.0, num_buckets=0)
    with pytest.raises(L.BCGError) as e:
        bcg.bcg_plan_build(np.zeros(2, np.int32), 5, np.float32([2.0]), C=1, H=4, W=4,
                           region_count=np.int32([3, 0]), region_frac=np.zeros((2, 2, 4)),
                           region_strength=np.ones((2, 2), np.float32), max_regions=2)
    assert e.value.code == L.BCG_EINVAL
    with pytest.raises(L.BCGError):
        bcg.bcg_plan_build(np.zeros(1, np.int32), 5, np.float32([np.inf]))
    with pytest.raises(L.BCGError):  # negative strength
        bcg.bcg_plan_build(np.zeros(1, np.int32), 5, np.float32([2.0]), C=1, H=4, W=4,
                           region_count=np.int32([1]), region_frac=np.zeros((1, 1, 4)),
                           region_strength=np.float32([[-1.0]]), max_regions=1)


def test_device_entry_points_validate_before_launch():
    lib = L.lib()
    a = L.StepArgs()
    a.n, a.C, a.H, a.W = 2, 0, 4, 4
    assert lib.guided_step(C.byref(a), None) == L.BCG_ESHAPE
    a.C = 4
    a.dtype = 7
    assert lib.guided_step(C.byref(a), None) == L.BCG_EDTYPE
    a.dtype, a.sampler, a.num_sigmas, a.s2, a.n_active = 0, 5, 11, 0.25, 1
    assert lib.guided_step(C.byref(a), None) == L.BCG_EINVAL
    a.sampler = 0
    assert lib.guided_step(C.byref(a), None) == L.BCG_EINVAL      # NULL device pointers
    assert b"NULL" in lib.bcg_last_error()
    a.n_active = 0
    assert lib.guided_step(C.byref(a), None) == L.BCG_OK          # nothing to do, no launch
    assert lib.latent_init(1, 1, 1, 1, 9, None, None, None, 1, None, None, None) == L.BCG_EDTYPE
    assert lib.mask_blend(1, 1, 1, 1, 0, None, None, None, 3, None, None) == L.BCG_EINVAL
    assert lib.area_accumulate(1, 1, 1, 1, 0, 0, None, 0, None, None, None, None, None, None,
                               None, None) == L.BCG_EINVAL
    assert lib.guided_step_workspace_size(4, 16, 128, 128, 1) == 4 * 16 * 128 * 3 * 4


@pytest.mark.host
def test_plan_with_cached_coverage_equals_full_plan():
    inp = W.make_inputs(W.config("regional_inpaint"))
    sp = inp.spec
    table = bcg.bucket_table("linear", 2.0, 1.2, 0, sp.num_buckets)
    ov = inp.cfg_override.copy()
    ov[::3] = 1.0
    full = bcg.bcg_plan_build(inp.start_step + 3, sp.steps, table, C=sp.C, H=sp.H, W=sp.W,
                              cfg_override=ov, region_count=inp.region_count,
                              region_frac=inp.region_frac, region_strength=inp.region_strength,
                              max_regions=sp.regions)
    fast = bcg.bcg_plan_build(inp.start_step + 3, sp.steps, table, C=sp.C, H=sp.H, W=sp.W,
                              cfg_override=ov, max_regions=sp.regions, covered=full.covered)
    for k in ("bucket_id", "scale", "uncond_row", "cond_row", "order", "bucket_offset",
              "uncond_offset", "covered"):
        assert np.array_equal(getattr(full, k), getattr(fast, k)), k
    assert fast.n_active == full.n_active and fast.n_uncond == full.n_uncond


def _fake(k):
    """A non-NULL pointer value that validation accepts and nothing dereferences."""
    return C.c_void_p(0x100000 * k)


def test_device_plan_entry_points_validate_before_launch():
    lib = L.lib()
    d = L.DevicePlan(10, 4, 0, _fake(1), None, None, _fake(2), None)
    assert lib.bcg_plan_device(3, C.byref(d), None) == L.BCG_EINVAL   # nothing to write
    assert b"nothing" in lib.bcg_last_error()
    assert lib.bcg_plan_device(0, C.byref(d), None) == L.BCG_OK       # no samples, no launch
    d.step_out = _fake(2).value + 4                                  # overlaps step_in
    assert lib.bcg_plan_device(3, C.byref(d), None) == L.BCG_EINVAL
    assert b"overlaps" in lib.bcg_last_error()
    d.step_out = _fake(3)
    d.bucket_id = _fake(4)                                           # outputs half given
    assert lib.bcg_plan_device(3, C.byref(d), None) == L.BCG_EINVAL
    d.bucket_id = None
    for field, bad in (("steps", 0), ("steps", L.BCG_MAX_DEVICE_STEPS + 1),
                       ("num_buckets", 0), ("num_buckets", L.BCG_MAX_DEVICE_BUCKETS + 1),
                       ("wrap", 2)):
        good = getattr(d, field)
        setattr(d, field, bad)
        assert lib.bcg_plan_device(3, C.byref(d), None) == L.BCG_EINVAL, field
        setattr(d, field, good)
    assert lib.bcg_plan_device(-1, C.byref(d), None) == L.BCG_ESHAPE

    a = L.StepArgs()
    a.n, a.C, a.H, a.W, a.num_sigmas, a.s2 = 2, 4, 8, 8, 11, 0.25
    a.x = a.x_out = a.sigmas = a.mu_uncond = a.mu_cond = _fake(5)
    assert lib.guided_step_dplan(C.byref(a), None, None) == L.BCG_EINVAL
    a.scale = _fake(6)                                                # plan rows must be NULL
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    assert b"device plan" in lib.bcg_last_error()
    a.scale = None
    a.stats = _fake(7)
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    a.stats = None
    a.num_sigmas = 10                                                 # < steps + 1
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    a.num_sigmas = 11
    a.max_regions, a.region_count = 2, _fake(8)                       # regions need coverage
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    assert b"coverage" in lib.bcg_last_error()
    a.max_regions, a.region_count = 0, None
    a.n = 0                                                           # no samples, no launch
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_OK


@pytest.mark.parametrize("field,bad,word", [
    ("queue_len", 1, b"queue_len"),                # fewer requests than the 2 slots
    ("queue_len", 1 << 24, b"queue_len"),
    ("queue_ring", 2, b"queue_ring"),
    ("wrap", 1, b"wrap"),
    ("noise", None, b"noise"),
    ("slot_req_out", None, b"slot_req"),
    ("queue_out", None, b"queue_in/out"),
    ("region_range", 9, b"validity"),              # validity ranges without covered_sets
    ("join_front", 3, b"join_front"),              # more than the 2 slots
    ("join_in", None, b"join_in"),
])
def test_queue_plan_validates_before_launch(field, bad, word):
    """Continuous batching's device-plan fields: each inconsistent setting is
    rejected with a message before anything is launched."""
    lib = L.lib()
    d = L.DevicePlan(10, 4, 0, _fake(1), None, None, _fake(2), _fake(3))
    d.record_in, d.record_out, d.sigmas, d.num_sigmas = _fake(10), _fake(11), _fake(12), 11
    d.queue_len, d.queue_ring, d.noise = 4, 1, _fake(13)
    d.slot_req_in, d.slot_req_out, d.queue_in, d.queue_out = _fake(14), _fake(15), _fake(16), _fake(17)
    d.join_front, d.join_in, d.join_out = 1, _fake(18), _fake(19)
    a = L.StepArgs()
    a.n, a.C, a.H, a.W, a.num_sigmas, a.s2 = 2, 4, 8, 8, 11, 0.25
    a.x, a.x_out, a.sigmas, a.mu_uncond, a.mu_cond = _fake(5), _fake(6), _fake(12), _fake(7), _fake(8)
    if field == "region_range":
        d.region_range = _fake(bad)
    else:
        setattr(d, field, bad)
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL, field
    assert word in lib.bcg_last_error(), lib.bcg_last_error()


def test_queue_plan_other_rejections():
    lib = L.lib()
    d = L.DevicePlan(10, 4, 0, _fake(1), None, None, _fake(2), _fake(3))
    d.record_in, d.record_out, d.sigmas, d.num_sigmas = _fake(10), _fake(11), _fake(12), 11
    d.queue_len, d.queue_ring, d.noise = 4, 1, _fake(13)
    d.slot_req_in, d.slot_req_out, d.queue_in, d.queue_out = _fake(14), _fake(15), _fake(16), _fake(17)
    a = L.StepArgs()
    a.n, a.C, a.H, a.W, a.num_sigmas, a.s2 = 2, 4, 8, 8, 11, 0.25
    a.x, a.x_out, a.sigmas, a.mu_uncond, a.mu_cond = _fake(5), _fake(6), _fake(12), _fake(7), _fake(8)
    d.slot_req_out = _fake(14).value + 4                                # overlaps slot_req_in
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    assert b"overlap" in lib.bcg_last_error()
    d.slot_req_out = _fake(15)
    d.join_front, d.join_in, d.join_out = 2, _fake(18), _fake(18).value + 4  # join_out overlaps join_in
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    assert b"join_out" in lib.bcg_last_error()
    d.join_front, d.join_in, d.join_out = 0, None, None
    a.stats = _fake(20)                                                 # no statistics with a queue
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    assert b"stats" in lib.bcg_last_error()
    a.stats = None
    a.H = a.W = 7                                                       # the vector path is required
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    assert b"vector" in lib.bcg_last_error()
    a.H = a.W = 8
    d.noise = _fake(13).value + 4                                       # misaligned noise
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    d.noise = _fake(13)
    rin = d.record_in
    d.record_in = None                                                  # (a plan launch reads no records)
    assert lib.bcg_plan_device(2, C.byref(d), None) == L.BCG_EINVAL     # a queue needs the step
    assert b"inside guided_step_dplan" in lib.bcg_last_error()
    d.record_in = rin
    q = d.queue_len
    d.queue_len = 0                                                     # queue arrays without a queue
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    assert b"queue_len = 0" in lib.bcg_last_error()
    d.queue_len = q
    a.n = 0                                                             # no slots: nothing launched
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_OK


def test_loop_create_validates_device_plan_mode():
    lib = L.lib()
    start = np.zeros(2, np.int32)
    table = np.float32([2.0, 1.5])
    plan = L.PlanIn(2, 10, 2, 4, 8, 8, 0, table.ctypes.data, None, None, None, None, None, None)
    step = L.StepArgs()
    step.n, step.C, step.H, step.W, step.num_sigmas, step.s2 = 2, 4, 8, 8, 11, 0.25
    d = L.LoopDesc(plan, start.ctypes.data, 0, 1, None, None, 1, 0, 1, 0, step, 1, 5000, None,
                   L.DevicePlan(0, 0, 0, _fake(1)))
    h = C.c_void_p()
    assert lib.bcg_loop_create(C.byref(d), C.byref(h)) == L.BCG_EINVAL   # dev_steps NULL
    d.dev_steps = _fake(2)
    assert lib.bcg_loop_create(C.byref(d), C.byref(h)) == L.BCG_EINVAL   # G beyond 4096
    assert b"graph_launches" in lib.bcg_last_error()
    d.device_plan, d.graph_launches = 0, 4                               # graphs need device plans
    d.host_slab = d.dev_slab = _fake(3)
    assert lib.bcg_loop_create(C.byref(d), C.byref(h)) == L.BCG_EINVAL
    d.device_plan = 2
    assert lib.bcg_loop_create(C.byref(d), C.byref(h)) == L.BCG_EINVAL
    assert not h.value
    # continuous batching: device plans with records, the queue state and the noise
    d.device_plan, d.graph_launches, d.dev_records = 1, 0, _fake(4)
    d.queue_len, d.noise, d.dev_queue = 4, _fake(5), _fake(6)
    for field, bad, word in (("dev_queue", None, b"dev_queue"), ("noise", None, b"noise"),
                             ("dev_records", None, b"dev_records"), ("queue_len", 1, b"queue_len >= n"),
                             ("wrap", 1, b"wrap = 0"), ("join_front", 3, b"join_front")):
        good = getattr(d, field)
        setattr(d, field, bad)
        assert lib.bcg_loop_create(C.byref(d), C.byref(h)) == L.BCG_EINVAL, field
        assert word in lib.bcg_last_error(), (field, lib.bcg_last_error())
        setattr(d, field, good)
    start[1] = 10                                                        # a start step past the schedule
    assert lib.bcg_loop_create(C.byref(d), C.byref(h)) == L.BCG_EINVAL
    assert b"start[1]" in lib.bcg_last_error()
    assert not h.value


def test_rows_entry_point_validates_before_launch():
    lib = L.lib()
    a = L.RowsArgs()
    a.n, a.C, a.H, a.W, a.num_sigmas, a.rows, a.n_active = 2, 4, 8, 8, 11, 4, 2
    a.phase = 7
    assert lib.guided_step_rows(C.byref(a), None) == L.BCG_EINVAL
    a.phase = L.BCG_PHASE["euler"]
    assert lib.guided_step_rows(C.byref(a), None) == L.BCG_EINVAL       # NULL pointers
    for f, k in (("x", 1), ("x_out", 2), ("pred", 3), ("sigmas", 4), ("order", 5), ("step_idx", 6),
                 ("scale", 7), ("uncond_row", 8), ("cond_row", 9)):
        setattr(a, f, _fake(k))
    a.pred = _fake(2).value + 64                                        # overlaps x_out
    assert lib.guided_step_rows(C.byref(a), None) == L.BCG_EINVAL
    assert b"overlaps" in lib.bcg_last_error()
    a.pred = _fake(3)
    a.phase = L.BCG_PHASE["heun_predict"]                               # needs d
    assert lib.guided_step_rows(C.byref(a), None) == L.BCG_EINVAL
    a.d = _fake(10)
    a.phase = L.BCG_PHASE["heun_correct"]                               # needs x_tilde
    assert lib.guided_step_rows(C.byref(a), None) == L.BCG_EINVAL
    a.x_orig = _fake(11)                                                # half an inpaint
    a.x_tilde = _fake(12)
    assert lib.guided_step_rows(C.byref(a), None) == L.BCG_EINVAL
    a.x_orig = None
    a.dtype = 5
    assert lib.guided_step_rows(C.byref(a), None) == L.BCG_EDTYPE
    a.dtype, a.n_active = 0, 0                                          # nothing to do, no launch
    assert lib.guided_step_rows(C.byref(a), None) == L.BCG_OK


def test_rows_dplan_entry_point_validates_before_launch():
    lib = L.lib()
    a = L.RowsArgs()
    a.n, a.C, a.H, a.W, a.num_sigmas, a.rows, a.n_active = 2, 4, 8, 8, 11, 4, 2
    a.phase = L.BCG_PHASE["euler"]
    for f, k in (("x", 1), ("x_out", 2), ("pred", 3), ("sigmas", 4), ("order", 5), ("step_idx", 6),
                 ("scale", 7), ("uncond_row", 8), ("cond_row", 9)):
        setattr(a, f, _fake(k))
    assert lib.guided_step_rows_dplan(C.byref(a), None, None) == L.BCG_EINVAL   # no plan
    d = L.DevicePlan(10, 2, 1, _fake(20))
    d.step_in = _fake(21)
    assert lib.guided_step_rows_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL  # nothing to write
    d.step_out = _fake(7)                                              # the update's scale
    assert lib.guided_step_rows_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    assert b"overlap" in lib.bcg_last_error()
    d.step_out = _fake(22)
    d.record_out, d.sigmas, d.num_sigmas = _fake(5).value + 4, _fake(23), 11   # into the order
    assert lib.guided_step_rows_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    d.record_out = None
    d.step_in = _fake(2).value + 64                                    # reads x_out as it is written
    assert lib.guided_step_rows_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    assert b"overlap" in lib.bcg_last_error()
    d.step_in = _fake(21)
    a.phase = 7                                                        # the update's own checks
    assert lib.guided_step_rows_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    a.phase = L.BCG_PHASE["euler"]
    d.steps = 0                                                        # the plan's own checks
    assert lib.guided_step_rows_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    d.steps = 10
    a.n, a.n_active = 0, 0                                             # no samples, no launch
    assert lib.guided_step_rows_dplan(C.byref(a), C.byref(d), None) == L.BCG_OK


@pytest.mark.host
def test_sigma_crop_bit_exact_and_errors():
    rng = np.random.default_rng(3)
    for _ in range(100):
        steps = int(rng.integers(1, 60))
        sig, _ = bcg.sigma_schedule(14.6, 0.03, steps, float(rng.choice([1.0, 0.6])))
        last = int(rng.integers(-1, steps + 3))
        end = steps if last < 0 or last > steps else last
        start = int(rng.integers(0, end + 1))
        force = bool(rng.integers(0, 2))
        got = bcg.sigma_crop(sig, start, last, force)
        want = D.crop_sigmas(sig, start, None if last < 0 else last, force)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    with pytest.raises(L.BCGError):
        bcg.sigma_crop(sig, 5, 2)


@pytest.mark.host
def test_mid_peak_table_bit_exact():
    rng = np.random.default_rng(4)
    for _ in range(50):
        p0, p1, p2 = float(rng.uniform(1, 3)), float(rng.uniform(1, 8)), float(rng.uniform(0.05, 0.95))
        nb = int(rng.integers(1, 40))
        got = bcg.bucket_table("mid_peak", p0, p1, p2, nb)
        want = D.bucket_table("mid_peak", p0, p1, p2, nb)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    for bad in (0.0, 1.0, -0.5):
        with pytest.raises(L.BCGError):
            bcg.bucket_table("mid_peak", 1.2, 2.0, bad, 4)


@pytest.mark.host
def test_bucket_bounds_and_interpolated_plan_bit_exact():
    rng = np.random.default_rng(5)
    for kind, p in (("linear", (2.0, 1.2, 0.0)), ("front_high", (2.0, 1.2, 0.2)),
                    ("mid_peak", (1.2, 3.0, 0.4)), ("const", (7.0, 0.0, 0.0))):
        for nb in (1, 3, 8, 16, 37):
            lo, hi = bcg.bucket_bounds(kind, *p, num_buckets=nb)
            rlo, rhi = D.bucket_bounds(kind, *p, nb)
            assert np.array_equal(lo.view(np.uint32), rlo.view(np.uint32))
            assert np.array_equal(hi.view(np.uint32), rhi.view(np.uint32))
            for _ in range(5):
                n = int(rng.integers(1, 60))
                steps = int(rng.integers(1, 80))
                t = rng.integers(-2, steps + 2, n).astype(np.int32)
                ov = np.where(rng.random(n) < 0.2, np.float32(1.0), np.float32(np.nan)).astype(np.float32)
                got = bcg.bcg_plan_build(t, steps, lo, cfg_override=ov, bucket_cfg_end=hi)
                ref = D.build_plan(t, steps, nb, rlo, ov, None, rhi)
                assert np.array_equal(got.scale.view(np.uint32), ref["scale"].view(np.uint32))
                assert np.array_equal(got.order[:got.n_active], ref["order"])
                assert np.array_equal(got.uncond_row, ref["uncond_row"])
    with pytest.raises(L.BCGError):
        bcg.bcg_plan_build(np.zeros(1, np.int32), 5, np.float32([2.0]),
                           bucket_cfg_end=np.float32([np.inf]))


@pytest.mark.host
def test_plan_records_from_host_plan():
    sig, _ = bcg.sigma_schedule(14.6, 0.03, 10)
    t = np.int32([0, 9, 10, -1, 4])
    table = np.float32([2.0, 1.0])
    p = bcg.bcg_plan_build(t, 10, table, cfg_override=np.float32([np.nan, np.nan, np.nan, np.nan, 1.0]))
    r = bcg.api.plan_records(p, t, 10, sig)
    flags = r[:, 3].view(np.uint32)
    assert list(flags & 3) == [3, 1, 0, 0, 1]      # active, uncond kept / skipped at scale 1
    assert list(flags >> 2) == [15, 15, 0, 0, 15]  # no validity ranges: every region valid
    assert r[0, 0] == sig[0] and r[1, 1] == sig[10] == 0 and r[4, 2] == np.float32(1.0)
    assert (r[2:4] == 0).all()


@pytest.mark.host
def test_plan_with_validity_ranges_bit_exact():
    sp = W.small_spec(n=40, C=2, H=24, W=32, steps=20, num_buckets=4, regions=3, region_ranges=True,
                      curve=W.Curve("linear", 2.0, 1.0), skip_frac=0.5, seed=12)
    inp = W.make_inputs(sp)
    table = D.bucket_table("linear", 2.0, 1.0, 0.0, 4)
    kw = dict(C=sp.C, H=sp.H, W=sp.W, cfg_override=inp.cfg_override, max_regions=3,
              region_range=inp.region_range)
    full0 = bcg.bcg_plan_build(np.zeros(sp.n, np.int32), sp.steps, table, region_count=inp.region_count,
                               region_frac=inp.region_frac, region_strength=inp.region_strength, **kw)
    for k in range(sp.steps):
        t = (inp.start_step + k).astype(np.int32)
        ref = D.build_plan(t, sp.steps, 4, table, inp.cfg_override, D.coverage(inp, t))
        for p in (bcg.bcg_plan_build(t, sp.steps, table, region_count=inp.region_count,
                                     region_frac=inp.region_frac,
                                     region_strength=inp.region_strength, **kw),
                  bcg.bcg_plan_build(t, sp.steps, table, region_count=inp.region_count,
                                     covered_sets=full0.covered_sets, **kw)):
            assert np.array_equal(p.uncond_row, ref["uncond_row"]), k
            assert np.array_equal(p.scale.view(np.uint32), ref["scale"].view(np.uint32))
            for i in range(sp.n):
                if 0 <= t[i] < sp.steps:
                    want = sum(1 << r for r in D.valid_regions(inp, i, int(t[i])))
                    assert p.region_valid[i] == want, (k, i)
    with pytest.raises(L.BCGError):  # ranges without region arrays or subset coverage
        bcg.bcg_plan_build(np.zeros(sp.n, np.int32), sp.steps, table, covered=full0.covered, **kw)


def _weight_args(rows=64, cols=128, patches=()):
    arr = (L.Patch * max(len(patches), 1))(*patches)
    a = L.WeightArgs(rows, cols, L.BCG_BF16, L.BCG_BF16, len(patches), L.BCG_ROUND["stochastic"], 5,
                     _fake(1), _fake(2), C.addressof(arr) if patches else None)
    return a, arr


def test_weight_patch_validates_before_launch():
    lib = L.lib()
    diff = lambda **kw: L.Patch(**{**dict(kind=0, offset=0, rows=64, rank=0, dtype=L.BCG_BF16,
                                          strength_patch=1.0, strength_model=1.0, diff=_fake(3)), **kw})
    lowr = lambda **kw: L.Patch(**{**dict(kind=1, offset=0, rows=64, rank=16, dtype=L.BCG_BF16,
                                          strength_patch=1.0, strength_model=1.0, up=_fake(4),
                                          down=_fake(5)), **kw})
    assert lib.weight_patch(None, None) == L.BCG_EINVAL
    cases = [
        (dict(rows=-1), [], L.BCG_ESHAPE),
        ({}, [diff(offset=10)], L.BCG_ESHAPE),           # rows [10, 74) outside 64
        ({}, [diff(offset=-1, rows=4)], L.BCG_ESHAPE),
        ({}, [lowr(rank=0)], L.BCG_ESHAPE),
        ({}, [lowr(dtype=L.BCG_F32)], L.BCG_EDTYPE),
        ({}, [diff(dtype=7)], L.BCG_EDTYPE),
        ({}, [diff(kind=3)], L.BCG_EINVAL),
        ({}, [diff(diff=None)], L.BCG_EINVAL),
        ({}, [lowr(down=None)], L.BCG_EINVAL),
        ({}, [diff(diff=C.c_void_p(_fake(2).value + 64))], L.BCG_EINVAL),  # diff overlaps out
    ]
    for kw, pats, code in cases:
        a, keep = _weight_args(patches=pats, **{k: v for k, v in kw.items() if k in ("rows", "cols")})
        assert lib.weight_patch(C.byref(a), None) == code, (kw, code, lib.bcg_last_error())
    a, keep = _weight_args(patches=[diff()] * 9)
    a.num_patches = 9
    assert lib.weight_patch(C.byref(a), None) == L.BCG_EINVAL
    a, keep = _weight_args()
    a.rounding = 2
    assert lib.weight_patch(C.byref(a), None) == L.BCG_EINVAL
    a.rounding, a.w_dtype = 0, 5
    assert lib.weight_patch(C.byref(a), None) == L.BCG_EDTYPE
    a.w_dtype, a.out_dtype, a.out = L.BCG_F32, L.BCG_BF16, C.c_void_p(_fake(1).value + 2)
    assert lib.weight_patch(C.byref(a), None) == L.BCG_EINVAL       # w and out overlap
    assert b"overlap" in lib.bcg_last_error()
    # an empty weight is a no-op, even with NULL arrays
    a, keep = _weight_args(rows=0, patches=[diff(rows=0, diff=None)])
    a.w = a.out = None
    assert lib.weight_patch(C.byref(a), None) == L.BCG_OK


@pytest.mark.host
def test_area_slices_round_exact_products_ties_up():
    # The library's slices at and around every rounding tie of every extent
    # n <= 256: one sample per fraction f, one region (f, 0, 0, f), so the row
    # offset and the column side both come from f*n.
    from area_cases import near_tie_fractions, nearest_by_search
    for n in range(1, 257):
        fr = near_tie_fractions(n)
        k = len(fr)
        frac = np.zeros((k, 1, 4))
        frac[:, 0, 0] = fr
        frac[:, 0, 3] = fr
        got = bcg.bcg_plan_build(np.zeros(k, np.int32), 1, np.float32([2.0]), C=1, H=n, W=n,
                                 region_count=np.ones(k, np.int32), region_frac=frac,
                                 region_strength=np.ones((k, 1), np.float32), max_regions=1)
        for j, f in enumerate(fr):
            m = nearest_by_search(f, n)
            y0 = min(max(m, 0), n - 1)
            assert tuple(got.region_box[j, 0]) == (y0, y0 + 1, 0, min(max(m, 1), n)), (n, f)
            assert tuple(got.region_box[j, 0]) == D.area_box(frac[j, 0], n, n)


def test_dplan_step_rejects_plan_overlaps():
    # The plan's workgroup of guided_step_dplan runs alongside the step: its
    # outputs may not alias anything the step reads or writes, and nothing the
    # step or the plan reads may alias the step's output.  Every call below is
    # rejected before any launch.
    lib = L.lib()
    n, Cc, H, Wd = 2, 4, 8, 8
    a = L.StepArgs()
    a.n, a.C, a.H, a.W, a.num_sigmas, a.s2 = n, Cc, H, Wd, 11, 0.25
    a.x, a.x_out, a.sigmas, a.mu_uncond, a.mu_cond = _fake(5), _fake(6), _fake(7), _fake(8), _fake(9)
    # (pointer fields of a ctypes structure read back as ints)
    d = L.DevicePlan(10, 4, 0, _fake(1), None, None, _fake(2), _fake(3))
    cases = [("step_out", a.x + 16),          # plan output inside x
             ("step_out", a.x_out),           # ... inside x_out
             ("step_out", a.mu_cond + 4),     # ... inside a mean table
             ("step_out", a.sigmas)]          # ... over the schedule
    for field, ptr in cases:
        setattr(d, field, C.c_void_p(ptr))
        assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL, (field, ptr)
        assert b"overlap" in lib.bcg_last_error()
    d.step_out = _fake(3)
    d.record_out = C.c_void_p(a.mu_uncond)     # records over the uncond means
    d.record_in = _fake(11)
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    assert b"overlap" in lib.bcg_last_error()
    d.record_out = _fake(12)
    a.x_out = C.c_void_p(d.step_in)                  # the step's output over the plan's input
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    assert b"overlap" in lib.bcg_last_error()
    a.x_out = C.c_void_p(a.mu_cond - 64)       # ... over a mean table the step reads
    assert lib.guided_step_dplan(C.byref(a), C.byref(d), None) == L.BCG_EINVAL
    assert b"overlap" in lib.bcg_last_error()
