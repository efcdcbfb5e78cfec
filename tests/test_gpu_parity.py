"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars (written into each test):
  * integers (plans, boxes) bit-exact -- covered on the CPU in test_host_lib;
  * every stored state equal to mode M (the fixed fp32 evaluation order) bit
    for bit, step after step, over whole trajectories;
  * each step, teacher-forced from the mode D state, within 1e-5 of
    max|ref| per sample (fp32 storage), or within half a bf16 ulp of the
    unrounded mode D value plus that 1e-5 (bf16 storage);
  * the final latent within 2e-2 absolute of mode M (bf16 storage), and
    per element within max(2e-2, 1 bf16 ulp) of mode D unless inside the
    bound of carried storage-rounding flips (storage_flip_bound); within
    1e-4 relative of mode D for fp32 storage.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from oracle import definition as D
from oracle import mirror32 as M

from gpu_helpers import (bf16_ulp, gpu_step_from, gpu_trajectory, oracle_step_D,
                          oracle_step_M, per_sample_rel_err, storage_flip_bound, to_dev, to_np)

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


def _check_step_vs_D(inp, got, ref_d, tag):
    for i, ref in ref_d.items():
        scale = max(np.abs(ref).max(), 1e-30)
        err = np.abs(got[i].astype(np.float64) - ref)
        if inp.spec.dtype == "f32":
            assert err.max() <= 1e-5 * scale, f"{tag} sample {i}: {err.max() / scale:.3g} rel"
        else:
            bound = 0.5 * bf16_ulp(ref) + 1e-5 * scale
            assert np.all(err <= bound), f"{tag} sample {i}: {float((err - bound).max()):.3g} over"


def _check_full(inp, idx, launches=None):
    """Whole trajectory on the GPU vs mode M (bit-exact, every launch) and mode D."""
    sp = inp.spec
    s = _sampler(inp)
    xg, states = gpu_trajectory(s, launches, keep_samples=idx)
    xm, mstates = M.trajectory32(inp, launches=launches, samples=idx, keep=True)
    for k, st in enumerate(states):
        ref = mstates[k + 1][idx]
        bad = ~(st == ref)
        assert not bad.any(), (f"{sp.name}: launch {k} differs from mode M at {int(bad.sum())} "
                               f"elements, max {float(np.abs(st - ref).max()):.3g}")
    xd = D.trajectory(inp, launches=launches, samples=idx)
    err = np.abs(xg[idx].astype(np.float64) - xd[idx])
    if sp.dtype == "bf16":
        # 2e-2 absolute vs mode M (the same fp32 decisions; in fact identical) ...
        assert np.abs(xg[idx] - xm[idx]).max() <= 2e-2
        # ... and vs mode D per element within max(2e-2, one bf16 ulp of the
        # reference).  Mode D's float64 steps round to a neighbouring bf16
        # code now and then (a flip); a flip made while |x| is large is
        # carried to the end by the later steps, so an element over that bar
        # must be inside the bound the storage roundings allow
        # (storage_flip_bound: the flips carried by the step Jacobians).
        bar = np.maximum(2e-2, bf16_ulp(xd[idx]))
        over = np.argwhere(err > bar)
        for q in over:
            i = idx[q[0]]
            fb = storage_flip_bound(inp, i, launches)[tuple(q[1:])]
            assert err[tuple(q)] <= fb, (f"{sp.name}: sample {i} element {tuple(q[1:])}: "
                                         f"{err[tuple(q)]:.4g} over the flip bound {fb:.4g}")
        print(f"{sp.name}: {int((err > 0).sum())} of {err.size} elements differ from mode D "
              f"(bf16 code flips), {len(over)} over max(2e-2, 1 ulp), max {err.max():.4g}")
    else:
        assert per_sample_rel_err(xg, xd, idx).max() <= 1e-4
    return xg


def _teacher_forced(inp, idx, launches):
    sp = inp.spec
    sig, table, cov = D.run_setup(inp)
    s = _sampler(inp)
    _, dstates = D.trajectory(inp, launches=max(launches) + 1, samples=idx, keep=True)
    for k in launches:
        x_in = D.init_latent(inp, sig, sp.dtype).astype(np.float32)
        x_in[idx] = dstates[k][idx]
        got, plan = gpu_step_from(s, k, x_in)
        p = D.build_plan(inp.start_step.astype(np.int64) + k, sp.steps, sp.num_buckets, table,
                         inp.cfg_override, cov)
        _check_step_vs_D(inp, got, oracle_step_D(inp, sig, p, k, x_in, idx), f"{sp.name} k={k}")
        ref_m = oracle_step_M(inp, sig, p, k, x_in, idx)
        for i, r in ref_m.items():
            assert np.array_equal(got[i], r), f"{sp.name} k={k} sample {i} differs from mode M"
        # inactive samples are not written
        for i in idx:
            if p["bucket_id"][i] < 0:
                assert np.isnan(got[i]).all()


# ---------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("name", ["tiny", "mixed_bucket", "throughput_bf16_heun", "regional_inpaint"])
def test_workload_full_trajectory(name):
    inp = W.make_inputs(W.config(name))
    _check_full(inp, list(range(inp.spec.n)))


@pytest.mark.parametrize("name", ["tiny", "mixed_bucket", "throughput_bf16_heun", "regional_inpaint"])
def test_workload_teacher_forced_steps(name):
    inp = W.make_inputs(W.config(name))
    sp = inp.spec
    launches = list(range(sp.steps)) if sp.n * sp.C * sp.H * sp.W <= 1 << 20 else \
        [0, 1, sp.steps // 2, sp.steps - 2, sp.steps - 1]
    idx = list(range(sp.n)) if sp.n <= 16 else list(range(0, sp.n, 5))
    _teacher_forced(inp, idx, launches)


LARGE_SAMPLES = [0, 37, 101, 255]


def test_large_full_size_sampled_trajectories():
    """Full-size large workload in the bench's launch shape; sampled samples checked."""
    inp = W.make_inputs(W.config("large_bf16"))
    _check_full(inp, LARGE_SAMPLES)


def test_large_full_size_teacher_forced():
    inp = W.make_inputs(W.config("large_bf16"))
    _teacher_forced(inp, LARGE_SAMPLES, [0, 24, 49])


# ---------------------------------------------------------------- small shapes, edge cases

SMALL = [
    dict(dtype="bf16", sampler="euler", regions=2),   # the large workload's variant
    dict(dtype="f32", sampler="euler"),
    dict(dtype="f32", sampler="heun"),
    dict(dtype="bf16", sampler="euler"),
    dict(dtype="bf16", sampler="heun"),
    dict(dtype="f32", sampler="euler", regions=1),
    dict(dtype="f32", sampler="heun", regions=3, inpaint=True),
    dict(dtype="bf16", sampler="euler", regions=2, inpaint=True),
    dict(dtype="bf16", sampler="heun", regions=4),
    dict(dtype="f32", sampler="euler", regions=4, inpaint=True),
]


@pytest.mark.parametrize("shape", [(3, 3, 17, 40), (4, 2, 13, 21), (2, 5, 1, 8), (3, 64, 4, 8)])
@pytest.mark.parametrize("kw", SMALL)
def test_small_shapes_full_trajectory(shape, kw):
    # (17, 40): vector path with a ragged last tile; (13, 21): H*W odd -> scalar
    # path; (1, 8): a single row; C = 64: the channel limit
    n, C, H, Wd = shape
    sp = W.small_spec(n=n, C=C, H=H, W=Wd, steps=5, num_buckets=3, feather=3, **kw)
    _check_full(W.make_inputs(sp), list(range(n)))


def test_many_samples_multi_vector_lanes():
    # 700 samples with a ragged last tile (the automatic shape: one vector per lane)
    sp = W.small_spec(n=700, C=1, H=40, W=64, steps=3, regions=2, inpaint=True, feather=4)
    _check_full(W.make_inputs(sp), list(range(0, 700, 7)))


MULTI_VECTOR = [dict(dtype="bf16", sampler="euler", regions=2),
                dict(dtype="f32", sampler="heun", regions=3),
                dict(dtype="bf16", sampler="heun", regions=1, inpaint=True),
                dict(dtype="f32", sampler="euler")]


@pytest.mark.parametrize("vpt", [2, 3])
@pytest.mark.parametrize("hint", [0, 1])
@pytest.mark.parametrize("C", [16, 12, 5])
@pytest.mark.parametrize("kw", MULTI_VECTOR)
def test_multi_vector_lanes_match_mirror(vpt, hint, C, kw):
    # Lanes taking several vectors (the launch shape forced to vpt vectors per
    # lane of 256): H*W = 40*64 is 320 bf16 / 640 fp32 vectors, so the last
    # pass of each workgroup is ragged; the streaming variants request the next
    # pass's head stage during the current one.  Every sample bit for bit equal
    # to mode M and to the automatic launch shape.
    sp = W.small_spec(n=3, C=C, H=40, W=64, steps=5, num_buckets=3, feather=3, **kw)
    inp = W.make_inputs(sp)
    s = _sampler(inp)
    sig, table, cov = D.run_setup(inp)
    k = 1
    x_in = D.init_latent(inp, sig, sp.dtype).astype(np.float32)
    x = to_dev(x_in, sp.dtype)
    auto, forced = torch.full_like(x, float("nan")), torch.full_like(x, float("nan"))
    s.step(k, x, auto, cache_hint=hint)
    s.step(k, x, forced, cache_hint=hint, launch_vpt=vpt)
    torch.cuda.synchronize()
    got = to_np(forced)
    assert np.array_equal(to_np(auto), got, equal_nan=True)
    p = D.build_plan(inp.start_step.astype(np.int64) + k, sp.steps, sp.num_buckets, table,
                     inp.cfg_override, cov)
    for i, r in oracle_step_M(inp, sig, p, k, x_in, list(range(sp.n))).items():
        assert np.array_equal(got[i], r), f"sample {i} differs from mode M"


def test_region_edge_cases():
    sp = W.small_spec(n=5, C=3, H=16, W=24, regions=3, steps=4, skip_frac=0.0, mixed_start=False,
                      curve=W.Curve("const", 1.0), num_buckets=1, feather=4)
    inp = W.make_inputs(sp)
    inp.region_count[:] = [0, 1, 2, 3, 3]            # a sample with no regions
    inp.region_strength[4, 1] = 0.0                  # a zero-strength region
    inp.region_frac[3, 0] = (0, 0, 1, 1)             # a full-frame region (covers -> skip)
    _check_full(inp, list(range(5)))
    # feather 0 (no ramp) and a feather wider than the boxes
    for F in (0, 64):
        _check_full(W.make_inputs(dataclasses.replace(sp, feather=F)), list(range(5)))


def test_scale_zero_and_one_special_cases():
    base = W.small_spec(n=3, C=2, H=8, W=16, steps=4, skip_frac=0.0, num_buckets=1,
                        mixed_start=False, regions=2)
    for v in (0.0, 1.0):
        inp = W.make_inputs(dataclasses.replace(base, curve=W.Curve("const", v)))
        _check_full(inp, [0, 1, 2])


def test_all_inactive_launch_writes_nothing():
    sp = W.small_spec(n=3, C=2, H=8, W=8, steps=4)
    inp = W.make_inputs(sp)
    inp.start_step[:] = 9                            # beyond the trajectory
    s = _sampler(inp)
    x = to_dev(np.ones((3, 2, 8, 8)), sp.dtype)
    s.step(0, x)
    torch.cuda.synchronize()
    assert (to_np(x) == 1).all()


def test_in_place_equals_out_of_place_and_deterministic():
    inp = W.make_inputs(W.small_spec(n=4, C=4, H=32, W=32, regions=2, inpaint=True,
                                     dtype="bf16", sampler="heun"))
    s = _sampler(inp)
    x0 = s.init_state()
    a = x0.clone(); b = torch.empty_like(x0); c = x0.clone()
    s.step(1, a)
    s.step(1, x0, b)
    s.step(1, c)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("kw", [dict(dtype="bf16", regions=2), dict(dtype="f32", inpaint=True, regions=3, sampler="heun")])
def test_streaming_cache_hint_is_bit_identical(kw):
    inp = W.make_inputs(W.small_spec(n=4, C=4, H=32, W=32, **kw))
    s = _sampler(inp)
    x0 = s.init_state()
    a = torch.empty_like(x0); b = torch.empty_like(x0)
    s.step(1, x0, a, cache_hint=0)
    s.step(1, x0, b, cache_hint=1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# The streaming (nontemporal) variants take their pipeline shape from the
# channel count: 2 channels per stage without prefetch up to 4 channels, the
# per-variant stage table beyond, and its full-stage form (no per-channel
# bounds checks) when C is a multiple of two stages.  Every variant at each
# shape: bit for bit equal to the cache-keep variant on every sample, and to
# mode M on two.  (Lanes take one vector each here; several vectors per lane,
# with the next one's head stage prefetched, are forced through the launch
# shape in test_multi_vector_lanes_match_mirror.)
STREAM_SHAPES = [
    (4, 16, 16, 32),   # the stage table's shape, full stages
    (3, 5, 16, 24),    # width-4 variants fall back; width 2 ends on a 1-channel stage
    (3, 9, 13, 21),    # H*W odd (scalar path); width 4 ends on a 1-channel stage
    (5, 12, 16, 24),   # width 4 with bounds checks: the last stage pair is half full
    (6, 24, 8, 16),    # full stages, three stage pairs
    (800, 8, 64, 64),  # full stages, a grid of 1,600 workgroups
]


@pytest.mark.parametrize("shape", STREAM_SHAPES)
@pytest.mark.parametrize("kw", SMALL)
def test_streaming_pipeline_shapes(shape, kw):
    n, C, H, Wd = shape
    sp = W.small_spec(n=n, C=C, H=H, W=Wd, steps=5, num_buckets=3, feather=3, **kw)
    inp = W.make_inputs(sp)
    s = _sampler(inp)
    sig, table, cov = D.run_setup(inp)
    k = 1
    x_in = D.init_latent(inp, sig, sp.dtype).astype(np.float32)
    x = to_dev(x_in, sp.dtype)
    keep, stream = torch.full_like(x, float("nan")), torch.full_like(x, float("nan"))
    s.step(k, x, keep, cache_hint=0)
    s.step(k, x, stream, cache_hint=1)
    torch.cuda.synchronize()
    got = to_np(stream)
    assert np.array_equal(to_np(keep), got, equal_nan=True)
    p = D.build_plan(inp.start_step.astype(np.int64) + k, sp.steps, sp.num_buckets, table,
                     inp.cfg_override, cov)
    active = np.flatnonzero(p["bucket_id"] >= 0)
    assert active.size > 0
    for i, r in oracle_step_M(inp, sig, p, k, x_in, [int(active[0]), int(active[-1])]).items():
        assert np.array_equal(got[i], r), f"sample {i} differs from mode M"
    for i in np.flatnonzero(p["bucket_id"] < 0):
        assert np.isnan(got[i]).all()


@pytest.mark.parametrize("upload_batch,async_upload", [(1, False), (3, False), (8, True), (2, True)])
def test_native_loop_matches_python_loop(upload_batch, async_upload):
    inp = W.make_inputs(W.small_spec(n=5, C=3, H=16, W=24, regions=2, inpaint=True, steps=7,
                                     sampler="heun", dtype="bf16"))
    ref, _ = gpu_trajectory(_sampler(inp))
    s = _sampler(inp)
    x = s.init_state()
    loop = s.native_loop(x, upload_batch=upload_batch, async_upload=async_upload)
    loop.run(0, 3)
    ms = loop.run(3, 4, timing=True)
    torch.cuda.synchronize()
    loop.close()
    assert ms > 0
    assert np.array_equal(to_np(x), ref)


def test_native_loop_replicas_round_robin():
    inp = W.make_inputs(W.small_spec(n=3, C=2, H=8, W=16, regions=1, steps=6))
    s = _sampler(inp)
    x = torch.stack([s.init_state(), s.init_state()])
    loop = s.native_loop(x, upload_batch=2)
    loop.run(0, 6)
    torch.cuda.synchronize()
    loop.close()
    s2 = _sampler(inp)
    for r in range(2):  # launches r, r+2, r+4 are replica r's steps 0, 1, 2
        y = s2.init_state()
        for m in range(3):
            s2.step(m, y)
        torch.cuda.synchronize()
        assert torch.equal(x[r], y)


def test_batch_permutation_permutes_outputs():
    inp = W.make_inputs(W.small_spec(n=6, C=3, H=16, W=16, regions=2, steps=6))
    perm = np.array([3, 0, 5, 1, 4, 2])
    xa, _ = gpu_trajectory(_sampler(inp))
    xb, _ = gpu_trajectory(_sampler(inp.subset(perm)))
    assert np.array_equal(xa[perm], xb)


def test_bucket_count_invariance_gpu():
    base = W.small_spec(n=3, C=2, H=8, W=16, steps=16, curve=W.Curve("const", 1.7))
    outs = [gpu_trajectory(_sampler(W.make_inputs(dataclasses.replace(base, num_buckets=nb))))[0]
            for nb in (1, 4, 8, 16)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_resume_equals_uninterrupted():
    from bucketed_classifier_free_amd import Interrupted
    inp = W.make_inputs(W.small_spec(n=3, C=2, H=8, W=16, steps=6, sampler="heun"))
    full, _ = gpu_trajectory(_sampler(inp))
    s = _sampler(inp)
    x = s.init_state()
    with pytest.raises(Interrupted) as e:
        s.run(x, cancel=lambda k=iter(range(100)): next(k) >= 3)
    assert e.value.step == 3
    for k in range(3, 6):
        s.step(k, x)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(x), full)


def test_mask_broadcast_single_mask():
    sp = W.small_spec(n=3, C=2, H=8, W=16, steps=4, inpaint=True)
    inp = W.make_inputs(sp)
    inp.mask[:] = inp.mask[0]
    a, _ = gpu_trajectory(_sampler(inp))
    from bucketed_classifier_free_amd import GuidedSampler
    s = GuidedSampler.from_inputs(inp)
    s.d_mask = s.d_mask[:1].contiguous()
    b, _ = gpu_trajectory(s)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- latent init, stats

@pytest.mark.parametrize("name", ["tiny", "regional_inpaint", "throughput_bf16_heun"])
def test_latent_init_matches_oracle(name):
    inp = W.make_inputs(W.config(name))
    s = _sampler(inp)
    x = to_np(s.init_state())
    sig, _, _ = D.run_setup(inp)
    assert np.array_equal(x, M.init_latent32(inp, sig))
    d = D.init_latent(inp, sig, inp.spec.dtype)
    assert np.abs(x - d).max() <= (1e-6 * np.abs(d).max() if inp.spec.dtype == "f32"
                                   else 0.5 * bf16_ulp(np.abs(d).max()) + 1e-6)


@pytest.mark.parametrize("kw", [dict(regions=0), dict(regions=3, inpaint=True), dict(regions=2, dtype="bf16")])
def test_norm_stats_match_oracle(kw):
    from bucketed_classifier_free_amd import guided_step_workspace_size
    inp = W.make_inputs(W.small_spec(n=5, C=3, H=12, W=100, steps=5, skip_frac=0.4, **kw))
    sp = inp.spec
    s = _sampler(inp)
    sig, table, cov = D.run_setup(inp)
    x = s.init_state()
    x_np = to_np(x)
    stats = torch.zeros((sp.n, 3), device="cuda")
    ws = torch.empty(guided_step_workspace_size(sp.n, sp.C, sp.H, sp.W) // 4 + 1, device="cuda")
    p = s.step(0, x, torch.empty_like(x), stats=stats, workspace=ws)
    torch.cuda.synchronize()
    got = to_np(stats)
    dplan = D.build_plan(inp.start_step.astype(np.int64), sp.steps, sp.num_buckets, table,
                         inp.cfg_override, cov)
    for i in range(sp.n):
        if p.bucket_id[i] < 0:
            continue
        t = int(inp.start_step[i])
        ref = D.norm_stats(x_np[i].astype(np.float64), float(sig[t]), float(p.scale[i]),
                           D.sample_params(inp, i), bool(dplan["need_uncond"][i]))
        np.testing.assert_allclose(got[i], ref, rtol=1e-5, atol=1e-6)


FUSED_STATS = [dict(dtype="bf16", regions=2, H=12, W=128),              # 16 lanes a row
               dict(dtype="f32", regions=3, inpaint=True, H=9, W=128),  # 32 lanes a row
               dict(dtype="bf16", sampler="heun", H=20, W=32),           # 4 lanes a row
               dict(dtype="f32", regions=1, sampler="heun", H=7, W=4),   # 1 lane a row
               dict(dtype="bf16", regions=4, inpaint=True, H=40, W=64, vpt=2),
               dict(dtype="f32", regions=2, H=64, W=256, vpt=3)]         # 64 lanes a row


@pytest.mark.parametrize("kw", FUSED_STATS)
def test_fused_norm_stats_match_oracle(kw):
    # Shapes whose latent rows are power-of-two lane groups: the statistics
    # come from the step itself (no second pass over x); the step's output is
    # the same as without them, bit for bit.
    from bucketed_classifier_free_amd import guided_step_workspace_size
    kw = dict(kw)
    vpt = kw.pop("vpt", 0)
    inp = W.make_inputs(W.small_spec(n=5, C=3, steps=5, skip_frac=0.4, **kw))
    sp = inp.spec
    s = _sampler(inp)
    sig, table, cov = D.run_setup(inp)
    x = s.init_state()
    x_np = to_np(x)
    stats = torch.full((sp.n, 3), float("nan"), device="cuda")
    ws = torch.empty(guided_step_workspace_size(sp.n, sp.C, sp.H, sp.W) // 4 + 1, device="cuda")
    y, y0 = torch.full_like(x, float("nan")), torch.full_like(x, float("nan"))
    k = 1
    p = s.step(k, x, y, stats=stats, workspace=ws, launch_vpt=vpt)
    s.step(k, x, y0, launch_vpt=vpt)
    torch.cuda.synchronize()
    bits = torch.int16 if sp.dtype == "bf16" else torch.int32
    assert torch.equal(y.view(bits), y0.view(bits))
    got = to_np(stats)
    dplan = D.build_plan(inp.start_step.astype(np.int64) + k, sp.steps, sp.num_buckets, table,
                         inp.cfg_override, cov)
    for i in range(sp.n):
        if p.bucket_id[i] < 0:
            assert np.isnan(got[i]).all()
            continue
        t = int(inp.start_step[i]) + k
        ref = D.norm_stats(x_np[i].astype(np.float64), float(sig[t]), float(p.scale[i]),
                           D.sample_params(inp, i), bool(dplan["need_uncond"][i]))
        np.testing.assert_allclose(got[i], ref, rtol=1e-5, atol=1e-6)


# ---------------------------------------------------------------- standalone kernels

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(3, 4, 16, 32), (2, 3, 7, 9)])
def test_mask_blend_matches_oracle(dtype, shape):
    from bucketed_classifier_free_amd import mask_blend
    rng = np.random.default_rng(4)
    n, C, H, Wd = shape
    a = rng.standard_normal(shape).astype(np.float32)
    b = rng.standard_normal(shape).astype(np.float32)
    m = np.where(rng.random((n, 1, H, Wd)) < 0.5, 1.0, rng.random((n, 1, H, Wd))).astype(np.float32)
    if dtype == "bf16":
        a = D.round_bf16(a).astype(np.float32); b = D.round_bf16(b).astype(np.float32)
    A, B = to_dev(a, dtype), to_dev(b, dtype)
    out = torch.empty_like(A)
    mask_blend(A, B, torch.from_numpy(m).cuda(), out)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(out), M.mask_blend32(a, b, m, dtype))
    ref = np.stack([D.inpaint_blend(a[i].astype(np.float64), b[i].astype(np.float64), m[i, 0])
                    for i in range(n)])
    err = np.abs(to_np(out) - ref)
    if dtype == "f32":
        assert err.max() <= 1e-6 * np.abs(ref).max()
    else:
        assert np.all(err <= 0.5 * bf16_ulp(ref) + 1e-6)
    # in place into a, and the single broadcast mask
    mask_blend(A, B, torch.from_numpy(m[:1]).cuda(), A)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(A), M.mask_blend32(a, b, np.broadcast_to(m[:1], m.shape), dtype))


@pytest.mark.parametrize("shape,R", [((3, 4, 20, 30), 3), ((2, 2, 9, 13), 4), ((2, 3, 16, 16), 1)])
def test_area_accumulate_matches_oracle(shape, R):
    from bucketed_classifier_free_amd import area_accumulate, bcg_plan_build
    n, C, H, Wd = shape
    rng = np.random.default_rng(5)
    frac = np.stack([rng.uniform(0, 0.6, (n, R)), rng.uniform(0, 0.6, (n, R)),
                     rng.uniform(0.2, 0.6, (n, R)), rng.uniform(0.2, 0.6, (n, R))], -1)
    cnt = np.full(n, R, np.int32)
    cnt[-1] = max(R - 1, 1)
    st = rng.uniform(0.5, 1.5, (n, R)).astype(np.float32)
    plan = bcg_plan_build(np.zeros(n, np.int32), 1, np.float32([2.0]), C=C, H=H, W=Wd,
                          region_count=cnt, region_frac=frac, region_strength=st, max_regions=R)
    total = int(plan.region_off[-1])
    pred = rng.standard_normal(total).astype(np.float32)
    fb = rng.standard_normal(shape).astype(np.float32)
    out = torch.empty(shape, device="cuda")
    ws = torch.empty((n, H, Wd), device="cuda")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    area_accumulate(dev(pred), dev(plan.region_off), dev(cnt), dev(plan.region_box), dev(st), out,
                    feather=3, fallback=dev(fb), wsum_out=ws)
    torch.cuda.synchronize()
    got, gws = to_np(out), to_np(ws)
    for i in range(n):
        boxes = [tuple(plan.region_box[i, r]) for r in range(cnt[i])]
        crops = []
        for r, (y0, y1, x0, x1) in enumerate(boxes):
            o = int(plan.region_off[i * R + r])
            crops.append(pred[o:o + C * (y1 - y0) * (x1 - x0)].reshape(C, y1 - y0, x1 - x0))
        want, wsum = M.area_accumulate32(crops, boxes, st[i, :cnt[i]], H, Wd, 3, fb[i])
        assert np.array_equal(got[i], want)
        assert np.array_equal(gws[i], wsum)
        # mode D: weighted mean of the crops, fallback where uncovered
        wts = [D.region_weight(b, s, H, Wd, 3) for b, s in zip(boxes, st[i, :cnt[i]])]
        full = []
        for (y0, y1, x0, x1), cr in zip(boxes, crops):
            f = np.zeros((C, H, Wd)); f[:, y0:y1, x0:x1] = cr; full.append(f)
        ref = D.regional_cond(full, wts, fb[i].astype(np.float64))
        assert np.abs(got[i] - ref).max() <= 1e-5 * np.abs(ref).max()
