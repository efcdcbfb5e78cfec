"""Continuous batching on the device plan: slots refilled from a queue of
requests inside the step launches (guided_step_dplan through the native loop),
against the oracle's serve_trajectory: every slot's state after every launch
bit for bit equal to the fp32 mirror, the final states within the bars of
the float64 definition.
"""
import numpy as np
import pytest
import torch

import workloads as W
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


def _sampler(inp):
    from bucketed_classifier_free_amd import GuidedSampler
    return GuidedSampler.from_inputs(inp)


def _serve_gpu(inp, n_slots, launches, ring=False, reps=1, graph=0, per_launch=True, join_front=None):
    """Slot states after each launch (one replica's launches) from the native loop."""
    sp = inp.spec
    s = _sampler(inp)
    shape = (reps, n_slots, sp.C, sp.H, sp.W) if reps > 1 else (n_slots, sp.C, sp.H, sp.W)
    x = torch.full(shape, float("nan"), dtype=s.tdtype, device="cuda")  # every slot joins first
    loop = s.native_loop(x, device_plan=True, records=True, slots=n_slots, ring=ring,
                         graph_launches=graph, join_front=join_front)
    states = []
    step = reps if per_launch else reps * launches
    for k0 in range(0, reps * launches, step):
        loop.run(k0, step)
        torch.cuda.synchronize()
        states.append(to_np(x))
    loop.close()
    return states


def _check_final(inp, n, got, ref_d, req):
    """Final slot states vs mode D: fp32 within 1e-4 relative; bf16 per element
    within max(2e-2, 1 ulp), or else inside the carried-flip bound of the
    request the slot finished with (its solo trajectory)."""
    from gpu_helpers import storage_flip_bound
    sp = inp.spec
    for s in range(got.shape[0]):
        err = np.abs(got[s].astype(np.float64) - ref_d[s])
        if sp.dtype == "f32":
            assert err.max() <= 1e-4 * max(np.abs(ref_d[s]).max(), 1e-30), s
            continue
        over = err > np.maximum(2e-2, bf16_ulp(ref_d[s]))
        if over.any():
            r = int(req[req[:, s] >= 0, s][-1])
            solo = inp.subset([r])
            solo.start_step[:] = inp.start_step[r] if r < n else 0
            fb = storage_flip_bound(solo, 0, sp.steps - int(solo.start_step[0]))
            assert np.all(err[over] <= fb[over]), (s, r)


QUEUE_KW = [dict(dtype="f32", sampler="euler", regions=2),
            dict(dtype="bf16", sampler="euler", regions=2),
            dict(dtype="f32", sampler="heun", regions=3, inpaint=True),
            dict(dtype="bf16", sampler="heun", inpaint=True),
            dict(dtype="f32", sampler="euler"),
            dict(dtype="bf16", sampler="euler", regions=1, inpaint=True)]


@pytest.mark.parametrize("kw", QUEUE_KW)
@pytest.mark.parametrize("shape", [(3, 9, 4, 16, 24), (5, 13, 16, 8, 32)])
def test_queue_drains_matching_mirror_every_launch(kw, shape):
    # n slots, Q requests, channels, H, W; run until the queue has drained
    n, Q, C, H, Wd = shape
    sp = W.small_spec(n=Q, C=C, H=H, W=Wd, steps=4, num_buckets=3, feather=3, skip_frac=0.25, **kw)
    inp = W.make_inputs(sp)
    launches = -(-Q // n) * sp.steps + sp.steps
    got = _serve_gpu(inp, n, launches)
    _, mstates, (req, tt, join) = M.serve_trajectory32(inp, n, launches, keep=True)
    for k in range(launches):
        assert np.array_equal(got[k], mstates[k]), f"launch {k} differs from mode M"
    assert (req[-1] == -1).all()  # drained: every slot empty at the end
    xd, _, _ = D.serve_trajectory(inp, n, launches)
    _check_final(inp, n, got[-1], xd, req)


# the schedule and guidance variants under continuous batching: a mid-peak
# curve with within-bucket interpolation, regions with validity ranges (each
# request's own), Heun with inpainting
QUEUE_VARIANTS = [dict(dtype="f32", sampler="euler", regions=2, region_ranges=True, bucket_interp=True,
                       curve=W.Curve("mid_peak", 1.2, 3.0, 0.4)),
                  dict(dtype="bf16", sampler="heun", regions=1, region_ranges=True, inpaint=True,
                       curve=W.Curve("linear", 2.0, 1.0))]


@pytest.mark.parametrize("kw", QUEUE_VARIANTS)
def test_queue_variants_match_mirror_every_launch(kw):
    n, Q = 4, 11
    sp = W.small_spec(n=Q, C=3, H=16, W=24, steps=5, num_buckets=3, feather=3, skip_frac=0.25, **kw)
    inp = W.make_inputs(sp)
    launches = -(-Q // n) * sp.steps + sp.steps
    got = _serve_gpu(inp, n, launches)
    _, mstates, (req, _, _) = M.serve_trajectory32(inp, n, launches, keep=True)
    for k in range(launches):
        assert np.array_equal(got[k], mstates[k]), f"launch {k} differs from mode M"
    assert (req[-1] == -1).all()


@pytest.mark.parametrize("reps,graph,jf", [(1, 0, None), (2, 6, 0), (3, 4, 1), (1, 5, 2)])
def test_queue_ring_replicas_and_graphs(reps, graph, jf):
    # the endless queue (request ids modulo the pool), several replicas served
    # round robin, replays of captured graphs: each replica follows the oracle
    sp = W.small_spec(n=7, C=3, H=8, W=16, steps=5, num_buckets=3, regions=2, feather=2, dtype="bf16")
    inp = W.make_inputs(sp)
    n, launches = 4, 19
    got = _serve_gpu(inp, n, launches, ring=True, reps=reps, graph=graph, join_front=jf)
    _, mstates, (req, _, _) = M.serve_trajectory32(inp, n, launches, ring=True, keep=True)
    assert (req >= 0).all() and req.max() == sp.n - 1
    for k in range(launches):
        for r in range(reps):
            g = got[k][r] if reps > 1 else got[k]
            assert np.array_equal(g, mstates[k]), f"launch {k} replica {r}"


def test_queue_large_shape_sampled_slots():
    """256 slots of the large bf16 workload (16x128x128, 2 regions, 8 buckets)
    fed from a queue of 300 requests, two replicas, graph replays, streaming:
    sampled slots (some refilled within the run) against the mirror."""
    import dataclasses
    sp = dataclasses.replace(W.config("large_bf16"), n=300)
    inp = W.make_inputs(sp)
    n, launches = 256, 10
    s = _sampler(inp)
    x = torch.empty((2, n, sp.C, sp.H, sp.W), dtype=s.tdtype, device="cuda")
    loop = s.native_loop(x, device_plan=True, records=True, slots=n, graph_launches=4)
    refilled = [int(v) for v in np.flatnonzero(inp.start_step[:n] >= sp.steps - 4)[:3]]
    idx = sorted(set([0, 101] + refilled))
    _, mstates, (req, _, join) = M.serve_trajectory32(inp, n, launches, slots=idx, keep=True)
    assert join[1:, refilled].any()
    for k in range(launches):
        loop.run(2 * k, 2)
        torch.cuda.synchronize()
        for r in range(2):
            assert np.array_equal(to_np(x[r, idx]), mstates[k][idx]), f"launch {k} replica {r}"
    loop.close()
