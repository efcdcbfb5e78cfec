"""guided_step_dplan_static: the device-plan step whose statistics' partials
live in the library's static scratch (for callers that cannot allocate),
against guided_step_dplan with a caller workspace: outputs and statistics bit
for bit, on consecutive calls that share the scratch, the later ones smaller.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bucketed_classifier_free_amd
    bucketed_classifier_free_amd.load()  # fails loudly without libbcg.so


def _step(s, x, t, y, stats, static, workspace=None, k=0):
    from bucketed_classifier_free_amd import api
    kw = dict(steps=s.steps, bucket_cfg=s.d_table, step_in=torch.from_numpy(np.ascontiguousarray(t, np.int32)).cuda(),
              cfg_override=s.d_override, covered=s.d_covered, wrap=s.wrap, bucket_cfg_end=s.d_table_end,
              region_range=s.d_region_range, covered_sets=s.d_covered_sets, sampler=s.sampler, s2=s.s2,
              feather=s.feather, region_count=s.d_region_count, region_box=s.d_region_box,
              region_strength=s.d_region_strength, mu_region=s.d_mu_region, x_orig=s.d_x_orig,
              mask=s.d_mask, stats=stats)
    if static:
        api.guided_step_dplan_static(x, y, s.d_sigmas, s.d_mu_u, s.d_mu_c, **kw)
    else:
        api.guided_step_dplan(x, y, s.d_sigmas, s.d_mu_u, s.d_mu_c, workspace=workspace, **kw)


def _compare(inp, k):
    from bucketed_classifier_free_amd import GuidedSampler, guided_step_workspace_size
    sp = inp.spec
    s = GuidedSampler.from_inputs(inp, wrap=True)
    x = s.init_state()
    t = s.step_indices(k)
    ya, yb = torch.full_like(x, float("nan")), torch.full_like(x, float("nan"))
    sa = torch.full((sp.n, 3), float("nan"), device="cuda")
    sb = torch.full((sp.n, 3), float("nan"), device="cuda")
    ws = torch.empty(guided_step_workspace_size(sp.n, sp.C, sp.H, sp.W) // 4 + 1, device="cuda")
    _step(s, x, t, ya, sa, static=True)
    _step(s, x, t, yb, sb, static=False, workspace=ws)
    torch.cuda.synchronize()
    bits = torch.int16 if sp.dtype == "bf16" else torch.int32
    assert torch.equal(ya.view(bits), yb.view(bits))
    assert torch.equal(sa.view(torch.int32), sb.view(torch.int32))
    assert torch.isfinite(sa).all()  # every sample is active (wrapping steps)


def test_static_scratch_matches_workspace_on_consecutive_calls():
    large = W.make_inputs(W.config("large_bf16"))
    _compare(large, 5)                                      # 256 samples: 384 KiB of partials
    _compare(large.subset(np.arange(40, 77)), 11)           # 37 samples, the same scratch again
    mixed = W.make_inputs(W.config("mixed_bucket"))
    _compare(mixed.subset([6, 1, 3]), 2)                    # 3 fp32 samples, 32 lanes a row


def test_static_scratch_rejects_oversize_and_workspace():
    from bucketed_classifier_free_amd import GuidedSampler
    from bucketed_classifier_free_amd import _lib as L
    # 2,000 samples of 1x128x4 fp32: one lane a row, 256 row groups a sample,
    # 6 MB of partials > 4 MiB: rejected before any launch
    inp = W.make_inputs(W.small_spec(n=2000, C=1, H=128, W=4, steps=4))
    s = GuidedSampler.from_inputs(inp, wrap=True)
    x = s.init_state()
    y = torch.empty_like(x)
    st = torch.zeros((inp.spec.n, 3), device="cuda")
    with pytest.raises(L.BCGError) as e:
        _step(s, x, s.step_indices(0), y, st, static=True)
    assert e.value.code == L.BCG_EINVAL and "static scratch" in str(e.value)
    lib = L.lib()
    a = L.StepArgs()
    a.workspace = 0x1000
    d = L.DevicePlan()
    assert lib.guided_step_dplan_static(C_ref(a), C_ref(d), None) == L.BCG_EINVAL


def C_ref(o):
    import ctypes
    return ctypes.byref(o)
