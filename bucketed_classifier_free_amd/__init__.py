"""MI355X-native bucketed classifier-free guidance: the per-step guided
denoising update of a diffusion sampler as hand-written HIP for gfx950, and
the weight-patch kernel (diff and low-rank patches, stochastic rounding).

The compute lives in ``libbcg.so`` (C ABI in ``include/bcg.h``); this package
is its ctypes binding plus the host sampler loop.  The library is loaded on
first use; every entry point raises if it has not been built (there is no
fallback implementation).
"""
from . import _lib
from ._lib import BCGError
from .api import (Plan, area_accumulate, bcg_plan_build, bcg_plan_device, bucket_bounds, bucket_table,
                  guided_step, guided_step_dplan, guided_step_dplan_static, guided_step_rows,
                  guided_step_rows_dplan,
                  guided_step_workspace_size,
                  latent_init, mask_blend, sigma_crop, sigma_schedule, WeightPatch, weight_patch)
from .sampler import GuidedSampler, Interrupted


def load():
    """Load libbcg.so now (raises RuntimeError if it is missing)."""
    return _lib.lib()

__all__ = ["BCGError", "Plan", "GuidedSampler", "Interrupted", "area_accumulate",
           "bcg_plan_build", "bcg_plan_device", "bucket_bounds", "bucket_table", "guided_step",
           "guided_step_dplan", "guided_step_dplan_static", "guided_step_rows", "guided_step_rows_dplan", "guided_step_workspace_size",
           "latent_init",
           "mask_blend", "sigma_crop", "sigma_schedule", "WeightPatch", "weight_patch"]
