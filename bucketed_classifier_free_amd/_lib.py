"""ctypes view of libbcg (include/bcg.h).  Loading fails loudly if the
library has not been built: there is no fallback implementation."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbcg.so")

BCG_OK, BCG_EINVAL, BCG_ESHAPE, BCG_EDTYPE, BCG_EHIP = 0, -1, -2, -3, -4
BCG_F32, BCG_BF16 = 0, 1
BCG_EULER, BCG_HEUN = 0, 1
BCG_SCHED_LOGLINEAR = 0
BCG_CACHE_KEEP, BCG_CACHE_STREAM = 0, 1
BCG_PHASE = {"euler": 0, "heun_predict": 1, "heun_correct": 2}
BCG_CURVE = {"const": 0, "linear": 1, "front_high": 2, "mid_peak": 3}
BCG_MAX_REGIONS = 4
BCG_MAX_CHANNELS = 64
BCG_MAX_FEATHER = 64
BCG_MAX_DEVICE_BUCKETS = 1024
BCG_MAX_DEVICE_STEPS = 1 << 20
BCG_MAX_PATCHES = 8
BCG_STATIC_SCRATCH_BYTES = 4 << 20
BCG_PATCH = {"diff": 0, "lowrank": 1}
BCG_ROUND = {"nearest": 0, "stochastic": 1}
ABI_VERSION = 9

# Every symbol the header declares (checked by the CPU test suite).
EXPORTS = ["bcg_last_error", "bcg_abi_version", "sigma_schedule", "sigma_crop", "bucket_table",
           "bucket_bounds",
           "bcg_plan_build", "guided_step", "guided_step_workspace_size", "latent_init",
           "area_accumulate", "mask_blend", "bcg_plan_records", "bcg_plan_device", "guided_step_dplan",
           "guided_step_dplan_static", "guided_step_rows",
           "guided_step_rows_dplan",
           "bcg_loop_create", "bcg_loop_run", "bcg_loop_last_run", "bcg_loop_destroy", "weight_patch"]

vp, i32p, i64p, f32p, f64p = (C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_int64),
                              C.POINTER(C.c_float), C.POINTER(C.c_double))


class PlanIn(C.Structure):
    _fields_ = [("n", C.c_int32), ("steps", C.c_int32), ("num_buckets", C.c_int32),
                ("C", C.c_int32), ("H", C.c_int32), ("W", C.c_int32),
                ("max_regions", C.c_int32),
                ("bucket_cfg", vp), ("step_idx", vp), ("cfg_override", vp),
                ("region_count", vp), ("region_frac", vp), ("region_strength", vp),
                ("covered", vp), ("bucket_cfg_end", vp), ("region_range", vp),
                ("covered_sets", vp)]


class PlanOut(C.Structure):
    _fields_ = [("bucket_id", vp), ("scale", vp), ("uncond_row", vp), ("cond_row", vp),
                ("order", vp), ("bucket_count", vp), ("bucket_offset", vp),
                ("uncond_offset", vp), ("region_box", vp), ("region_off", vp),
                ("covered_out", vp), ("n_active", C.c_int32), ("n_uncond", C.c_int32),
                ("covered_sets_out", vp), ("region_valid", vp)]


class StepArgs(C.Structure):
    _fields_ = [("n", C.c_int32), ("C", C.c_int32), ("H", C.c_int32), ("W", C.c_int32),
                ("dtype", C.c_int32), ("sampler", C.c_int32), ("max_regions", C.c_int32),
                ("feather", C.c_int32), ("n_active", C.c_int32), ("num_sigmas", C.c_int32),
                ("mask_per_sample", C.c_int32), ("cache_hint", C.c_int32), ("s2", C.c_float),
                ("x", vp), ("x_out", vp), ("sigmas", vp), ("order", vp), ("step_idx", vp),
                ("scale", vp), ("uncond_row", vp), ("mu_uncond", vp), ("mu_cond", vp),
                ("region_count", vp), ("region_box", vp), ("region_strength", vp),
                ("mu_region", vp), ("x_orig", vp), ("mask", vp), ("stats", vp),
                ("workspace", vp), ("workspace_bytes", C.c_size_t), ("region_range", vp),
                ("steps", C.c_int32), ("launch_vpt", C.c_int32)]


class RowsArgs(C.Structure):
    _fields_ = [("n", C.c_int32), ("C", C.c_int32), ("H", C.c_int32), ("W", C.c_int32),
                ("dtype", C.c_int32), ("phase", C.c_int32), ("n_active", C.c_int32),
                ("num_sigmas", C.c_int32), ("rows", C.c_int32), ("mask_per_sample", C.c_int32),
                ("cache_hint", C.c_int32), ("x", vp), ("x_out", vp), ("d", vp), ("x_tilde", vp),
                ("pred", vp), ("sigmas", vp), ("order", vp), ("step_idx", vp), ("scale", vp),
                ("uncond_row", vp), ("cond_row", vp), ("x_orig", vp), ("mask", vp),
                ("launch_vpt", C.c_int32)]


class DevicePlan(C.Structure):
    _fields_ = [("steps", C.c_int32), ("num_buckets", C.c_int32), ("wrap", C.c_int32),
                ("bucket_cfg", vp), ("cfg_override", vp), ("covered", vp), ("step_in", vp),
                ("step_out", vp), ("bucket_id", vp), ("scale", vp), ("uncond_row", vp),
                ("cond_row", vp), ("order", vp), ("bucket_count", vp), ("bucket_offset", vp),
                ("uncond_offset", vp), ("totals", vp), ("bucket_cfg_end", vp),
                ("record_in", vp), ("record_out", vp), ("sigmas", vp), ("num_sigmas", C.c_int32),
                ("region_range", vp), ("covered_sets", vp), ("region_count", vp),
                ("max_regions", C.c_int32),
                ("queue_len", C.c_int32), ("queue_ring", C.c_int32), ("noise", vp),
                ("slot_req_in", vp), ("slot_req_out", vp), ("queue_in", vp), ("queue_out", vp),
                ("join_front", C.c_int32), ("join_in", vp), ("join_out", vp)]


class Patch(C.Structure):
    _fields_ = [("kind", C.c_int32), ("offset", C.c_int32), ("rows", C.c_int32), ("rank", C.c_int32),
                ("dtype", C.c_int32), ("strength_patch", C.c_float), ("strength_model", C.c_float),
                ("reserved", C.c_int32), ("diff", vp), ("up", vp), ("down", vp)]


class WeightArgs(C.Structure):
    _fields_ = [("rows", C.c_int32), ("cols", C.c_int32), ("w_dtype", C.c_int32),
                ("out_dtype", C.c_int32), ("num_patches", C.c_int32), ("rounding", C.c_int32),
                ("seed", C.c_uint64), ("w", vp), ("out", vp), ("patches", vp)]


class LoopDesc(C.Structure):
    _fields_ = [("plan", PlanIn), ("start", vp), ("wrap", C.c_int32), ("rows", C.c_int32),
                ("host_slab", vp), ("dev_slab", vp), ("replicas", C.c_int32),
                ("replica_stride", C.c_int64), ("upload_batch", C.c_int32),
                ("async_upload", C.c_int32), ("step", StepArgs),
                ("device_plan", C.c_int32), ("graph_launches", C.c_int32), ("dev_steps", vp),
                ("dplan", DevicePlan), ("dev_records", vp),
                ("queue_len", C.c_int32), ("queue_ring", C.c_int32), ("noise", vp), ("dev_queue", vp),
                ("join_front", C.c_int32)]


_lib = None


def _signatures():
    """Argument and result types of every exported function."""
    ip = C.POINTER(C.c_int)
    return {
        "bcg_last_error": ([], C.c_char_p),
        "bcg_abi_version": ([], C.c_int),
        "sigma_schedule": ([C.c_int, C.c_double, C.c_double, C.c_int, C.c_double, vp, ip], C.c_int),
        "bucket_table": ([C.c_int, C.c_double, C.c_double, C.c_double, C.c_int, vp], C.c_int),
        "bucket_bounds": ([C.c_int, C.c_double, C.c_double, C.c_double, C.c_int, vp, vp], C.c_int),
        "sigma_crop": ([vp, C.c_int, C.c_int, C.c_int, C.c_int, vp, ip], C.c_int),
        "bcg_plan_build": ([C.POINTER(PlanIn), C.POINTER(PlanOut)], C.c_int),
        "bcg_plan_records": ([C.c_int, C.c_int, vp, vp, vp, vp, vp, C.c_int, vp], C.c_int),
        "guided_step": ([C.POINTER(StepArgs), vp], C.c_int),
        "bcg_plan_device": ([C.c_int, C.POINTER(DevicePlan), vp], C.c_int),
        "guided_step_rows": ([C.POINTER(RowsArgs), vp], C.c_int),
        "guided_step_rows_dplan": ([C.POINTER(RowsArgs), C.POINTER(DevicePlan), vp], C.c_int),
        "guided_step_dplan": ([C.POINTER(StepArgs), C.POINTER(DevicePlan), vp], C.c_int),
        "guided_step_dplan_static": ([C.POINTER(StepArgs), C.POINTER(DevicePlan), vp], C.c_int),
        "guided_step_workspace_size": ([C.c_int] * 5, C.c_size_t),
        "latent_init": ([C.c_int] * 5 + [vp, vp, vp, C.c_int, vp, vp, vp], C.c_int),
        "area_accumulate": ([C.c_int] * 6 + [vp, C.c_int64] + [vp] * 7 + [vp], C.c_int),
        "mask_blend": ([C.c_int] * 5 + [vp, vp, vp, C.c_int, vp, vp], C.c_int),
        "bcg_loop_create": ([C.POINTER(LoopDesc), C.POINTER(vp)], C.c_int),
        "bcg_loop_run": ([vp, C.c_int, C.c_int, vp, C.POINTER(C.c_float)], C.c_int),
        "bcg_loop_destroy": ([vp], C.c_int),
        "bcg_loop_last_run": ([vp, C.POINTER(C.c_int32), C.POINTER(C.c_int32)], C.c_int),
        "weight_patch": ([C.POINTER(WeightArgs), vp], C.c_int),
    }


# The functions of the host half (bcg_host.cpp: plain C++, no GPU calls).
HOST_EXPORTS = ["bcg_last_error", "bcg_abi_version", "sigma_schedule", "bucket_table", "bucket_bounds",
                "sigma_crop", "bcg_plan_build", "bcg_plan_records"]


def configure(cdll, names):
    """Set the argument and result types of the functions ``names`` of a
    loaded library and return it."""
    sig = _signatures()
    for name in names:
        fn = getattr(cdll, name)
        fn.argtypes, fn.restype = sig[name]
    return cdll


def lib():
    """The loaded library (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libbcg.so not found at {LIB_PATH}; build it with "
                               "`python -m bucketed_classifier_free_amd.build`")
        _lib = configure(C.CDLL(LIB_PATH), EXPORTS)
    return _lib


class BCGError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libbcg error {code}: {msg}")
        self.code = code


def check(rc: int):
    if rc != BCG_OK:
        raise BCGError(rc, lib().bcg_last_error().decode())
