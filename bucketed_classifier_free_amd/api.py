"""Thin Python wrappers over libbcg with the C ABI's names.

Argument marshalling only: checks of dtype, device, contiguity and shape
(raising ValueError before any call), pointer extraction, and the current
torch stream as the HIP stream.  Every step of the path runs inside libbcg.
"""
from __future__ import annotations

import ctypes as ct
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib as L

_DT = {torch.float32: L.BCG_F32, torch.bfloat16: L.BCG_BF16}
_SAMPLER = {"euler": L.BCG_EULER, "heun": L.BCG_HEUN}


def _np_ptr(a):
    return None if a is None else a.ctypes.data


def _np(a, dtype, shape=None, name="array"):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=dtype)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"{name}: shape {a.shape}, expected {tuple(shape)}")
    return a


def _dev(t, name, dtype=None, shape=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ---------------------------------------------------------------- host calls

def sigma_schedule(sigma_max: float, sigma_min: float, steps: int, denoise: float = 1.0,
                   kind: int = L.BCG_SCHED_LOGLINEAR):
    """float32[steps+1] descending sigmas and the base schedule length."""
    out = np.empty(steps + 1 if steps >= 1 else 1, np.float32)
    nb = ct.c_int(0)
    L.check(L.lib().sigma_schedule(kind, sigma_max, sigma_min, steps, denoise, _np_ptr(out),
                                   ct.byref(nb)))
    return out, nb.value


def sigma_crop(sigmas, start_step: int, last_step: int = -1, force_full_denoise: bool = False):
    """sigmas[start_step .. last_step] (staged sampling), last sigma forced to
    0 with ``force_full_denoise`` (see include/bcg.h)."""
    s = _np(sigmas, np.float32, name="sigmas")
    out = np.empty(max(s.size, 1), np.float32)
    cnt = ct.c_int(0)
    L.check(L.lib().sigma_crop(_np_ptr(s), s.size, int(start_step), int(last_step),
                               1 if force_full_denoise else 0, _np_ptr(out), ct.byref(cnt)))
    return out[:cnt.value].copy()


def bucket_table(curve: str, p0: float, p1: float = 0.0, p2: float = 0.0, num_buckets: int = 1):
    if curve not in L.BCG_CURVE:
        raise ValueError(f"unknown curve {curve!r}")
    out = np.empty(max(num_buckets, 1), np.float32)
    L.check(L.lib().bucket_table(L.BCG_CURVE[curve], p0, p1, p2, num_buckets, _np_ptr(out)))
    return out


def bucket_bounds(curve: str, p0: float, p1: float = 0.0, p2: float = 0.0, num_buckets: int = 1):
    """The curve at the start and end of each bucket (float32 lo, hi): the
    tables of the within-bucket interpolation."""
    if curve not in L.BCG_CURVE:
        raise ValueError(f"unknown curve {curve!r}")
    lo = np.empty(max(num_buckets, 1), np.float32)
    hi = np.empty(max(num_buckets, 1), np.float32)
    L.check(L.lib().bucket_bounds(L.BCG_CURVE[curve], p0, p1, p2, num_buckets, _np_ptr(lo),
                                  _np_ptr(hi)))
    return lo, hi


@dataclass
class Plan:
    bucket_id: np.ndarray
    scale: np.ndarray
    uncond_row: np.ndarray
    cond_row: np.ndarray
    order: np.ndarray
    bucket_count: np.ndarray
    bucket_offset: np.ndarray
    uncond_offset: np.ndarray
    region_box: np.ndarray | None
    region_off: np.ndarray | None
    covered: np.ndarray
    n_active: int
    n_uncond: int
    covered_sets: np.ndarray | None = None
    region_valid: np.ndarray | None = None


def plan_out_arrays(n, nb, R, bucket_id=None, scale=None, uncond_row=None, order=None):
    """Output arrays of bcg_plan_build (optionally writing into given views)."""
    z = lambda a, k, dt: a if a is not None else np.empty(k, dt)
    return dict(bucket_id=z(bucket_id, n, np.int32), scale=z(scale, n, np.float32),
                uncond_row=z(uncond_row, n, np.int32), cond_row=np.empty(n, np.int32),
                order=z(order, n, np.int32), bucket_count=np.empty(nb, np.int32),
                bucket_offset=np.empty(nb + 1, np.int32), uncond_offset=np.empty(nb + 1, np.int32),
                region_box=np.empty((n, R, 4), np.int32) if R > 0 else None,
                region_off=np.empty(n * R + 1, np.int64) if R > 0 else None,
                covered=np.empty(n, np.uint8), covered_sets=np.empty(n, np.uint16),
                region_valid=np.empty(n, np.int32))


def bcg_plan_build(step_idx, steps: int, bucket_cfg, *, C: int = 1, H: int = 1, W: int = 1,
                   cfg_override=None, region_count=None, region_frac=None,
                   region_strength=None, max_regions: int = 0, covered=None, out=None,
                   bucket_cfg_end=None, region_range=None, covered_sets=None) -> Plan:
    """Bucket plan of one step (host arrays in, host arrays out).

    ``covered`` (optional, [n] bool/uint8) supplies the per-sample coverage
    flags of an earlier plan; the region arrays are then not used.
    ``bucket_cfg_end`` (optional) turns on the within-bucket interpolation.
    ``region_range`` ([n, R, 2] progress ranges) limits each region to the
    steps it is valid at; ``covered_sets`` caches the subset coverage."""
    step_idx = _np(step_idx, np.int32, name="step_idx")
    n = step_idx.size
    cfg = _np(bucket_cfg, np.float32, name="bucket_cfg")
    nb = cfg.size
    R = int(max_regions)
    ov = _np(cfg_override, np.float32, (n,), "cfg_override")
    rc = _np(region_count, np.int32, (n,), "region_count") if R > 0 and region_count is not None else None
    rf = _np(region_frac, np.float64, (n, R, 4), "region_frac") if rc is not None else None
    rs = _np(region_strength, np.float32, (n, R), "region_strength") if rc is not None else None
    cov = _np(covered, np.uint8, (n,), "covered")
    cend = _np(bucket_cfg_end, np.float32, (nb,), "bucket_cfg_end")
    rr = _np(region_range, np.float64, (n, R, 2), "region_range") if R > 0 and region_range is not None else None
    cs = _np(covered_sets, np.uint16, (n,), "covered_sets")
    o = out if out is not None else plan_out_arrays(n, nb, R)
    pin = L.PlanIn(n, steps, nb, C, H, W, R, _np_ptr(cfg), _np_ptr(step_idx), _np_ptr(ov),
                   _np_ptr(rc), _np_ptr(rf), _np_ptr(rs), _np_ptr(cov), _np_ptr(cend), _np_ptr(rr),
                   _np_ptr(cs))
    pout = L.PlanOut(*(_np_ptr(o[k]) for k in ("bucket_id", "scale", "uncond_row", "cond_row",
                                               "order", "bucket_count", "bucket_offset",
                                               "uncond_offset", "region_box", "region_off",
                                               "covered")),
                     0, 0, _np_ptr(o.get("covered_sets")), _np_ptr(o.get("region_valid")))
    L.check(L.lib().bcg_plan_build(ct.byref(pin), ct.byref(pout)))
    return Plan(o["bucket_id"], o["scale"], o["uncond_row"], o["cond_row"], o["order"],
                o["bucket_count"], o["bucket_offset"], o["uncond_offset"], o["region_box"],
                o["region_off"], o["covered"].astype(bool), int(pout.n_active),
                int(pout.n_uncond), o.get("covered_sets"), o.get("region_valid"))


# ---------------------------------------------------------------- device calls

def guided_step_workspace_size(n, C, H, W, dtype=torch.float32) -> int:
    return int(L.lib().guided_step_workspace_size(n, C, H, W, _DT[dtype]))


def _step_args(x, x_out, sigmas, mu_uncond, mu_cond, plan_rows, *, n_active, sampler, s2, feather,
               region_count, region_box, region_strength, mu_region, x_orig, mask, stats,
               workspace, cache_hint, region_range=None, steps=0, launch_vpt=0, static_scratch=False,
               tables=None):
    """Checks the tensors of a guided step and packs them into StepArgs.
    ``plan_rows`` = (order, step_idx, scale, uncond_row) or None (device plan)."""
    _dev(x, "x")
    if x.dim() != 4:
        raise ValueError("x must be [n, C, H, W]")
    if x.dtype not in _DT:
        raise ValueError(f"x: unsupported dtype {x.dtype}")
    n, Cc, H, W = x.shape
    _dev(x_out, "x_out", x.dtype, x.shape)
    _dev(sigmas, "sigmas", torch.float32)
    if sigmas.dim() != 1:
        raise ValueError("sigmas must be 1-D")
    order = step_idx = scale = uncond_row = None
    if plan_rows is not None:
        order, step_idx, scale, uncond_row = plan_rows
        _dev(order, "order", torch.int32)
        if order.numel() < n_active:
            raise ValueError("order shorter than n_active")
        for t, nm, dt in ((step_idx, "step_idx", torch.int32), (scale, "scale", torch.float32),
                          (uncond_row, "uncond_row", torch.int32)):
            _dev(t, nm, dt)
            if t.numel() < n:
                raise ValueError(f"{nm}: needs {n} entries")
    nt = n if tables is None else int(tables)  # per-sample tables (requests under a queue)
    _dev(mu_uncond, "mu_uncond", torch.float32, (nt, Cc))
    _dev(mu_cond, "mu_cond", torch.float32, (nt, Cc))
    R = 0
    if region_count is not None:
        _dev(region_count, "region_count", torch.int32, (nt,))
        _dev(region_box, "region_box", torch.int32)
        if region_box.dim() != 3 or region_box.shape[0] != nt or region_box.shape[2] != 4:
            raise ValueError("region_box must be [n, R, 4]")
        R = region_box.shape[1]
        _dev(region_strength, "region_strength", torch.float32, (nt, R))
        _dev(mu_region, "mu_region", torch.float32, (nt, R, Cc))
    mps = 0
    if x_orig is not None or mask is not None:
        _dev(x_orig, "x_orig", x.dtype, (nt, Cc, H, W))
        _dev(mask, "mask", torch.float32)
        if tuple(mask.shape) == (nt, 1, H, W):
            mps = 1
        elif tuple(mask.shape) != (1, 1, H, W):
            raise ValueError(f"mask: shape {tuple(mask.shape)} is neither [n,1,H,W] nor [1,1,H,W]")
    wsb = 0
    if stats is not None:
        _dev(stats, "stats", torch.float32, (n, 3))
        if not static_scratch:  # the static entry point brings its own
            _dev(workspace, "workspace")
            wsb = workspace.numel() * workspace.element_size()
    if sampler not in _SAMPLER:
        raise ValueError(f"unknown sampler {sampler!r}")
    if region_range is not None:
        _dev(region_range, "region_range", torch.float64, (n, R, 2))
    return L.StepArgs(n, Cc, H, W, _DT[x.dtype], _SAMPLER[sampler], R, int(feather), int(n_active),
                      sigmas.numel(), mps, int(cache_hint), float(s2),
                      _ptr(x), _ptr(x_out), _ptr(sigmas), _ptr(order), _ptr(step_idx), _ptr(scale),
                      _ptr(uncond_row), _ptr(mu_uncond), _ptr(mu_cond), _ptr(region_count),
                      _ptr(region_box), _ptr(region_strength), _ptr(mu_region), _ptr(x_orig),
                      _ptr(mask), _ptr(stats), _ptr(workspace), wsb, _ptr(region_range), int(steps),
                      int(launch_vpt))


def guided_step(x, x_out, sigmas, order, step_idx, scale, uncond_row, mu_uncond, mu_cond, *,
                n_active: int, sampler: str, s2: float, feather: int = 0,
                region_count=None, region_box=None, region_strength=None, mu_region=None,
                x_orig=None, mask=None, stats=None, workspace=None, cache_hint: int = 0,
                region_range=None, steps: int = 0, launch_vpt: int = 0, stream=None):
    """One fused guided sampler step (see include/bcg.h).  All tensors on the GPU.
    ``launch_vpt`` > 0 fixes the pixel vectors per lane of the launch shape."""
    a = _step_args(x, x_out, sigmas, mu_uncond, mu_cond, (order, step_idx, scale, uncond_row),
                   n_active=n_active, sampler=sampler, s2=s2, feather=feather,
                   region_count=region_count, region_box=region_box,
                   region_strength=region_strength, mu_region=mu_region, x_orig=x_orig, mask=mask,
                   stats=stats, workspace=workspace, cache_hint=cache_hint,
                   region_range=region_range, steps=steps, launch_vpt=launch_vpt)
    L.check(L.lib().guided_step(ct.byref(a), _stream(stream)))


def _rows_args(x, x_out, pred, sigmas, order, step_idx, scale, uncond_row, cond_row, *,
               n_active, phase, d, x_tilde, x_orig, mask, cache_hint, launch_vpt=0) -> L.RowsArgs:
    _dev(x, "x")
    if x.dim() != 4 or x.dtype not in _DT:
        raise ValueError("x must be [n, C, H, W] float32 or bfloat16")
    n, Cc, H, W = x.shape
    _dev(x_out, "x_out", x.dtype, x.shape)
    _dev(pred, "pred", x.dtype)
    if pred.dim() != 4 or tuple(pred.shape[1:]) != (Cc, H, W):
        raise ValueError("pred must be [rows, C, H, W]")
    _dev(sigmas, "sigmas", torch.float32)
    _dev(order, "order", torch.int32)
    if order.numel() < n_active:
        raise ValueError("order shorter than n_active")
    for t, nm, dt in ((step_idx, "step_idx", torch.int32), (scale, "scale", torch.float32),
                      (uncond_row, "uncond_row", torch.int32), (cond_row, "cond_row", torch.int32)):
        _dev(t, nm, dt)
        if t.numel() < n:
            raise ValueError(f"{nm}: needs {n} entries")
    if phase not in L.BCG_PHASE:
        raise ValueError(f"unknown phase {phase!r}")
    _dev(d, "d", torch.float32, x.shape, allow_none=True)
    _dev(x_tilde, "x_tilde", x.dtype, x.shape, allow_none=True)
    mps = 0
    if x_orig is not None or mask is not None:
        _dev(x_orig, "x_orig", x.dtype, x.shape)
        _dev(mask, "mask", torch.float32)
        if tuple(mask.shape) == (n, 1, H, W):
            mps = 1
        elif tuple(mask.shape) != (1, 1, H, W):
            raise ValueError(f"mask: shape {tuple(mask.shape)} is neither [n,1,H,W] nor [1,1,H,W]")
    a = L.RowsArgs(n, Cc, H, W, _DT[x.dtype], L.BCG_PHASE[phase], int(n_active), sigmas.numel(),
                   pred.shape[0], mps, int(cache_hint), _ptr(x), _ptr(x_out), _ptr(d),
                   _ptr(x_tilde), _ptr(pred), _ptr(sigmas), _ptr(order), _ptr(step_idx),
                   _ptr(scale), _ptr(uncond_row), _ptr(cond_row), _ptr(x_orig), _ptr(mask),
                   int(launch_vpt))
    return a


def guided_step_rows(x, x_out, pred, sigmas, order, step_idx, scale, uncond_row, cond_row, *,
                     n_active: int, phase: str = "euler", d=None, x_tilde=None, x_orig=None,
                     mask=None, cache_hint: int = 0, launch_vpt: int = 0, stream=None):
    """The guided update from materialised branch predictions ``pred``
    [rows, C, H, W] in the plan's [uncond | cond] layout (see include/bcg.h);
    ``phase`` is "euler", "heun_predict" (writes ``d`` and x~ to x_out) or
    "heun_correct" (reads ``d`` and, for last steps, ``x_tilde``)."""
    a = _rows_args(x, x_out, pred, sigmas, order, step_idx, scale, uncond_row, cond_row,
                   n_active=n_active, phase=phase, d=d, x_tilde=x_tilde, x_orig=x_orig, mask=mask,
                   cache_hint=cache_hint, launch_vpt=launch_vpt)
    L.check(L.lib().guided_step_rows(ct.byref(a), _stream(stream)))


def guided_step_rows_dplan(x, x_out, pred, sigmas, order, step_idx, scale, uncond_row, cond_row, *,
                           n_active: int, plan: L.DevicePlan, phase: str = "euler", d=None,
                           x_tilde=None, x_orig=None, mask=None, cache_hint: int = 0, stream=None):
    """guided_step_rows, and in the same launch the device plan ``plan``
    (from device_plan(): typically the next step's) as bcg_plan_device builds it."""
    a = _rows_args(x, x_out, pred, sigmas, order, step_idx, scale, uncond_row, cond_row,
                   n_active=n_active, phase=phase, d=d, x_tilde=x_tilde, x_orig=x_orig, mask=mask,
                   cache_hint=cache_hint)
    if not isinstance(plan, L.DevicePlan):
        raise ValueError("plan must come from device_plan()")
    L.check(L.lib().guided_step_rows_dplan(ct.byref(a), ct.byref(plan), _stream(stream)))


# ---------------------------------------------------------------- device plans

_PLAN_KEYS = ("bucket_id", "scale", "uncond_row", "cond_row", "order", "bucket_count",
              "bucket_offset", "uncond_offset", "totals")


def device_plan_arrays(n: int, nb: int, device="cuda") -> dict:
    """Device output arrays of one device-built plan."""
    e = lambda k, dt: torch.empty(k, dtype=dt, device=device)
    i32 = torch.int32
    return dict(bucket_id=e(n, i32), scale=e(n, torch.float32), uncond_row=e(n, i32),
                cond_row=e(n, i32), order=e(n, i32), bucket_count=e(nb, i32),
                bucket_offset=e(nb + 1, i32), uncond_offset=e(nb + 1, i32), totals=e(2, i32))


def device_plan(steps: int, bucket_cfg, step_in, *, step_out=None, cfg_override=None,
                covered=None, wrap: bool = False, out=None, bucket_cfg_end=None,
                record_in=None, record_out=None, sigmas=None, region_range=None,
                covered_sets=None, region_count=None, queue=None) -> L.DevicePlan:
    """Packs the device arrays of a device-built plan (see include/bcg.h).
    ``queue`` (continuous batching) is a dict: len, ring, noise [len, C, H, W]
    fp32, slot_req_in / slot_req_out [n] and queue_in / queue_out [1] int32,
    optionally join_front J with join_in / join_out [J] int32; the per-sample
    tables then hold ``len`` requests."""
    _dev(step_in, "step_in", torch.int32)
    n = step_in.numel()
    nt = int(queue["len"]) if queue else n  # entries of the per-sample tables
    _dev(bucket_cfg, "bucket_cfg", torch.float32)
    nb = bucket_cfg.numel()
    _dev(step_out, "step_out", torch.int32, allow_none=True)
    if step_out is not None and step_out.numel() < n:
        raise ValueError("step_out: needs n entries")
    _dev(cfg_override, "cfg_override", torch.float32, (nt,), allow_none=True)
    _dev(covered, "covered", torch.int32, (nt,), allow_none=True)
    _dev(bucket_cfg_end, "bucket_cfg_end", torch.float32, (nb,), allow_none=True)
    R = 0
    if region_range is not None:
        _dev(region_range, "region_range", torch.float64)
        if region_range.dim() != 3 or region_range.shape[0] != nt or region_range.shape[2] != 2:
            raise ValueError("region_range must be [n, R, 2] (one row per request under continuous batching)")
        R = region_range.shape[1]
        _dev(covered_sets, "covered_sets", torch.int16, (nt,))
    _dev(region_count, "region_count", torch.int32, (nt,), allow_none=True)
    _dev(record_in, "record_in", torch.float32, (n, 4), allow_none=True)
    _dev(record_out, "record_out", torch.float32, (n, 4), allow_none=True)
    _dev(sigmas, "sigmas", torch.float32, allow_none=True)
    ptrs = [None] * len(_PLAN_KEYS)
    if out is not None:
        for k, dt, size in (("bucket_id", torch.int32, n), ("scale", torch.float32, n),
                            ("uncond_row", torch.int32, n), ("cond_row", torch.int32, n),
                            ("order", torch.int32, n), ("bucket_count", torch.int32, nb),
                            ("bucket_offset", torch.int32, nb + 1),
                            ("uncond_offset", torch.int32, nb + 1), ("totals", torch.int32, 2)):
            _dev(out[k], k, dt)
            if out[k].numel() < size:
                raise ValueError(f"{k}: needs {size} entries")
        ptrs = [_ptr(out[k]) for k in _PLAN_KEYS]
    q = [0, 0, None, None, None, None, None, 0, None, None]
    if queue:
        _dev(queue["noise"], "noise", torch.float32)
        if queue["noise"].shape[0] != nt:
            raise ValueError("noise: needs one entry per request")
        for k in ("slot_req_in", "slot_req_out"):
            _dev(queue[k], k, torch.int32, (n,))
        for k in ("queue_in", "queue_out"):
            _dev(queue[k], k, torch.int32, (1,))
        J = int(queue.get("join_front", 0))
        if J:
            for k in ("join_in", "join_out"):
                _dev(queue[k], k, torch.int32, (J,))
        q = [nt, 1 if queue.get("ring") else 0, _ptr(queue["noise"]), _ptr(queue["slot_req_in"]),
             _ptr(queue["slot_req_out"]), _ptr(queue["queue_in"]), _ptr(queue["queue_out"]), J,
             _ptr(queue.get("join_in")) if J else None, _ptr(queue.get("join_out")) if J else None]
    return L.DevicePlan(int(steps), nb, 1 if wrap else 0, _ptr(bucket_cfg), _ptr(cfg_override),
                        _ptr(covered), _ptr(step_in), _ptr(step_out), *ptrs, _ptr(bucket_cfg_end),
                        _ptr(record_in), _ptr(record_out), _ptr(sigmas),
                        0 if sigmas is None else sigmas.numel(), _ptr(region_range),
                        _ptr(covered_sets), _ptr(region_count), R, *q)


def plan_records(plan, step_idx, steps: int, sigmas, ranged: bool = False):
    """Sample records (float32 [n, 4]: sigma, sigma', scale, flag bits) of the
    step indices of a host plan (see include/bcg.h)."""
    t = _np(step_idx, np.int32, name="step_idx")
    n = t.size
    sg = _np(sigmas, np.float32, name="sigmas")
    out = np.zeros((n, 4), np.float32)
    L.check(L.lib().bcg_plan_records(n, int(steps), _np_ptr(t), _np_ptr(np.ascontiguousarray(plan.scale)),
                                     _np_ptr(np.ascontiguousarray(plan.uncond_row)),
                                     _np_ptr(np.ascontiguousarray(plan.region_valid)) if ranged else None,
                                     _np_ptr(sg),
                                     sg.size, _np_ptr(out)))
    return out


def bcg_plan_device(steps: int, bucket_cfg, step_in, *, step_out=None, cfg_override=None,
                    covered=None, wrap: bool = False, out=None, bucket_cfg_end=None,
                    record_out=None, sigmas=None, region_range=None, covered_sets=None,
                    region_count=None, stream=None):
    """The plan of one step built on the device (and the step advance, and
    the next step's sample records)."""
    d = device_plan(steps, bucket_cfg, step_in, step_out=step_out, cfg_override=cfg_override,
                    covered=covered, wrap=wrap, out=out, bucket_cfg_end=bucket_cfg_end,
                    record_out=record_out, sigmas=sigmas, region_range=region_range,
                    covered_sets=covered_sets, region_count=region_count)
    L.check(L.lib().bcg_plan_device(step_in.numel(), ct.byref(d), _stream(stream)))


def guided_step_dplan(x, x_out, sigmas, mu_uncond, mu_cond, *, steps: int, bucket_cfg, step_in,
                      step_out=None, cfg_override=None, covered=None, wrap: bool = False,
                      plan_out=None, bucket_cfg_end=None, record_in=None, record_out=None,
                      region_range=None, covered_sets=None,
                      sampler: str, s2: float, feather: int = 0,
                      region_count=None, region_box=None, region_strength=None, mu_region=None,
                      x_orig=None, mask=None, cache_hint: int = 0, stats=None, workspace=None,
                      launch_vpt: int = 0, queue=None, stream=None):
    """guided_step with the plan of the step built on the device, same launch.
    ``stats`` ([n, 3]) with ``workspace`` computes the norm statistics inside the step.
    ``queue`` (see device_plan) runs the n samples as slots of continuous batching."""
    a = _step_args(x, x_out, sigmas, mu_uncond, mu_cond, None, n_active=0, sampler=sampler,
                   s2=s2, feather=feather, region_count=region_count, region_box=region_box,
                   region_strength=region_strength, mu_region=mu_region, x_orig=x_orig, mask=mask,
                   stats=stats, workspace=workspace, cache_hint=cache_hint, launch_vpt=launch_vpt,
                   tables=None if not queue else int(queue["len"]))
    if step_in.numel() != x.shape[0]:
        raise ValueError("step_in: needs one entry per sample")
    d = device_plan(steps, bucket_cfg, step_in, step_out=step_out, cfg_override=cfg_override,
                    covered=covered, wrap=wrap, out=plan_out, bucket_cfg_end=bucket_cfg_end,
                    record_in=record_in, record_out=record_out, region_range=region_range,
                    covered_sets=covered_sets, region_count=region_count, queue=queue)
    L.check(L.lib().guided_step_dplan(ct.byref(a), ct.byref(d), _stream(stream)))



def guided_step_dplan_static(x, x_out, sigmas, mu_uncond, mu_cond, *, steps: int, bucket_cfg, step_in,
                             step_out=None, cfg_override=None, covered=None, wrap: bool = False,
                             plan_out=None, bucket_cfg_end=None, record_in=None, record_out=None,
                             region_range=None, covered_sets=None,
                             sampler: str, s2: float, feather: int = 0,
                             region_count=None, region_box=None, region_strength=None, mu_region=None,
                             x_orig=None, mask=None, cache_hint: int = 0, stats=None,
                             launch_vpt: int = 0, stream=None):
    """guided_step_dplan for callers that cannot allocate: the statistics'
    partials go to the library's static scratch (no workspace argument)."""
    a = _step_args(x, x_out, sigmas, mu_uncond, mu_cond, None, n_active=0, sampler=sampler,
                   s2=s2, feather=feather, region_count=region_count, region_box=region_box,
                   region_strength=region_strength, mu_region=mu_region, x_orig=x_orig, mask=mask,
                   stats=stats, workspace=None, cache_hint=cache_hint, launch_vpt=launch_vpt,
                   static_scratch=True)
    if step_in.numel() != x.shape[0]:
        raise ValueError("step_in: needs one entry per sample")
    d = device_plan(steps, bucket_cfg, step_in, step_out=step_out, cfg_override=cfg_override,
                    covered=covered, wrap=wrap, out=plan_out, bucket_cfg_end=bucket_cfg_end,
                    record_in=record_in, record_out=record_out, region_range=region_range,
                    covered_sets=covered_sets, region_count=region_count)
    L.check(L.lib().guided_step_dplan_static(ct.byref(a), ct.byref(d), _stream(stream)))


def latent_init(noise, sigmas, step_idx, x_out, latent=None, stream=None):
    """x_out = latent + noise * sigmas[step_idx[i]] per sample (see include/bcg.h)."""
    _dev(x_out, "x_out")
    if x_out.dim() != 4 or x_out.dtype not in _DT:
        raise ValueError("x_out must be a [n,C,H,W] float32/bfloat16 tensor")
    n, Cc, H, W = x_out.shape
    _dev(noise, "noise", torch.float32, x_out.shape)
    _dev(sigmas, "sigmas", torch.float32)
    _dev(step_idx, "step_idx", torch.int32, (n,))
    _dev(latent, "latent", x_out.dtype, x_out.shape, allow_none=True)
    L.check(L.lib().latent_init(n, Cc, H, W, _DT[x_out.dtype], _ptr(noise), _ptr(latent),
                                _ptr(sigmas), sigmas.numel(), _ptr(step_idx), _ptr(x_out),
                                _stream(stream)))


def area_accumulate(region_pred, region_off, region_count, region_box, region_strength, cond_out,
                    *, feather: int, fallback=None, wsum_out=None, stream=None):
    """Regional accumulation of packed crops into the full latent (include/bcg.h)."""
    _dev(cond_out, "cond_out", torch.float32)
    if cond_out.dim() != 4:
        raise ValueError("cond_out must be [n,C,H,W]")
    n, Cc, H, W = cond_out.shape
    _dev(region_pred, "region_pred", torch.float32)
    _dev(region_count, "region_count", torch.int32, (n,))
    _dev(region_box, "region_box", torch.int32)
    if region_box.dim() != 3 or region_box.shape[0] != n or region_box.shape[2] != 4:
        raise ValueError("region_box must be [n, R, 4]")
    R = region_box.shape[1]
    _dev(region_off, "region_off", torch.int64, (n * R + 1,))
    _dev(region_strength, "region_strength", torch.float32, (n, R))
    _dev(fallback, "fallback", torch.float32, cond_out.shape, allow_none=True)
    _dev(wsum_out, "wsum_out", torch.float32, (n, H, W), allow_none=True)
    L.check(L.lib().area_accumulate(n, Cc, H, W, int(feather), R, _ptr(region_pred),
                                    region_pred.numel(), _ptr(region_off), _ptr(region_count),
                                    _ptr(region_box), _ptr(region_strength), _ptr(fallback),
                                    _ptr(cond_out), _ptr(wsum_out), _stream(stream)))


def mask_blend(a, b, mask, out, stream=None):
    """out = mask*a + (1-mask)*b, mask broadcast over channels (include/bcg.h)."""
    _dev(a, "a")
    if a.dim() != 4 or a.dtype not in _DT:
        raise ValueError("a must be a [n,C,H,W] float32/bfloat16 tensor")
    n, Cc, H, W = a.shape
    _dev(b, "b", a.dtype, a.shape)
    _dev(out, "out", a.dtype, a.shape)
    _dev(mask, "mask", torch.float32)
    if tuple(mask.shape) == (n, 1, H, W):
        mps = 1
    elif tuple(mask.shape) == (1, 1, H, W):
        mps = 0
    else:
        raise ValueError(f"mask: shape {tuple(mask.shape)} is neither [n,1,H,W] nor [1,1,H,W]")
    L.check(L.lib().mask_blend(n, Cc, H, W, _DT[a.dtype], _ptr(a), _ptr(b), _ptr(mask), mps,
                               _ptr(out), _stream(stream)))


# ---------------------------------------------------------------- weight patches

@dataclass
class WeightPatch:
    """One patch of weight_patch: a ``diff`` [rows, cols] (float32 or
    bfloat16), or a low-rank pair ``up`` [rows, r] and ``down`` [r, cols]
    (bfloat16), covering weight rows [offset, offset + rows)."""
    strength_patch: float = 1.0
    strength_model: float = 1.0
    offset: int = 0
    diff: torch.Tensor | None = None
    up: torch.Tensor | None = None
    down: torch.Tensor | None = None


def _patch_struct(p: WeightPatch, cols: int):
    if (p.diff is None) == (p.up is None and p.down is None):
        raise ValueError("a patch is either a diff or a low-rank (up, down) pair")
    if p.diff is not None:
        _dev(p.diff, "diff")
        if p.diff.dim() != 2 or p.diff.shape[1] != cols or p.diff.dtype not in _DT:
            raise ValueError(f"diff must be [rows, {cols}] float32 or bfloat16")
        return L.Patch(L.BCG_PATCH["diff"], int(p.offset), p.diff.shape[0], 0, _DT[p.diff.dtype],
                       float(p.strength_patch), float(p.strength_model), 0, _ptr(p.diff), None, None)
    _dev(p.up, "up", torch.bfloat16)
    _dev(p.down, "down", torch.bfloat16)
    if p.up.dim() != 2 or p.down.dim() != 2 or p.down.shape[1] != cols or p.up.shape[1] != p.down.shape[0]:
        raise ValueError(f"up must be [rows, r] and down [r, {cols}]")
    return L.Patch(L.BCG_PATCH["lowrank"], int(p.offset), p.up.shape[0], p.up.shape[1], L.BCG_BF16,
                   float(p.strength_patch), float(p.strength_model), 0, None, _ptr(p.up), _ptr(p.down))


def weight_patch(w, out, patches=(), *, rounding: str = "stochastic", seed: int = 0, stream=None):
    """out = w with ``patches`` (WeightPatch list) applied in order and stored
    in out's dtype (bfloat16: nearest or stochastic rounding keyed by ``seed``);
    see include/bcg.h.  ``out`` may be ``w`` itself."""
    _dev(w, "w")
    if w.dim() != 2 or w.dtype not in _DT:
        raise ValueError("w must be a [rows, cols] float32 or bfloat16 tensor")
    _dev(out, "out", shape=w.shape)
    if out.dtype not in _DT:
        raise ValueError("out must be float32 or bfloat16")
    if rounding not in L.BCG_ROUND:
        raise ValueError(f"unknown rounding {rounding!r}")
    if len(patches) > L.BCG_MAX_PATCHES:
        raise ValueError(f"at most {L.BCG_MAX_PATCHES} patches per call")
    rows, cols = w.shape
    arr = (L.Patch * max(len(patches), 1))(*[_patch_struct(p, cols) for p in patches])
    a = L.WeightArgs(rows, cols, _DT[w.dtype], _DT[out.dtype], len(patches), L.BCG_ROUND[rounding],
                     int(seed) & (2 ** 64 - 1), _ptr(w), _ptr(out), ct.addressof(arr) if patches else None)
    L.check(L.lib().weight_patch(ct.byref(a), _stream(stream)))
