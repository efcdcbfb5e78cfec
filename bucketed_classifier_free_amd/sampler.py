"""The sampler loop around libbcg.

Per run: sigma schedule and bucket table (host C ABI), constants uploaded
once, latent initialised on the device.  Per step k: the bucket plan is built
on the host (C ABI) straight into a pinned staging row, copied to the device
asynchronously on the compute stream, and one fused ``guided_step`` launch
advances every active sample.  The host never waits on the device inside the
loop (the SGLang BCG write-up, section 4 stage 3: the plan is built by the
scheduler before the launch and is not changed during the step).
"""
from __future__ import annotations

import ctypes as ct

import numpy as np
import torch

from . import _lib as L
from . import api

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


class Interrupted(RuntimeError):
    """Raised between steps when the cancel callback asks to stop."""

    def __init__(self, step, x):
        super().__init__(f"sampling interrupted before step {step}")
        self.step = step
        self.x = x


class GuidedSampler:
    """One batch of samples with per-sample progress and bucketed guidance.

    ``wrap`` (steady-state continuous batching): sample i is at step
    (start_i + k) mod steps at launch k once start_i + k >= 0 (a finished
    slot restarts at step 0); otherwise sample i is active while
    0 <= start_i + k < steps.
    """

    def __init__(self, *, noise, mu_uncond, mu_cond, start_step, steps, num_buckets, curve,
                 sampler="euler", dtype="f32", sigma_max=14.6, sigma_min=0.03, denoise=1.0,
                 s2=0.25, cfg_override=None, region_count=None, region_frac=None,
                 region_strength=None, mu_region=None, feather=0, mask=None, x_orig=None,
                 device="cuda", wrap=False, sigma_start=0, sigma_last=-1,
                 force_full_denoise=False, bucket_interp=False, region_range=None):
        noise = np.ascontiguousarray(noise, np.float32)
        self.n, self.C, self.H, self.W = noise.shape
        self.steps, self.nb, self.sampler, self.dtype = int(steps), int(num_buckets), sampler, dtype
        self.s2, self.feather, self.wrap = float(s2), int(feather), bool(wrap)
        self.device = torch.device(device)
        self.tdtype = _TORCH_DT[dtype]
        self.start = np.ascontiguousarray(start_step, np.int32)
        self.override = None if cfg_override is None else np.ascontiguousarray(cfg_override, np.float32)
        self.sigmas, self.base_steps = api.sigma_schedule(sigma_max, sigma_min, self.steps, denoise)
        if sigma_start or sigma_last >= 0 or force_full_denoise:
            # staged sampling: the cropped sequence is the schedule from here on
            self.sigmas = api.sigma_crop(self.sigmas, sigma_start, sigma_last, force_full_denoise)
            self.steps = self.sigmas.size - 1
            if self.steps < 1:
                raise ValueError("the cropped schedule has no step to run")
        kind, p0, p1, p2 = curve
        if bucket_interp:  # scale interpolated within each bucket: start and end tables
            self.table, self.table_end = api.bucket_bounds(kind, p0, p1, p2, self.nb)
        else:
            self.table, self.table_end = api.bucket_table(kind, p0, p1, p2, self.nb), None
        n, R = self.n, 0
        if region_count is not None and int(np.max(region_count, initial=0)) > 0:
            R = int(np.asarray(region_frac).shape[1])
        self.R = R
        self.region_count = None if R == 0 else np.ascontiguousarray(region_count, np.int32)
        self.region_frac = None if R == 0 else np.ascontiguousarray(region_frac, np.float64)
        self.region_strength = None if R == 0 else np.ascontiguousarray(region_strength, np.float32)
        # per-cond validity ranges of sampling progress (none: always valid)
        self.region_range = (None if R == 0 or region_range is None
                             else np.ascontiguousarray(region_range, np.float64))
        dev = self.device
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
        self.d_sigmas = f32(self.sigmas)
        self.d_mu_u = f32(mu_uncond)
        self.d_mu_c = f32(mu_cond)
        self.d_noise = f32(noise)
        self.d_start = torch.from_numpy(self.start).to(dev)
        self.d_x_orig = None if x_orig is None else f32(x_orig).to(self.tdtype)
        self.d_mask = None if mask is None else f32(mask)
        # Plan staging: row k holds [step_idx | scale bits | uncond_row | order].
        self.h_slab = torch.empty((self.steps, 4 * n), dtype=torch.int32, pin_memory=True)
        self.d_slab = torch.empty((self.steps, 4 * n), dtype=torch.int32, device=dev)
        self._row_ev = [None] * self.steps
        self._tmp = api.plan_out_arrays(n, self.nb, R)
        # Region boxes and coverage do not change between steps: one full plan
        # gives them, later plans reuse the coverage flags.
        self.covered = self.covered_sets = None
        if R > 0:
            p = self._plan(np.zeros(n, np.int32), self._tmp)
            if self.region_range is not None:  # coverage per subset of valid regions
                self.covered_sets = p.covered_sets.copy()
            else:
                self.covered = p.covered.astype(np.uint8)
            self.d_region_box = torch.from_numpy(p.region_box.copy()).to(dev)
            self.d_region_count = torch.from_numpy(self.region_count).to(dev)
            self.d_region_strength = f32(self.region_strength)
            self.d_mu_region = f32(mu_region)
            self.region_box = p.region_box.copy()
            self.region_off = p.region_off.copy()
        else:
            self.d_region_box = self.d_region_count = self.d_region_strength = self.d_mu_region = None
        # Device copies of the plan inputs, for plans built on the device.
        self.d_table = f32(self.table)
        self.d_table_end = None if self.table_end is None else f32(self.table_end)
        self.d_override = None if self.override is None else f32(self.override)
        self.d_covered = (None if self.covered is None else
                          torch.from_numpy(self.covered.astype(np.int32)).to(dev))
        self.d_covered_sets = (None if self.covered_sets is None else
                               torch.from_numpy(self.covered_sets.view(np.int16)).to(dev))
        self.d_region_range = (None if self.region_range is None else
                               torch.from_numpy(self.region_range).to(dev))

    @classmethod
    def from_inputs(cls, inp, **kw):
        """Build from a ``workloads.Inputs``-like object (spec + arrays)."""
        sp = inp.spec
        c = sp.curve
        return cls(noise=inp.noise, mu_uncond=inp.mu_uncond, mu_cond=inp.mu_cond,
                   start_step=inp.start_step, steps=sp.steps, num_buckets=sp.num_buckets,
                   curve=(c.kind, c.p0, c.p1, c.p2), sampler=sp.sampler, dtype=sp.dtype,
                   sigma_max=sp.sigma_max, sigma_min=sp.sigma_min, denoise=sp.denoise, s2=sp.s2,
                   cfg_override=inp.cfg_override,
                   region_count=inp.region_count if sp.regions > 0 else None,
                   region_frac=inp.region_frac, region_strength=inp.region_strength,
                   mu_region=inp.mu_region, feather=sp.feather, mask=inp.mask,
                   x_orig=inp.x_orig, bucket_interp=sp.bucket_interp,
                   region_range=inp.region_range if sp.regions > 0 else None, **kw)

    # ------------------------------------------------------------ host plan

    def _plan(self, t, out):
        cov = getattr(self, "covered", None)
        sets = getattr(self, "covered_sets", None)
        return api.bcg_plan_build(t, self.steps, self.table, C=self.C, H=self.H, W=self.W,
                                  cfg_override=self.override, region_count=self.region_count,
                                  region_frac=self.region_frac,
                                  region_strength=self.region_strength, max_regions=self.R,
                                  covered=cov, out=out, bucket_cfg_end=self.table_end,
                                  region_range=self.region_range, covered_sets=sets)

    def step_indices(self, k: int) -> np.ndarray:
        t = self.start.astype(np.int64) + k
        if self.wrap:
            t = np.where(t >= 0, t % self.steps, t)
        return t.astype(np.int32)

    def plan(self, k: int):
        """The host plan of launch k (fresh arrays, for inspection)."""
        return self._plan(self.step_indices(k), None)

    # ------------------------------------------------------------ device

    def alloc_state(self):
        return torch.empty((self.n, self.C, self.H, self.W), dtype=self.tdtype, device=self.device)

    def init_state(self, x=None):
        """x = latent + noise * sigma[start] (the original latent when inpainting)."""
        x = self.alloc_state() if x is None else x
        api.latent_init(self.d_noise, self.d_sigmas, self.d_start, x, latent=self.d_x_orig)
        return x

    def upload_plan(self, k: int):
        """Build the plan of launch k into its staging row and queue its upload."""
        n = self.n
        row = k % self.steps
        ev = self._row_ev[row]
        if ev is not None:
            ev.synchronize()  # the previous upload from this row has finished
        h = self.h_slab[row].numpy()
        h[:n] = self.step_indices(k)
        o = self._tmp
        o["scale"] = h[n:2 * n].view(np.float32)
        o["uncond_row"] = h[2 * n:3 * n]
        o["order"] = h[3 * n:4 * n]
        p = self._plan(h[:n], o)
        d = self.d_slab[row]
        d.copy_(self.h_slab[row], non_blocking=True)
        if self._row_ev[row] is None:
            self._row_ev[row] = torch.cuda.Event()
        self._row_ev[row].record()
        return p, d

    def launch(self, d, n_active, x, x_out=None, stats=None, workspace=None, cache_hint=0,
               launch_vpt=0):
        n = self.n
        api.guided_step(x, x if x_out is None else x_out, self.d_sigmas, d[3 * n:4 * n], d[:n],
                        d[n:2 * n].view(torch.float32), d[2 * n:3 * n], self.d_mu_u, self.d_mu_c,
                        n_active=n_active, sampler=self.sampler, s2=self.s2,
                        feather=self.feather, region_count=self.d_region_count,
                        region_box=self.d_region_box, region_strength=self.d_region_strength,
                        mu_region=self.d_mu_region, x_orig=self.d_x_orig, mask=self.d_mask,
                        stats=stats, workspace=workspace, cache_hint=cache_hint,
                        region_range=self.d_region_range, steps=self.steps, launch_vpt=launch_vpt)

    def step(self, k: int, x, x_out=None, stats=None, workspace=None, cache_hint=0, launch_vpt=0):
        """Launch k of the loop: plan, upload, one fused guided step."""
        p, d = self.upload_plan(k)
        self.launch(d, p.n_active, x, x_out, stats, workspace, cache_hint, launch_vpt)
        return p

    def records(self, k: int):
        """Sample records of launch k's step indices (host float32 [n, 4])."""
        return api.plan_records(self.plan(k), self.step_indices(k), self.steps, self.sigmas,
                                ranged=self.region_range is not None)

    def dplan_step(self, x, step_in, step_out=None, x_out=None, plan_out=None, cache_hint=0,
                   record_in=None, record_out=None, stats=None, workspace=None, launch_vpt=0):
        """One fused step whose plan is built on the device from ``step_in``
        (device int32 [n]); ``step_out`` receives the next step indices.
        ``record_in`` / ``record_out`` (device float32 [n, 4]) carry the
        sample records of this and the next step's indices."""
        api.guided_step_dplan(x, x if x_out is None else x_out, self.d_sigmas, self.d_mu_u,
                              self.d_mu_c, steps=self.steps, bucket_cfg=self.d_table,
                              step_in=step_in, step_out=step_out, cfg_override=self.d_override,
                              covered=self.d_covered, wrap=self.wrap, plan_out=plan_out,
                              bucket_cfg_end=self.d_table_end, record_in=record_in,
                              record_out=record_out, region_range=self.d_region_range,
                              covered_sets=self.d_covered_sets,
                              sampler=self.sampler, s2=self.s2, feather=self.feather,
                              region_count=self.d_region_count, region_box=self.d_region_box,
                              region_strength=self.d_region_strength, mu_region=self.d_mu_region,
                              x_orig=self.d_x_orig, mask=self.d_mask, cache_hint=cache_hint,
                              stats=stats, workspace=workspace, launch_vpt=launch_vpt)

    def run(self, x=None, launches=None, callback=None, cancel=None):
        """Whole loop from the initial latent; returns the final state.

        ``callback(k, x)`` runs after launch k; ``cancel()`` is checked before
        each launch and raises Interrupted (the state so far is resumable).
        """
        x = self.init_state() if x is None else x
        L = self.steps if launches is None else launches
        for k in range(L):
            if cancel is not None and cancel():
                raise Interrupted(k, x)
            self.step(k, x)
            if callback is not None:
                callback(k, x)
        return x

    # ------------------------------------------------------------ native loop

    def native_loop(self, x, x_out=None, upload_batch=8, async_upload=False, cache_hint=None,
                    device_plan=False, graph_launches=0, plan_outputs=True, records=True,
                    slots=None, ring=False, join_front=None):
        """A C++ loop (bcg_loop_*) advancing ``x`` (in place unless x_out).

        ``x`` may also be [replicas, n, C, H, W]: launch k then advances
        replica k mod replicas by one step of its own trajectory
        (independent batches served round-robin).  ``device_plan`` builds
        each step's plan on the device inside the step's launch (into
        ``loop.plan_out`` when ``plan_outputs``); ``graph_launches`` > 0
        replays a captured graph of that many launches.  ``slots`` (device
        plans) runs continuous batching: x holds that many slots, this
        sampler's samples are the queue of requests (the first ``slots``
        start in the slots at their start steps, the rest wait), and a freed
        slot takes the next request; ``ring`` serves the queue over and over;
        ``join_front`` joins a step are dispatched first (default: twice the
        mean refills per step plus 8, at most ``slots``)."""
        return NativeLoop(self, x, x_out, upload_batch, async_upload, cache_hint,
                          device_plan, graph_launches, plan_outputs, records, slots, ring, join_front)


class NativeLoop:
    """Owner of a bcg_loop handle and of the host/device arrays it points to."""

    def __init__(self, s: GuidedSampler, x, x_out=None, upload_batch=8, async_upload=False,
                 cache_hint=None, device_plan=False, graph_launches=0,
                 plan_outputs=True, records=True, slots=None, ring=False, join_front=None):
        queue = slots is not None
        if queue and not (device_plan and records and 1 <= int(slots) <= s.n):
            raise ValueError("continuous batching needs device plans with records and 1 <= slots <= n")
        n = int(slots) if queue else s.n
        J = 0
        if queue:
            J = min(n, 2 * (-(-n // s.steps)) + 8) if join_front is None else int(join_front)
        P = int(upload_batch)
        rows = 8 * P
        self.s = s
        self.x, self.x_out = x, (x if x_out is None else x_out)
        reps = x.shape[0] if x.dim() == 5 else 1
        shape = (reps, n, s.C, s.H, s.W) if x.dim() == 5 else (n, s.C, s.H, s.W)
        api._dev(x, "x", s.tdtype, shape)
        api._dev(self.x_out, "x_out", s.tdtype, shape)
        stride = n * s.C * s.H * s.W * x.element_size()
        if cache_hint is None:  # several batches in rotation: stream them past the caches
            cache_hint = L.BCG_CACHE_STREAM if reps > 1 else L.BCG_CACHE_KEEP
        if device_plan:
            self.h_slab = self.d_slab = None
            self.dev_steps = torch.empty((reps, 2, n), dtype=torch.int32, device=s.device)
            self.dev_records = (torch.zeros((reps, 2, n, 4), dtype=torch.float32, device=s.device)
                                if records else None)
            self.dev_queue = (torch.zeros((reps, 2, n + 1 + J), dtype=torch.int32, device=s.device)
                              if queue else None)
            self.plan_out = api.device_plan_arrays(n, s.nb, s.device) if plan_outputs else None
            qd = None
            if queue:
                qd = dict(len=s.n, ring=ring, noise=s.d_noise, slot_req_in=self.dev_queue[0, 0, :n],
                          slot_req_out=self.dev_queue[0, 1, :n], queue_in=self.dev_queue[0, 0, n:n + 1],
                          queue_out=self.dev_queue[0, 1, n:n + 1], join_front=J,
                          join_in=self.dev_queue[0, 0, n + 1:], join_out=self.dev_queue[0, 1, n + 1:])
            dplan = api.device_plan(s.steps, s.d_table, self.dev_steps[0, 0],
                                    step_out=self.dev_steps[0, 1], cfg_override=s.d_override,
                                    covered=s.d_covered, wrap=s.wrap, out=self.plan_out,
                                    bucket_cfg_end=s.d_table_end, sigmas=s.d_sigmas,
                                    region_range=s.d_region_range, covered_sets=s.d_covered_sets,
                                    region_count=s.d_region_count, queue=qd)
        else:
            self.h_slab = torch.empty((rows, 4 * n), dtype=torch.int32, pin_memory=True)
            self.d_slab = torch.empty((rows, 4 * n), dtype=torch.int32, device=s.device)
            self.dev_steps = self.dev_records = self.plan_out = self.dev_queue = None
            dplan = L.DevicePlan()
        keep = self._keep = []

        def npp(a, dt):
            if a is None:
                return None
            a = np.ascontiguousarray(a, dt)
            keep.append(a)
            return a.ctypes.data

        R = s.R
        plan = L.PlanIn(n, s.steps, s.nb, s.C, s.H, s.W, R, npp(s.table, np.float32), None,
                        npp(s.override, np.float32), npp(s.region_count, np.int32),
                        npp(s.region_frac, np.float64), npp(s.region_strength, np.float32),
                        npp(s.covered, np.uint8), npp(s.table_end, np.float32),
                        npp(s.region_range, np.float64), npp(s.covered_sets, np.uint16))
        ptr = api._ptr
        step = L.StepArgs(n, s.C, s.H, s.W, api._DT[s.tdtype], api._SAMPLER[s.sampler], R,
                          s.feather, 0, s.d_sigmas.numel(),
                          1 if s.d_mask is not None and s.d_mask.shape[0] == s.n else 0,
                          int(cache_hint), s.s2,
                          ptr(self.x), ptr(self.x_out), ptr(s.d_sigmas), None, None, None, None,
                          ptr(s.d_mu_u), ptr(s.d_mu_c), ptr(s.d_region_count),
                          ptr(s.d_region_box), ptr(s.d_region_strength), ptr(s.d_mu_region),
                          ptr(s.d_x_orig), ptr(s.d_mask), None, None, 0, ptr(s.d_region_range),
                          s.steps)
        self.desc = L.LoopDesc(plan, npp(s.start[:n], np.int32), 1 if s.wrap else 0, rows,
                               api._ptr(self.h_slab), api._ptr(self.d_slab), reps,
                               stride if reps > 1 else 0, P, 1 if async_upload else 0,
                               step, 1 if device_plan else 0,
                               int(graph_launches), api._ptr(self.dev_steps), dplan,
                               api._ptr(self.dev_records), s.n if queue else 0, 1 if ring else 0,
                               api._ptr(s.d_noise) if queue else None, api._ptr(self.dev_queue), J)
        self.handle = ct.c_void_p()
        L.check(L.lib().bcg_loop_create(ct.byref(self.desc), ct.byref(self.handle)))

    def run(self, k0: int, count: int, timing: bool = False):
        """Launches k0 .. k0+count-1 on the current stream; with ``timing`` the
        mean time per launch (ms) between one pair of HIP events around the
        whole run is returned."""
        ms = ct.c_float(0.0)
        L.check(L.lib().bcg_loop_run(self.handle, int(k0), int(count),
                                     torch.cuda.current_stream().cuda_stream,
                                     ct.byref(ms) if timing else None))
        return ms.value if timing else None

    def last_run(self):
        """(launches inside graph replays, launches launched directly) of the
        last run."""
        rep, dire = ct.c_int32(0), ct.c_int32(0)
        L.check(L.lib().bcg_loop_last_run(self.handle, ct.byref(rep), ct.byref(dire)))
        return rep.value, dire.value

    def close(self):
        if self.handle:
            L.lib().bcg_loop_destroy(self.handle)
            self.handle = ct.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
