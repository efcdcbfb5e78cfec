"""Shared helpers of the GPU tests: run the HIP path on seeded inputs and
bring results back as numpy float32 (the oracle sees only numpy arrays)."""
import numpy as np
import torch

from oracle import definition as D
from oracle import mirror32 as M

TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(TDT[dtype])


def to_np(t):
    return t.detach().float().cpu().numpy()


def gpu_step_from(sampler, k, x_in_np):
    """GPU output of launch k (out of place) from a given state."""
    x = to_dev(x_in_np, sampler.dtype)
    out = torch.full_like(x, float("nan"))
    sampler.step(k, x, out)
    torch.cuda.synchronize()
    return to_np(out), sampler.plan(k)


def gpu_trajectory(sampler, launches=None, keep_samples=None):
    """Full GPU loop; returns the final state and (optionally) per-launch states."""
    states = []
    cb = None
    if keep_samples is not None:
        def cb(k, x):
            states.append(to_np(x[keep_samples]))
    x = sampler.run(callback=cb, launches=launches)
    torch.cuda.synchronize()
    return to_np(x), states


def per_sample_rel_err(got, ref, idx):
    """max |got - ref| / max |ref| per sample in idx."""
    out = []
    for i in idx:
        d = np.abs(got[i].astype(np.float64) - ref[i]).max()
        out.append(d / max(np.abs(ref[i]).max(), 1e-30))
    return np.array(out)


def bf16_ulp(v):
    v = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(v, 1e-30)))
    return np.exp2(e - 7)


def oracle_step_D(inp, sig, plan, k, x_in, idx):
    """Mode D outputs (float64) of launch k for samples idx from state x_in."""
    t = inp.start_step.astype(np.int64) + k
    out = {}
    for i in idx:
        if plan["bucket_id"][i] < 0:
            continue
        ti = int(t[i])
        out[i] = D.step(x_in[i].astype(np.float64), float(sig[ti]), float(sig[ti + 1]),
                        float(plan["scale"][i]), D.sample_params(inp, i), inp.spec.sampler)
    return out


def oracle_step_M(inp, sig, plan, k, x_in, idx):
    """Mode M outputs (stored) of launch k for samples idx from state x_in."""
    t = inp.start_step.astype(np.int64) + k
    out = {}
    for i in idx:
        if plan["bucket_id"][i] < 0:
            continue
        ti = int(t[i])
        y = M.step32(x_in[i].astype(np.float32), sig[ti], sig[ti + 1], plan["scale"][i],
                     bool(plan["need_uncond"][i]), M.params32(inp, i), inp.spec.sampler)
        out[i] = M._store(y, inp.spec.dtype)
    return out


def storage_flip_bound(inp, i, launches=None):
    """Per-element bound on |x_M - x_D| for sample i after the trajectory,
    when both store every state in bf16 and the fp32 arithmetic is otherwise
    within 1e-5 of exact.

    Both sides round to bf16 after every step.  Where the exact step value
    lies close to a rounding midpoint the two sides can take neighbouring
    codes (a flip of one ulp of the state), and a flip made while |x| is large
    is carried to the end by the later steps.  With the linear stand-in the
    guided prediction is P(x) = A x + B per element, A = m s2/(s2 + sigma^2)
    (m the inpaint mask, 1 without one; the regional weights sum to one and
    the CFG combine keeps A), so one step maps a difference Delta to
    J Delta with
      Euler  J = 1 + (sigma'-sigma)/sigma (1 - A),
      Heun   J = 1 + h/2 [(1-A)/sigma + (1-A2)/sigma' (1 + h (1-A)/sigma)],
      last step (sigma' = 0) J = A,
    and the stored difference after a step is at most |J| Delta plus one
    ulp of the stored value (each side rounds to within half an ulp), plus
    the fp32 slack.  Starting from one ulp of the initial latent, the bound
    is the recurrence Delta_k = |J_k| Delta_{k-1} + ulp(X_k + |J_k| Delta_{k-1})
    + 2e-6 max|X_k| over the launches where the sample is active, X_k the
    mode D state."""
    sub = inp.subset([i])
    sp = sub.spec
    sig, _, _ = D.run_setup(sub)
    sig = sig.astype(np.float64)
    _, states = D.trajectory(sub, launches=launches, keep=True)
    m = 1.0 if sub.mask is None else sub.mask[0, 0].astype(np.float64)
    s2 = float(sp.s2)
    bound = bf16_ulp(states[0][0])
    for k in range(1, len(states)):
        t = int(sub.start_step[0]) + k - 1
        if not 0 <= t < sp.steps:
            continue
        s0, s1 = sig[t], sig[t + 1]
        A = m * s2 / (s2 + s0 * s0)
        if s1 == 0.0:
            J = A
        elif sp.sampler == "euler":
            J = 1.0 + (s1 - s0) / s0 * (1.0 - A)
        else:
            A2 = m * s2 / (s2 + s1 * s1)
            h = s1 - s0
            J = 1.0 + 0.5 * h * ((1.0 - A) / s0 + (1.0 - A2) / s1 * (1.0 + h * (1.0 - A) / s0))
        X = np.abs(states[k][0])
        carried = np.abs(J) * bound
        bound = carried + bf16_ulp(X + carried) + 2e-6 * X.max()
    return bound
