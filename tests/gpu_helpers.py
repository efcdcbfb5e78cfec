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
