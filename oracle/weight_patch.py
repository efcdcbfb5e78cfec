"""Weight patches and their rounding: the definition (float64) and the fp32
evaluation order of the kernel.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).  Page cited: "10 ·
ModelPatcher and weight views" (ComfyUI guide, model-patcher chapter),
sections "patches record format" (each entry: strength_patch, the patch
value, strength_model, an optional offset), "how a weight is patched" (all
patches of a key are overlaid in a compute precision, then stochastic
rounding or a cast writes the weight back), "strength_model and
strength_patch" (W' = strength_model*W + strength_patch*dW; dW from a LoRA
low-rank pair, a direct diff, ...) and "offset patch" (a patch acting on a
slice of the tensor only).

Readings (the page names these but does not spell them out):
* patches of one weight apply in order, each W <- sm*W + sp*dW on its slice;
* an offset patch covers rows [offset, offset + rows) of the 2-D weight
  (several modules packed along the output dimension);
* a low-rank pair (up [rows, r], down [r, cols]) is dW = up @ down;
* stochastic rounding of a float32 value to bfloat16: add 16 random bits to
  its bit pattern and keep the high 16 bits (probability of rounding away
  from zero = the dropped fraction, so the rounding is unbiased); the bits
  come from the counter-based generator Philox4x32-10 (Salmon, Moraes, Dror
  and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011) keyed by
  a 64-bit seed: element e uses the 16-bit half (e mod 2) of output word
  ((e mod 8) div 2) of the call whose counter is (e div 8 low, high, 0, 0).

Pins (tests/test_oracle_weight_pins.py): Philox against the published known-answer
vectors; rounding bracketing, exactness and unbiasedness; dW against numpy's
matmul; slices, strengths and order against closed forms.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import definition as D

M0, M1 = 0xD2511F53, 0xCD9E8D57  # Philox4x32 round multipliers
W0, W1 = 0x9E3779B9, 0xBB67AE85  # key schedule (Weyl) increments
MASK = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds on arrays of counters.

    ctr: uint64 array [..., 4] of 32-bit words; key: (k0, k1).  Each round:
    (hi0, lo0) = M0*c0, (hi1, lo1) = M1*c2 (64-bit products),
    c = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key is bumped by
    (W0, W1) between rounds.
    """
    c = np.asarray(ctr, np.uint64) & np.uint64(MASK)
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = np.uint64(key[0] & MASK), np.uint64(key[1] & MASK)
    m0, m1 = np.uint64(M0), np.uint64(M1)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + np.uint64(W0)) & np.uint64(MASK)
            k1 = (k1 + np.uint64(W1)) & np.uint64(MASK)
        p0 = m0 * c0
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1)


def random16(seed: int, idx):
    """The 16 random bits of elements idx (int64 array) under seed."""
    idx = np.asarray(idx, np.int64)
    blk = (idx >> 3).astype(np.uint64)
    ctr = np.stack([blk & np.uint64(MASK), blk >> np.uint64(32),
                    np.zeros_like(blk), np.zeros_like(blk)], axis=-1)
    out = philox4x32_10(ctr, (seed & MASK, (seed >> 32) & MASK))
    word = np.take_along_axis(out, ((idx & 7) >> 1)[..., None].astype(np.int64), axis=-1)[..., 0]
    half = (idx & 1).astype(np.uint64)
    return ((word >> (half * np.uint64(16))) & np.uint64(0xFFFF)).astype(np.uint32)


def sr_bf16(x32, seed: int, base: int = 0):
    """Stochastic rounding of float32 values (flat element indices base + k) to
    bfloat16, returned as float32 values.  Non-finite values keep the
    nearest-even rounding."""
    x32 = np.ascontiguousarray(x32, np.float32)
    bits = x32.view(np.uint32).astype(np.uint64)
    r = random16(seed, base + np.arange(x32.size, dtype=np.int64)).reshape(x32.shape).astype(np.uint64)
    up = ((bits + r) & np.uint64(0xFFFF0000)).astype(np.uint32).view(np.float32)
    return np.where(np.isfinite(x32), up, D.round_bf16(x32).astype(np.float32)).astype(np.float32)


@dataclass
class Patch:
    """One patch entry: dW = diff, or up @ down (low-rank), on rows
    [offset, offset + rows) of the weight; W <- sm*W + sp*dW there."""
    strength_patch: float
    strength_model: float = 1.0
    offset: int = 0
    diff: np.ndarray | None = None   # [rows, cols]
    up: np.ndarray | None = None     # [rows, r]
    down: np.ndarray | None = None   # [r, cols]

    @property
    def rows(self) -> int:
        return (self.diff if self.diff is not None else self.up).shape[0]

    def delta(self):
        if self.diff is not None:
            return np.asarray(self.diff, np.float64)
        return np.asarray(self.up, np.float64) @ np.asarray(self.down, np.float64)


def apply_patches(W, patches):
    """The patched weight in float64 (before rounding): each patch in order,
    W[slice] <- sm*W[slice] + sp*dW."""
    out = np.array(W, np.float64, copy=True)
    for p in patches:
        s = slice(p.offset, p.offset + p.rows)
        out[s] = p.strength_model * out[s] + p.strength_patch * p.delta()
    return out


def apply_patches32(W, patches, deltas32=None):
    """The kernel's float32 order: per element acc = W; for each patch covering
    the row, acc = fma(sp, d, sm*acc).  d is the diff (as float32), or for a
    low-rank patch the float32 product given in ``deltas32`` (its summation
    order is the matrix unit's), else up @ down in float64 rounded once."""
    from .mirror32 import fma32
    acc = np.array(W, np.float32, copy=True)
    for q, p in enumerate(patches):
        s = slice(p.offset, p.offset + p.rows)
        if p.diff is not None:
            d = np.asarray(p.diff, np.float32)
        elif deltas32 is not None and deltas32[q] is not None:
            d = np.asarray(deltas32[q], np.float32)
        else:
            d = p.delta().astype(np.float32)
        acc[s] = fma32(np.float32(p.strength_patch), d, np.float32(p.strength_model) * acc[s])
    return acc


def store(x32, dtype: str, rounding: str = "nearest", seed: int = 0):
    """The written weight: float32 as is, or bfloat16 by nearest-even or
    stochastic rounding (flat element index = position in x32)."""
    x32 = np.asarray(x32, np.float32)
    if dtype == "f32":
        return x32.copy()
    if rounding == "stochastic":
        return sr_bf16(x32, seed)
    return D.round_bf16(x32).astype(np.float32)


# ------------------------------------------------------------ seeded workloads

def held(a, dtype: str):
    """An input as a device array of that storage type holds it (float32)."""
    a = np.asarray(a, np.float32)
    return D.round_bf16(a).astype(np.float32) if dtype == "bf16" else a.copy()


def patches_of(inp):
    """The patches of a ``workloads.weights.WeightInputs`` with their tensors
    rounded to their storage types (low-rank factors are bfloat16) and the
    strengths to float32, as the kernel receives them."""
    out = []
    for pd in inp.patches:
        ps = pd.spec
        sp, sm = float(np.float32(ps.strength_patch)), float(np.float32(ps.strength_model))
        if ps.kind == "diff":
            out.append(Patch(sp, sm, ps.offset, diff=held(pd.diff, ps.dtype)))
        else:
            out.append(Patch(sp, sm, ps.offset, up=held(pd.up, "bf16"), down=held(pd.down, "bf16")))
    return out


def reference(inp):
    """Mode D: the patched weight in float64, before the store."""
    return apply_patches(held(inp.w, inp.spec.w_dtype), patches_of(inp))


def reference32(inp, deltas32=None):
    """Mode M: the float32 value the kernel stores from (its evaluation order)."""
    return apply_patches32(held(inp.w, inp.spec.w_dtype), patches_of(inp), deltas32)


def written(inp, acc32):
    """What the kernel writes for the float32 values ``acc32``."""
    sp = inp.spec
    return store(acc32, sp.out_dtype, sp.rounding, sp.sr_seed)


def delta_error_bound(inp):
    """Per-element bound on |acc32 - reference| for any summation order of the
    low-rank products (each addition rounded to float32): a sum of r terms
    carries at most gamma_r * sum|terms| with gamma_r = r u / (1 - r u),
    u = 2^-24 (Higham, "Accuracy and Stability of Numerical Algorithms",
    section 3.1); each patch then adds the rounding of sm*acc and of the fused
    multiply-add, u |value| each, and scales the earlier error by |sm|."""
    u = 2.0 ** -24
    pats = patches_of(inp)
    acc = np.array(held(inp.w, inp.spec.w_dtype), np.float64)
    err = np.zeros_like(acc)
    for p in pats:
        s = slice(p.offset, p.offset + p.rows)
        if p.diff is not None:
            d_err = np.zeros((p.rows, acc.shape[1]))
        else:
            r = p.up.shape[1]
            g = r * u / (1 - r * u)
            d_err = g * (np.abs(p.up.astype(np.float64)) @ np.abs(p.down.astype(np.float64)))
        prev, e = acc[s], err[s]
        new = p.strength_model * prev + p.strength_patch * p.delta()
        sm, sp = abs(p.strength_model), abs(p.strength_patch)
        # acc32 = prev + e; m = fl(sm*acc32); result = fl(sp*d32 + m)
        err[s] = (sp * d_err + sm * e + u * (1 + u) * sm * (np.abs(prev) + e)
                  + u * (np.abs(new) + sp * d_err + sm * e))
        acc[s] = new
    return err
