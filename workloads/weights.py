"""Seeded synthetic inputs for the weight-patch workload.

Random numbers only: no patch arithmetic, no rounding to a storage type (each
side rounds the float32 draws to bfloat16 itself where a tensor is stored in
it).  The model-patcher page of the ComfyUI guide ("10 · ModelPatcher and
weight views") motivates the shapes: one checkpoint with three LoRA sets
stacked on it (its opening example), each set contributing one low-rank patch
per weight, and fused weights that pack several logical modules along the
output dimension, patched slice by slice ("offset patch").  The large shapes
are transformer linear weights of hidden size 3072: a 4x MLP projection
[12288, 3072] and a fused q/k/v projection [9216, 3072].

Draw order per spec (fixed, so a seed reproduces every array): the weight,
then for each patch in order its diff, or its up and then its down factor.
Every draw is float64 from numpy's PCG64 ``default_rng(seed)``, rounded to
float32 once.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["PatchSpec", "WeightSpec", "PatchData", "WeightInputs", "WEIGHT_CONFIGS",
           "weight_config", "make_weight_inputs"]


@dataclass(frozen=True)
class PatchSpec:
    kind: str                    # "diff" or "lowrank"
    offset: int = 0              # first weight row covered
    rows: int | None = None      # rows covered (None: every row from offset on)
    rank: int = 0                # low-rank r
    strength_patch: float = 1.0
    strength_model: float = 1.0
    dtype: str = "bf16"          # storage of the patch tensors ("f32" or "bf16"; low-rank: bf16)


@dataclass(frozen=True)
class WeightSpec:
    name: str
    rows: int
    cols: int
    w_dtype: str = "bf16"
    out_dtype: str = "bf16"
    patches: tuple = ()
    rounding: str = "stochastic"  # "nearest" or "stochastic" (bf16 output)
    sr_seed: int = 0              # key of the rounding generator
    seed: int = 0                 # seed of the draws
    dyadic: bool = False          # low-rank factors on the grid k/64, |k| <= 8
    w_std: float = 0.02


@dataclass
class PatchData:
    spec: PatchSpec
    rows: int
    diff: np.ndarray | None      # f32 [rows, cols]
    up: np.ndarray | None        # f32 [rows, rank]
    down: np.ndarray | None      # f32 [rank, cols]


@dataclass
class WeightInputs:
    spec: WeightSpec
    w: np.ndarray                # f32 [rows, cols]
    patches: list


def _f32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def make_weight_inputs(spec: WeightSpec) -> WeightInputs:
    """Draw the weight and every patch tensor of ``spec``.

    Weight ~ N(0, w_std); a diff ~ N(0, w_std / 10); low-rank factors
    up ~ N(0, 0.01), down ~ N(0, 0.05), or, with ``dyadic``, integers in
    [-8, 8] divided by 64 (every product and every partial sum of up @ down
    is then a float32 number, whatever the summation order).
    """
    rng = np.random.default_rng(spec.seed)
    w = _f32(rng.standard_normal((spec.rows, spec.cols)) * spec.w_std)
    out = []
    for p in spec.patches:
        rows = spec.rows - p.offset if p.rows is None else p.rows
        diff = up = down = None
        if p.kind == "diff":
            diff = _f32(rng.standard_normal((rows, spec.cols)) * (spec.w_std / 10))
        elif spec.dyadic:
            up = _f32(rng.integers(-8, 9, size=(rows, p.rank)) / 64.0)
            down = _f32(rng.integers(-8, 9, size=(p.rank, spec.cols)) / 64.0)
        else:
            up = _f32(rng.standard_normal((rows, p.rank)) * 0.01)
            down = _f32(rng.standard_normal((p.rank, spec.cols)) * 0.05)
        out.append(PatchData(p, rows, diff, up, down))
    return WeightInputs(spec, w, out)


def _wcfgs():
    three_lora = (PatchSpec("lowrank", rank=16, strength_patch=1.0),
                  PatchSpec("lowrank", rank=32, strength_patch=0.8),
                  PatchSpec("lowrank", rank=64, strength_patch=0.6))
    qkv = tuple(PatchSpec("lowrank", offset=o, rows=3072, rank=32, strength_patch=0.8)
                for o in (0, 3072, 6144))
    return {
        # three LoRA sets stacked on an MLP projection weight
        "mlp_three_lora_bf16": WeightSpec("mlp_three_lora_bf16", 12288, 3072, patches=three_lora,
                                          sr_seed=0x5EED0001, seed=20261211),
        # one LoRA set on a fused q/k/v weight: one offset patch per packed module
        "qkv_offset_lora_bf16": WeightSpec("qkv_offset_lora_bf16", 9216, 3072, patches=qkv,
                                           sr_seed=0x5EED0002, seed=20261212),
        # a full-weight difference (a merged fine-tune) with a model strength
        "mlp_diff_bf16": WeightSpec("mlp_diff_bf16", 12288, 3072,
                                    patches=(PatchSpec("diff", strength_patch=1.0,
                                                       strength_model=0.9),),
                                    sr_seed=0x5EED0003, seed=20261213),
    }


WEIGHT_CONFIGS = _wcfgs()


def weight_config(name: str) -> WeightSpec:
    return WEIGHT_CONFIGS[name]
