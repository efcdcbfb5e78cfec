"""Pins of the weight-patch oracle (oracle/weight_patch.py) to facts fixed
outside itself: the published known-answer vectors of Philox4x32-10, the
defining properties of stochastic rounding (bracketing, exactness,
unbiasedness), closed forms of the patch composition, brute force for the
low-rank product and the error bound of the float32 evaluation order."""
import os

import numpy as np
import pytest
import torch

from oracle import weight_patch as P
from workloads import weights as WW

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- Philox

def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(v, 16) for v in line.split()])
    return rows


def test_philox_known_answer_vectors():
    kat = _kat()
    assert len(kat) == 3
    for r in kat:
        got = P.philox4x32_10(np.array([r[:4]], np.uint64), (r[4], r[5]))[0]
        assert [int(v) for v in got] == r[6:], [hex(int(v)) for v in got]


def test_random_bits_uniform_and_keyed():
    e = np.arange(1 << 18, dtype=np.int64)
    r = P.random16(0x1234_5678_9ABC, e)
    assert r.max() < 65536
    # chi-square over the top byte, and per position in the 8-element block
    for sel in [slice(None)] + [slice(k, None, 8) for k in range(8)]:
        h = np.bincount((r[sel] >> 8).astype(np.int64), minlength=256)
        exp = h.sum() / 256
        chi2 = ((h - exp) ** 2 / exp).sum()
        assert chi2 < 255 + 6 * np.sqrt(2 * 255), chi2
    # the key and both counter words matter
    assert not np.array_equal(r[:4096], P.random16(0x1234_5678_9ABD, e[:4096]))
    assert not np.array_equal(r[:4096], P.random16(0x1234_5678_9ABC | (1 << 40), e[:4096]))
    hi = e[:4096] + (np.int64(1) << 35)  # counter word 1 = 1
    assert not np.array_equal(r[:4096], P.random16(0x1234_5678_9ABC, hi))


# ---------------------------------------------------------------- stochastic rounding

def _bracket(x):
    """The bfloat16 neighbours lo <= x <= hi, from torch's nearest rounding and
    nextafter on bfloat16."""
    t = torch.from_numpy(x)
    a = t.to(torch.bfloat16)
    up = torch.nextafter(a, torch.full_like(a, float("inf")))
    dn = torch.nextafter(a, torch.full_like(a, -float("inf")))
    af = a.float()
    lo = torch.where(af <= t, af, dn.float())
    hi = torch.where(af <= t, up.float(), af)
    hi = torch.where(af == t, af, hi)
    return lo.numpy(), hi.numpy()


def test_sr_brackets_and_keeps_representable_values():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, 100000))).astype(np.float32)
    rep = torch.from_numpy(x[:5000]).to(torch.bfloat16).float().numpy()
    x = np.concatenate([x, rep, np.float32([0.0, -0.0, 1.0, -3.5])])
    got = P.sr_bf16(x, seed=99)
    lo, hi = _bracket(x)
    assert np.all((got == lo) | (got == hi))
    exact = lo == hi
    assert exact.sum() >= 5004 and np.array_equal(got[exact], x[exact])
    # every result is a bfloat16 value
    assert np.all((got.view(np.uint32) & 0xFFFF) == 0)


def test_sr_is_unbiased():
    """P(round away from zero) = dropped fraction; so E[sr(x)] = x."""
    for v in [1.0 + 2 ** -9, -3.0 - 0.3 * 2 ** -6, 0.1, 1234.567]:
        x = np.full(1 << 17, v, np.float32)
        got = P.sr_bf16(x, seed=7).astype(np.float64)
        lo, hi = _bracket(x[:1])
        p = (float(x[0]) - lo[0]) / (hi[0] - lo[0])
        frac_hi = np.mean(got == hi[0])
        assert abs(frac_hi - p) < 5 * np.sqrt(p * (1 - p) / x.size) + 2 ** -16, (v, frac_hi, p)
        assert abs(got.mean() - float(x[0])) < 5 * (hi[0] - lo[0]) / np.sqrt(x.size)


def test_sr_non_finite_values_round_to_nearest():
    x = np.float32([np.nan, np.inf, -np.inf])
    got = P.sr_bf16(x, seed=1)
    assert np.isnan(got[0]) and got[1] == np.inf and got[2] == -np.inf


def test_sr_element_index_sets_the_bits():
    """Element e of a batch at base b draws the same bits as element b + e of
    a batch at base 0 (the rounding of an element depends on its flat index
    only, not on how the weight is cut into pieces)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal(4096).astype(np.float32)
    whole = P.sr_bf16(x, seed=11)
    for base in (0, 1, 7, 8, 1000):
        assert np.array_equal(P.sr_bf16(x[base:], seed=11, base=base), whole[base:])


# ---------------------------------------------------------------- patch composition

def _w(rows=11, cols=13, seed=0):
    return np.random.default_rng(seed).standard_normal((rows, cols))


def test_single_patch_special_cases():
    W = _w()
    d = _w(seed=1)
    assert np.array_equal(P.apply_patches(W, [P.Patch(0.0, 1.0, diff=d)]), W)
    assert np.array_equal(P.apply_patches(W, [P.Patch(1.0, 0.0, diff=d)]), d)
    assert np.array_equal(P.apply_patches(W, [P.Patch(0.0, 0.0, diff=d)]), np.zeros_like(W))
    assert np.allclose(P.apply_patches(W, [P.Patch(1.0, 1.0, diff=-W)]), 0.0)
    # W' = sm W + sp dW at two strengths is affine in each
    a = P.apply_patches(W, [P.Patch(0.3, 2.0, diff=d)])
    assert np.allclose(a, 2.0 * W + 0.3 * d)


def test_patches_apply_in_order():
    W, d1, d2 = _w(), _w(seed=1), _w(seed=2)
    p1, p2 = P.Patch(1.0, 0.5, diff=d1), P.Patch(1.0, 2.0, diff=d2)
    # 2 (0.5 W + d1) + d2 = W + 2 d1 + d2; the other order gives 0.5 (2 W + d2) + d1
    assert np.allclose(P.apply_patches(W, [p1, p2]), W + 2 * d1 + d2)
    assert np.allclose(P.apply_patches(W, [p2, p1]), W + d1 + 0.5 * d2)


def test_offset_patch_touches_its_rows_only():
    W = _w(rows=20)
    d = _w(rows=6, seed=1)
    out = P.apply_patches(W, [P.Patch(1.0, 3.0, offset=9, diff=d)])
    assert np.array_equal(out[:9], W[:9]) and np.array_equal(out[15:], W[15:])
    assert np.allclose(out[9:15], 3.0 * W[9:15] + d)


def test_lowrank_delta_is_up_times_down_brute_force():
    rng = np.random.default_rng(4)
    up, down = rng.standard_normal((5, 3)), rng.standard_normal((3, 7))
    want = np.zeros((5, 7))
    for i in range(5):
        for j in range(7):
            for k in range(3):
                want[i, j] += up[i, k] * down[k, j]
    got = P.Patch(1.0, up=up, down=down).delta()
    assert got.shape == (5, 7) and np.allclose(got, want, rtol=1e-14, atol=0)
    out = P.apply_patches(np.zeros((9, 7)), [P.Patch(0.5, offset=2, up=up, down=down)])
    assert np.allclose(out[2:7], 0.5 * want) and not out[:2].any() and not out[7:].any()


# ---------------------------------------------------------------- float32 order and workloads

def _spec(**kw):
    base = dict(name="t", rows=70, cols=136, w_dtype="bf16", out_dtype="bf16",
                patches=(WW.PatchSpec("lowrank", rank=24, strength_patch=0.7),
                         WW.PatchSpec("diff", offset=5, rows=40, strength_patch=1.3, strength_model=0.9),
                         WW.PatchSpec("lowrank", offset=33, rows=37, rank=8, strength_patch=-0.4,
                                      strength_model=1.1)),
                seed=3, sr_seed=77)
    base.update(kw)
    return WW.WeightSpec(**base)


def test_workload_draws_are_reproducible_and_shaped():
    a, b = WW.make_weight_inputs(_spec()), WW.make_weight_inputs(_spec())
    assert np.array_equal(a.w, b.w) and a.w.shape == (70, 136)
    assert [p.rows for p in a.patches] == [70, 40, 37]
    assert a.patches[0].up.shape == (70, 24) and a.patches[0].down.shape == (24, 136)
    assert a.patches[1].diff.shape == (40, 136)
    d = WW.make_weight_inputs(_spec(dyadic=True))
    k = d.patches[0].up * 64
    assert np.array_equal(k, np.round(k)) and np.abs(k).max() <= 8


@pytest.mark.parametrize("dyadic", [False, True])
def test_float32_order_within_derived_bound(dyadic):
    inp = WW.make_weight_inputs(_spec(dyadic=dyadic, w_dtype="f32"))
    ref = P.reference(inp)
    bound = P.delta_error_bound(inp)
    pats = P.patches_of(inp)
    # the low-rank products summed in three different float32 orders
    orders = [None,
              [None if p.diff is not None else (p.up.astype(np.float32) @ p.down.astype(np.float32))
               for p in pats],
              [None if p.diff is not None else
               (p.up.astype(np.float32)[:, ::-1, None] * p.down.astype(np.float32)[None, ::-1, :]
                ).cumsum(axis=1, dtype=np.float32)[:, -1, :]
               for p in pats]]
    for dl in orders:
        got = P.reference32(inp, dl).astype(np.float64)
        assert np.all(np.abs(got - ref) <= bound)
    if dyadic:  # every low-rank delta is exact in float32
        for p in pats:
            if p.diff is None:
                assert np.array_equal((p.up.astype(np.float32) @ p.down.astype(np.float32)).astype(np.float64),
                                      p.delta())


def test_bound_is_not_vacuous():
    """The bound is a few float32 ulps of the result, not a blanket tolerance."""
    inp = WW.make_weight_inputs(_spec(w_dtype="f32"))
    ref = P.reference(inp)
    assert np.median(P.delta_error_bound(inp) / np.maximum(np.abs(ref), 1e-30)) < 2e-6


def test_written_bf16_nearest_and_stochastic():
    inp = WW.make_weight_inputs(_spec())
    acc = P.reference32(inp)
    sr = P.written(inp, acc)
    lo, hi = _bracket(acc)
    assert np.all((sr == lo) | (sr == hi))
    nr = P.written(WW.make_weight_inputs(_spec(rounding="nearest")), acc)
    assert np.array_equal(nr, torch.from_numpy(acc).to(torch.bfloat16).float().numpy())
    f32 = P.written(WW.make_weight_inputs(_spec(out_dtype="f32")), acc)
    assert np.array_equal(f32, acc)
