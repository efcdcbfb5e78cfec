"""weight_patch on the GPU against the weight-patch oracle.

Bit for bit where the float32 result is fixed independently of the matrix
unit's summation order: diff patches, and low-rank factors on the dyadic grid
(every product and partial sum of up @ down is then a float32 number), across
weight/output dtypes, nearest and stochastic rounding (the Philox bits
included), row offsets, ragged tiles, ranks that are not multiples of the
16-wide k-step or the 32-row staging chunk, and the element path (cols not a
multiple of 8).  With random low-rank factors: inside the error bound derived
from the float32 evaluation order (oracle ``delta_error_bound``), and for
bfloat16 outputs within the two neighbours that bound allows.  The large
workload shapes are checked on sampled rows.
"""
import numpy as np
import pytest
import torch

from oracle import definition as D
from oracle import weight_patch as P
from workloads import weights as WW

pytestmark = pytest.mark.gpu

TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bucketed_classifier_free_amd
    bucketed_classifier_free_amd.load()  # fails loudly without libbcg.so


def _dev_patches(inp):
    from bucketed_classifier_free_amd import WeightPatch
    out = []
    for pd in inp.patches:
        ps = pd.spec
        if ps.kind == "diff":
            out.append(WeightPatch(ps.strength_patch, ps.strength_model, ps.offset,
                                   diff=torch.from_numpy(pd.diff).cuda().to(TDT[ps.dtype])))
        else:
            out.append(WeightPatch(ps.strength_patch, ps.strength_model, ps.offset,
                                   up=torch.from_numpy(pd.up).cuda().to(torch.bfloat16),
                                   down=torch.from_numpy(pd.down).cuda().to(torch.bfloat16)))
    return out


def _run(inp, in_place=False, seed=None):
    from bucketed_classifier_free_amd import weight_patch
    sp = inp.spec
    w = torch.from_numpy(inp.w).cuda().to(TDT[sp.w_dtype])
    out = w if in_place else torch.full(w.shape, float("nan"), dtype=TDT[sp.out_dtype], device="cuda")
    weight_patch(w, out, _dev_patches(inp), rounding=sp.rounding,
                 seed=sp.sr_seed if seed is None else seed)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _rd_ru(x):
    """The bfloat16 values nearest below and above float64 values x
    (rounding towards -inf and towards +inf)."""
    x = np.asarray(x, np.float64)
    a = torch.from_numpy(D.round_bf16(x).astype(np.float32)).to(torch.bfloat16)  # exact
    up = torch.nextafter(a, torch.full_like(a, float("inf"))).double().numpy()
    dn = torch.nextafter(a, torch.full_like(a, -float("inf"))).double().numpy()
    af = a.double().numpy()
    return np.where(af <= x, af, dn), np.where(af >= x, af, up)


def _check_bound(inp, got, ref, err):
    """got (as stored) is what some float32 value within [ref - err, ref + err]
    stores to: itself (f32), its nearest bfloat16, or one of its two bfloat16
    neighbours (stochastic)."""
    sp = inp.spec
    got = got.astype(np.float64)
    if sp.out_dtype == "f32":
        ok = np.abs(got - ref) <= err
    elif sp.rounding == "nearest":
        ok = (got >= D.round_bf16(ref - err)) & (got <= D.round_bf16(ref + err))
    else:
        ok = (got >= _rd_ru(ref - err)[0]) & (got <= _rd_ru(ref + err)[1])
    assert ok.all(), f"{np.sum(~ok)} elements outside the bound"


def _spec(rows=70, cols=136, patches=None, **kw):
    if patches is None:
        patches = (WW.PatchSpec("lowrank", rank=24, strength_patch=0.7),
                   WW.PatchSpec("diff", offset=5, rows=40, strength_patch=1.3, strength_model=0.9),
                   WW.PatchSpec("lowrank", offset=33, rows=37, rank=8, strength_patch=-0.4,
                                strength_model=1.1),
                   WW.PatchSpec("diff", offset=60, rows=10, strength_patch=0.5, dtype="f32"))
    base = dict(name="t", rows=rows, cols=cols, patches=tuple(patches), seed=3, sr_seed=0x1234_5678_9ABC_DEF0)
    base.update(kw)
    return WW.WeightSpec(**base)


SMALL = (WW.PatchSpec("lowrank", rank=24, strength_patch=0.7),
         WW.PatchSpec("diff", offset=5, rows=20, strength_patch=1.3, strength_model=0.9),
         WW.PatchSpec("lowrank", offset=30, rows=7, rank=8, strength_patch=-0.4, strength_model=1.1),
         WW.PatchSpec("diff", offset=33, rows=4, strength_patch=0.5, dtype="f32"))

EXACT = [dict(w_dtype="bf16", out_dtype="bf16", rounding="stochastic"),
         dict(w_dtype="bf16", out_dtype="bf16", rounding="nearest"),
         dict(w_dtype="f32", out_dtype="f32"),
         dict(w_dtype="f32", out_dtype="bf16", rounding="stochastic"),
         dict(w_dtype="bf16", out_dtype="f32"),
         dict(rows=37, cols=61, w_dtype="bf16", out_dtype="bf16", rounding="stochastic", patches=SMALL),
         dict(rows=37, cols=61, w_dtype="f32", out_dtype="f32", patches=SMALL),  # element path
         dict(rows=200, cols=264, w_dtype="bf16", out_dtype="bf16", rounding="stochastic",
              patches=(WW.PatchSpec("lowrank", rank=72, strength_patch=0.9),
                       WW.PatchSpec("lowrank", offset=64, rows=100, rank=40, strength_patch=-1.2,
                                    strength_model=0.75),
                       WW.PatchSpec("lowrank", offset=150, rows=50, rank=3, strength_patch=2.0))),
         # every patch over every row, rows a multiple of 128 (the 128-row tiles), strength_model != 1
         dict(rows=256, cols=384, w_dtype="bf16", out_dtype="bf16", rounding="stochastic",
              patches=(WW.PatchSpec("lowrank", rank=32, strength_patch=0.9, strength_model=0.75),
                       WW.PatchSpec("lowrank", rank=16, strength_patch=-1.2))),
         dict(rows=256, cols=136, w_dtype="bf16", out_dtype="bf16", rounding="nearest",
              patches=(WW.PatchSpec("lowrank", rank=48, strength_patch=0.6),)),
         # patches on 128-row boundaries (each 128-row tile inside or outside each of them)
         dict(rows=384, cols=256, w_dtype="bf16", out_dtype="bf16", rounding="stochastic",
              patches=(WW.PatchSpec("lowrank", offset=128, rows=128, rank=16, strength_patch=1.5),
                       WW.PatchSpec("lowrank", offset=0, rows=256, rank=32, strength_patch=-0.5,
                                    strength_model=0.5),
                       WW.PatchSpec("lowrank", offset=256, rows=128, rank=48, strength_patch=0.25))),
         dict(rows=129, cols=8, w_dtype="bf16", out_dtype="bf16", rounding="stochastic",
              patches=(WW.PatchSpec("lowrank", rank=16), WW.PatchSpec("diff", offset=1, rows=127)))]


@pytest.mark.parametrize("kw", EXACT, ids=lambda k: "-".join(f"{v}" for v in k.values() if not isinstance(v, tuple)))
def test_weight_patch_bit_exact_on_dyadic_factors(kw):
    inp = WW.make_weight_inputs(_spec(dyadic=True, **kw))
    got = _run(inp)
    want = P.written(inp, P.reference32(inp))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
        f"{np.sum(got != want)} of {got.size} elements differ"


NONFINITE = {
    # every low-rank patch over every row (the strip kernel's full-cover path)
    "full": (WW.PatchSpec("lowrank", rank=16, strength_patch=0.7),
             WW.PatchSpec("lowrank", rank=32, strength_patch=-0.5)),
    # low-rank patches over parts of the rows
    "offset": (WW.PatchSpec("lowrank", offset=8, rows=100, rank=16, strength_patch=0.7),
               WW.PatchSpec("lowrank", offset=64, rows=64, rank=8, strength_patch=1.5, strength_model=0.5)),
    # one diff over every row (the pipelined streaming kernel), bf16 and fp32 diffs
    "diff": (WW.PatchSpec("diff", strength_patch=1.3, strength_model=0.9),),
    "diff_f32": (WW.PatchSpec("diff", strength_patch=-0.7, strength_model=1.1, dtype="f32"),),
    # two diffs over parts of the rows (the general streaming kernel)
    "diffs": (WW.PatchSpec("diff", offset=3, rows=90, strength_patch=1.3, strength_model=0.9),
              WW.PatchSpec("diff", offset=40, rows=88, strength_patch=0.5, dtype="f32")),
}


@pytest.mark.parametrize("rounding", ["stochastic", "nearest"])
@pytest.mark.parametrize("kind", list(NONFINITE))
def test_weight_patch_non_finite_weights(kind, rounding):
    """NaN and infinities in the weight: an infinity keeps its code, a NaN
    stays a NaN, and every finite element is bit-exact (dyadic factors), on
    each kernel's path."""
    inp = WW.make_weight_inputs(_spec(rows=128, cols=256, dyadic=True, w_dtype="bf16", out_dtype="bf16",
                                      rounding=rounding, patches=NONFINITE[kind]))
    idx = np.random.default_rng(11).choice(inp.w.size, 96, replace=False)
    inp.w.flat[idx[:32]] = np.nan
    inp.w.flat[idx[32:64]] = np.inf
    inp.w.flat[idx[64:]] = -np.inf
    got = _run(inp)
    with np.errstate(all="ignore"):  # the oracle's float64 steps on infinities and NaN
        want = P.written(inp, P.reference32(inp))
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn) and gn.sum() >= 32
    assert np.isinf(got).sum() >= 64
    assert np.array_equal(got[~gn].view(np.uint32), want[~wn].view(np.uint32)), \
        f"{np.sum(got[~gn] != want[~wn])} finite or infinite elements differ"


@pytest.mark.parametrize("out_dtype,rounding", [("f32", "nearest"), ("bf16", "nearest"), ("bf16", "stochastic")])
def test_weight_patch_random_factors_within_derived_bound(out_dtype, rounding):
    inp = WW.make_weight_inputs(_spec(rows=200, cols=264, w_dtype="f32", out_dtype=out_dtype,
                                      rounding=rounding, seed=9))
    got = _run(inp)
    _check_bound(inp, got, P.reference(inp), P.delta_error_bound(inp))
    if out_dtype == "bf16":
        # the float32 mirror's code, except where the summation order moved acc32
        # across a rounding decision (an ulp of acc32 decides 1 code in ~2^16)
        want = P.written(inp, P.reference32(inp))
        assert np.mean(got != want) < 1e-3


def test_weight_patch_in_place_equals_out_of_place_and_seed_matters():
    inp = WW.make_weight_inputs(_spec(rows=130, cols=256, w_dtype="bf16", out_dtype="bf16", seed=4))
    a = _run(inp)
    b = _run(inp, in_place=True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(a, _run(inp))  # deterministic
    c = _run(inp, seed=inp.spec.sr_seed + 1)
    assert 0.2 < np.mean(a != c) < 0.8  # another key draws other bits


def test_weight_patch_without_patches_is_a_cast():
    inp = WW.make_weight_inputs(_spec(rows=65, cols=200, w_dtype="f32", out_dtype="bf16",
                                      rounding="nearest", patches=()))
    got = _run(inp)
    assert np.array_equal(got, torch.from_numpy(inp.w).to(torch.bfloat16).float().numpy())


def _row_inputs(inp, r):
    """Weight row r alone, as a one-row workload (same patches, same strengths)."""
    sp = inp.spec
    pats, specs = [], []
    for pd in inp.patches:
        ps = pd.spec
        if not ps.offset <= r < ps.offset + pd.rows:
            continue
        k = r - ps.offset
        one = WW.PatchSpec(ps.kind, 0, 1, ps.rank, ps.strength_patch, ps.strength_model, ps.dtype)
        specs.append(one)
        pats.append(WW.PatchData(one, 1, None if pd.diff is None else pd.diff[k:k + 1],
                                 None if pd.up is None else pd.up[k:k + 1], pd.down))
    sub = WW.WeightSpec(sp.name, 1, sp.cols, sp.w_dtype, sp.out_dtype, tuple(specs), sp.rounding,
                        sp.sr_seed, sp.seed, sp.dyadic, sp.w_std)
    return WW.WeightInputs(sub, inp.w[r:r + 1], pats)


@pytest.mark.parametrize("name", list(WW.WEIGHT_CONFIGS))
def test_weight_patch_large_workloads_sampled_rows(name):
    inp = WW.make_weight_inputs(WW.weight_config(name))
    got = _run(inp)
    sp = inp.spec
    rows = sorted({0, 1, 63, 64, 3071, 3072, 3073, 6143, 6144, sp.rows // 2 + 17, sp.rows - 1})
    mism = 0
    for r in rows:
        sub = _row_inputs(inp, r)
        _check_bound(sub, got[r:r + 1], P.reference(sub), P.delta_error_bound(sub))
        acc = P.reference32(sub)[0]
        code = P.sr_bf16(acc, sp.sr_seed, base=r * sp.cols) if sp.rounding == "stochastic" \
            else P.store(acc, sp.out_dtype)
        if all(p.kind == "diff" for p in sp.patches):  # no summation-order freedom: exact
            assert np.array_equal(got[r], code), f"row {r}"
        mism += int(np.sum(got[r] != code))
    assert mism <= 1e-3 * len(rows) * sp.cols


# Every low-rank patch over every row of a weight of 384 x 384 units, a
# multiple of 256 of them (the unit kernel, one workgroup per CU): strength_model
# != 1, the most concatenated rank (128), two rounds of workgroups, four strips.
UNIT = {"three_sets_sm": ((12288, 3072), (WW.PatchSpec("lowrank", rank=16, strength_patch=1.0),
                                         WW.PatchSpec("lowrank", rank=32, strength_patch=0.8, strength_model=0.75),
                                         WW.PatchSpec("lowrank", rank=64, strength_patch=-0.6))),
        "rank_128": ((12288, 3072), (WW.PatchSpec("lowrank", rank=48, strength_patch=0.5),
                                    WW.PatchSpec("lowrank", rank=80, strength_patch=-1.5))),
        # 512 units: two rounds of workgroups
        "two_rounds": ((12288, 6144), (WW.PatchSpec("lowrank", rank=32, strength_patch=0.7),
                                       WW.PatchSpec("lowrank", rank=64, strength_patch=-0.3, strength_model=1.25))),
        # four 384-column strips, 64 row blocks
        "four_strips": ((24576, 1536), (WW.PatchSpec("lowrank", rank=16, strength_patch=2.0),
                                        WW.PatchSpec("lowrank", rank=16, strength_patch=-1.0),
                                        WW.PatchSpec("lowrank", rank=48, strength_patch=0.25)))}


@pytest.mark.parametrize("name", list(UNIT))
def test_weight_patch_unit_kernel_sampled_rows_bit_exact(name):
    """Dyadic factors (every partial sum a float32 number): sampled rows, in
    every unit row position and every wave of a unit, bit for bit against the
    oracle's float32 order with its Philox bits."""
    (rows, cols), pats = UNIT[name]
    sp = WW.WeightSpec(name="unit", rows=rows, cols=cols, w_dtype="bf16", out_dtype="bf16",
                       patches=pats, rounding="stochastic", sr_seed=0x0F1E_2D3C_4B5A_6978,
                       seed=7, dyadic=True)
    inp = WW.make_weight_inputs(sp)
    got = _run(inp)
    rng = np.random.default_rng(11)
    rows = sorted({0, 31, 32, 383, 384, sp.rows // 2 - 1, sp.rows - 1} | {int(r) for r in rng.integers(0, sp.rows, 40)})
    for r in rows:
        sub = _row_inputs(inp, r)
        code = P.sr_bf16(P.reference32(sub)[0], sp.sr_seed, base=r * sp.cols)
        assert np.array_equal(got[r], code), f"row {r}: {np.sum(got[r] != code)} elements differ"


def _misaligned(a, dtype=torch.bfloat16):
    """A contiguous device copy of `a` whose data pointer is 2 bytes past a
    16-byte boundary (a view one element into a larger buffer)."""
    flat = torch.from_numpy(np.ascontiguousarray(a, np.float32).ravel()).cuda().to(dtype)
    buf = torch.zeros(flat.numel() + 8, dtype=dtype, device="cuda")
    buf[1:1 + flat.numel()] = flat
    v = buf[1:1 + flat.numel()].view(a.shape)
    assert v.is_contiguous() and v.data_ptr() % 16 != 0
    return v


def test_weight_patch_rank_total_at_the_strip_limit():
    """Padded ranks summing to exactly 128 (the most the column-strip kernel
    holds), an offset patch among them, bit-exact."""
    pats = (WW.PatchSpec("lowrank", rank=64, strength_patch=0.5),
            WW.PatchSpec("lowrank", offset=70, rows=80, rank=60, strength_patch=-1.5, strength_model=0.5))
    inp = WW.make_weight_inputs(_spec(rows=150, cols=200, patches=pats, dyadic=True, seed=21))
    got = _run(inp)
    want = P.written(inp, P.reference32(inp))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("what", ["factors", "weight"])
def test_weight_patch_misaligned_arrays_bit_exact(what):
    """Factors (or the weight) 2 bytes off a 16-byte boundary take the element
    paths (no 16-byte accesses on them); results unchanged."""
    from bucketed_classifier_free_amd import WeightPatch, weight_patch
    inp = WW.make_weight_inputs(_spec(rows=90, cols=136, dyadic=True, seed=22))
    sp = inp.spec
    pats = []
    for pd in inp.patches:
        ps = pd.spec
        if ps.kind == "diff":
            pats.append(WeightPatch(ps.strength_patch, ps.strength_model, ps.offset,
                                    diff=torch.from_numpy(pd.diff).cuda().to(TDT[ps.dtype])))
        elif what == "factors":
            pats.append(WeightPatch(ps.strength_patch, ps.strength_model, ps.offset,
                                    up=_misaligned(pd.up), down=_misaligned(pd.down)))
        else:
            pats.append(WeightPatch(ps.strength_patch, ps.strength_model, ps.offset,
                                    up=torch.from_numpy(pd.up).cuda().to(torch.bfloat16),
                                    down=torch.from_numpy(pd.down).cuda().to(torch.bfloat16)))
    w = _misaligned(inp.w, TDT[sp.w_dtype]) if what == "weight" else \
        torch.from_numpy(inp.w).cuda().to(TDT[sp.w_dtype])
    out = torch.full(w.shape, float("nan"), dtype=TDT[sp.out_dtype], device="cuda")
    weight_patch(w, out, pats, rounding=sp.rounding, seed=sp.sr_seed)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    want = P.written(inp, P.reference32(inp))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
