"""Pins of the oracle's per-block decisions against exact references, on
about 10^5 blocks each: the NVFP4 tensor scale and block-scale codes, the
4/6 choice ("Quatro sobre seis", introduction: keep the lower-error of the
max-to-4 and max-to-6 scalings) in 1D, 2D and 2D-transposed blocks, the
scale search over every E4M3 code between those two, the MXFP4 exponent
pair, and the element codes under the chosen scale.

The oracle evaluates each candidate's squared error in float32, in a fixed
order (a reading: the pages fix only "lower error"). Here every decision is
compared with the exact-rational choice (tests/exact_ref.py) wherever the two
candidates' errors differ by more than the derived bound on that float32
evaluation (exact_ref.fp32_band, about 1e-6 relative); only closer pairs,
true near-ties that any float32 evaluation order may split either way, are
left out, and they must stay rare. Scale codes are compared with the exact
nearest E4M3 code except where the exact block scale lies within the float32
rounding of the oracle's s = a * fl(1 / (M S_t)) (3 roundings) of an E4M3
midpoint. CPU only."""
from fractions import Fraction

import numpy as np
import pytest

import exact_ref as X

NV, MX = 1, 0
FOS, B2D, TR, SEARCH = 1, 2, 4, 32
U = X.U


def unpack(codes):
    return np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)


def make_input(rng, rows, cols, blk_r, blk_c, lo=-6.0, hi=6.0, flat=0.3):
    """Values with full float32 mantissas and a log-uniform magnitude per
    blk_r x blk_c block (2^lo .. 2^hi): normal values in most blocks, and in
    a fraction `flat` of them magnitudes uniform in [0.4, 1] with random signs
    (blocks where max-to-4 often wins, also as 16 x 16 tiles); 3% outliers
    x3..x12 in the normal blocks and some exact zeros. Every candidate wins somewhere; ties and
    subnormal scales occur."""
    x = rng.standard_normal((rows, cols))
    fl = np.repeat(np.repeat(rng.random((rows // blk_r, cols // blk_c)) < flat, blk_r, axis=0), blk_c, axis=1)
    x = np.where(fl, rng.uniform(0.4, 1.0, (rows, cols)) * np.sign(x), x)
    mag = np.exp2(rng.uniform(lo, hi, (rows // blk_r, cols // blk_c)))
    x *= np.repeat(np.repeat(mag, blk_r, axis=0), blk_c, axis=1)
    out = (rng.random((rows, cols)) < 0.03) & ~fl
    x[out] *= rng.uniform(3, 12, out.sum())
    x[rng.random((rows, cols)) < 0.002] = 0.0
    return x.astype(np.float32)


def as_blocks(a, tile):
    """[R, C] -> [R/tile * C/16, tile * 16]: 1 x 16 blocks or 16 x 16 tiles,
    row-major over the block grid."""
    R, C = a.shape
    return a.reshape(R // tile, tile, C // 16, 16).transpose(0, 2, 1, 3).reshape(-1, tile * 16)


def correctly_rounded_f32(v: np.float32, exact: Fraction) -> bool:
    fv = Fraction(float(v))
    for nb in (np.nextafter(v, np.float32(np.inf)), np.nextafter(v, np.float32(0))):
        if abs(Fraction(float(nb)) - exact) < abs(fv - exact):
            return False
    return True


def candidate(blocks, code, St, k_sum):
    """Error (float64, exact to 1e-13) and float32-evaluation band of each
    block under E4M3 code `code` [n]; infinite error for a zero block
    (eff below the smallest normal float32: the reading makes such a
    candidate lose)."""
    eff = (np.float32(X.E4M3[code].astype(np.float32)) * np.float32(St)).astype(np.float64)
    zero = eff < X.FLT_MIN
    sse = np.full(len(code), np.inf)
    band = np.zeros(len(code))
    ok = ~zero
    if ok.any():
        t, g, s = X.block_terms(blocks[ok], eff[ok])
        sse[ok] = s
        band[ok] = X.fp32_band(t, g, eff[ok], k_sum)
    return sse, band


def check_codes(blocks, codes, chosen, St):
    """Element codes under the chosen scale: sign bit of x; magnitude the
    nearest E2M1 value of |x| / eff, except within the float32 rounding of
    q = fl(x fl(1/eff)) of a midpoint, where either neighbour is right; a
    zero block keeps only signs."""
    eff = (X.E4M3[chosen].astype(np.float32) * np.float32(St)).astype(np.float64)
    sign = np.signbit(blocks).astype(np.int64) * 8
    assert ((codes & 8) == sign).all()
    zero = eff < X.FLT_MIN
    assert ((codes[zero] & 7) == 0).all()
    t = np.abs(blocks[~zero].astype(np.float64)) / eff[~zero, None]
    want = X.e2m1_nearest(t).reshape(t.shape)
    got = codes[~zero] & 7
    near = X.e2m1_near_midpoint(t, 2.01 * U)
    assert ((got == want) | (near & (np.abs(got - want) <= 1))).all()
    return near.mean()


def run_nv(O, x, flags):
    q = O.quantize(x, NV, flags=flags)
    St = np.float32(q["tensor_scale"])
    T = float(np.abs(x).max())
    D = 1792 if flags & (FOS | SEARCH) else 2688
    assert correctly_rounded_f32(St, Fraction(T) / D)
    xs = x.T if flags & TR else x
    tile = 16 if flags & B2D else 1
    blocks = as_blocks(np.ascontiguousarray(xs), tile)
    chosen = q["scales"][::tile].reshape(-1).astype(np.int64)  # one byte per block, row-major over blocks
    codes = as_blocks(unpack(q["codes"]), tile).astype(np.int64)
    a = np.abs(blocks.astype(np.float64)).max(axis=1)
    s6, s4 = a / (6.0 * float(St)), a / (4.0 * float(St))
    c6, c4 = X.e4m3_rne(s6), X.e4m3_rne(s4)
    near = X.e4m3_near_midpoint(s6, 3.01 * U)
    if flags & (FOS | SEARCH):
        near |= X.e4m3_near_midpoint(s4, 3.01 * U)
    return dict(blocks=blocks, chosen=chosen, codes=codes, St=St, c6=c6, c4=c4, near=near,
                k_sum=14.0 if tile == 16 else 10.0)


def test_e2m1_nearest_is_exhaustive_search():
    rng = np.random.default_rng(39)
    mids = (X.GRID[:-1] + X.GRID[1:]) / 2
    t = np.concatenate([rng.uniform(0, 9, 200_000), X.GRID, mids, np.nextafter(mids, 0), np.nextafter(mids, 9),
                        [0.0, 1e-300, 6.0, 7.0, 1e6]])
    d = np.abs(t[:, None] - X.GRID[None, :])
    ties = d == d.min(axis=1, keepdims=True)
    want = np.where(ties.sum(axis=1) > 1, np.argmax(ties & (np.arange(8) % 2 == 0), axis=1), np.argmax(ties, axis=1))
    np.testing.assert_array_equal(X.e2m1_nearest(t), want)


def test_float64_sse_is_exact_to_1e13():
    """The float64 error sums of exact_ref equal the exact rational ones to
    1e-13 relative (the property that lets them stand for exact errors)."""
    rng = np.random.default_rng(40)
    x = make_input(rng, 64, 256, 1, 16)
    blocks = as_blocks(x, 1)[:300]
    eff = np.float32(2.0 ** rng.uniform(-8, 8, len(blocks))).astype(np.float64)
    _, g, sse = X.block_terms(blocks, eff)
    for i in range(len(blocks)):
        e = Fraction(float(eff[i]))
        want = sum((Fraction(float(gi)) * e - abs(Fraction(float(xi)))) ** 2 for gi, xi in zip(g[i], blocks[i]))
        assert abs(Fraction(float(sse[i])) - want) <= Fraction(1, 10 ** 13) * want


def test_nvfp4_plain_scale_codes_and_tensor_scale(oracle):
    """The block-scale code is the nearest E4M3 of amax / (6 S_t) and S_t the
    correctly rounded T / 2688, on 10^5 blocks."""
    rng = np.random.default_rng(41)
    x = make_input(rng, 4000, 400, 1, 16)
    r = run_nv(oracle, x, 0)
    ok = ~r["near"]
    assert r["near"].mean() < 1e-3
    np.testing.assert_array_equal(r["chosen"][ok], r["c6"][ok])
    assert check_codes(r["blocks"], r["codes"], r["chosen"], r["St"]) < 1e-3


@pytest.mark.parametrize("flags,shape", [(FOS, (4000, 400)), (FOS | B2D, (4096, 6400)),
                                         (FOS | B2D | TR, (6400, 4096))],
                         ids=["1d", "2d", "2d-transposed"])
def test_four_over_six_is_the_exact_argmin(oracle, flags, shape):
    rng = np.random.default_rng(42 + flags)
    x = make_input(rng, *shape, 16 if flags & B2D else 1, 16)
    r = run_nv(oracle, x, flags)
    n = len(r["chosen"])
    assert n >= 100_000
    e6, b6 = candidate(r["blocks"], r["c6"], r["St"], r["k_sum"])
    e4, b4 = candidate(r["blocks"], r["c4"], r["St"], r["k_sum"])
    exact = np.where(e4 < e6, r["c4"], r["c6"])
    gap = np.abs(e4 - e6)
    # exact ties keep 6; they arise where the two effective scales differ by
    # exactly 2 (E4M3 codes 1 and 2) and every value stays below 3 after
    # scaling, so the float32 evaluations scale by a power of two and tie too
    certain = ~r["near"] & ((r["c4"] == r["c6"]) | (gap == 0) | (gap > b4 + b6 + 1e-12 * (e4 + e6)))
    in_set = (r["chosen"] == r["c6"]) | (r["chosen"] == r["c4"])
    assert in_set[~r["near"]].all()
    bad = np.nonzero(certain & (r["chosen"] != exact))[0]
    assert len(bad) == 0, f"{len(bad)} decisions differ from the exact argmin, first block {bad[:5]}"
    assert (~certain).mean() < 0.005, (~certain).mean()
    four = (r["chosen"] == r["c4"]) & (r["c4"] != r["c6"])
    assert 0.05 < four.mean() < 0.95  # both candidates win often
    rel = (b4 + b6)[np.isfinite(e6) & (e6 > 0)] / e6[np.isfinite(e6) & (e6 > 0)]
    assert np.median(rel) < 1e-5  # the band is tight
    check_codes(r["blocks"], r["codes"], r["chosen"], r["St"])
    print(f"{n} blocks, {(~certain).sum()} near-ties or near-midpoint, 4 chosen in {four.mean():.3f}")


@pytest.mark.parametrize("flags,shape", [(SEARCH, (4000, 400)), (SEARCH | B2D, (2048, 6400)),
                                         (SEARCH | B2D | TR, (6400, 2048))],
                         ids=["1d", "2d", "2d-transposed"])
def test_scale_search_is_the_exact_argmin(oracle, flags, shape):
    """Every E4M3 code from the 6-candidate's to the 4-candidate's is tried;
    the chosen one has the smallest exact error (ties keep the smaller code)
    wherever the runner-up is not within the float32 band."""
    rng = np.random.default_rng(50 + flags)
    x = make_input(rng, *shape, 16 if flags & B2D else 1, 16)
    r = run_nv(oracle, x, flags)
    n = len(r["chosen"])
    assert n >= 50_000
    width = int((r["c4"] - r["c6"]).max()) + 1
    errs = np.full((n, width), np.inf)
    bands = np.zeros((n, width))
    for j in range(width):
        c = np.minimum(r["c6"] + j, 126)
        e, b = candidate(r["blocks"], c, r["St"], r["k_sum"])
        valid = r["c6"] + j <= r["c4"]
        errs[valid, j] = e[valid]
        bands[valid, j] = b[valid]
    best = np.argmin(errs, axis=1)
    eb = errs[np.arange(n), best]
    bb = bands[np.arange(n), best]
    others = errs.copy()
    others[np.arange(n), best] = np.inf
    margin = others - eb[:, None] - bands - bb[:, None]
    certain = ~r["near"] & (np.nan_to_num(margin, nan=np.inf, posinf=np.inf).min(axis=1) > 1e-12 * eb)
    certain |= ~r["near"] & ~np.isfinite(eb)  # every candidate a zero block: the 6 one stays
    exact = np.where(np.isfinite(eb), r["c6"] + best, r["c6"])
    assert ((r["chosen"] >= r["c6"]) & (r["chosen"] <= r["c4"]))[~r["near"]].all()
    bad = np.nonzero(certain & (r["chosen"] != exact))[0]
    assert len(bad) == 0, f"{len(bad)} decisions differ from the exact argmin, first block {bad[:5]}"
    assert (~certain).mean() < 0.01, (~certain).mean()
    inner = (r["chosen"] > r["c6"]) & (r["chosen"] < r["c4"])
    assert inner.mean() > 0.05  # codes strictly between the 4/6 pair do win
    check_codes(r["blocks"], r["codes"], r["chosen"], r["St"])


def test_mxfp4_exponent_pair_is_the_exact_argmin(oracle):
    """MXFP4 under 4/6: the exponent is e = floor(log2 amax) - 2 or e + 1,
    whichever has the smaller exact error (e + 1 iff 4 S_{e+1} < S_e with
    S the error of x 2^-e, exact in float64 here), on 10^5 blocks; codes
    are the nearest E2M1 values of x 2^-e (exact: no rounding in x 2^-e)."""
    rng = np.random.default_rng(60)
    x = make_input(rng, 2500, 1280, 1, 32, lo=-30, hi=30)
    q = oracle.quantize(x, MX, flags=FOS)
    blocks = x.reshape(-1, 32).astype(np.float64)
    n = len(blocks)
    assert n >= 100_000
    chosen = q["scales"].reshape(-1).astype(np.int64) - 127
    a = np.abs(blocks).max(axis=1)
    _, E = np.frexp(a)
    e0 = np.where(a > 0, np.clip(E - 3, -127, 127), -127)

    def scaled_err(e):
        t = np.abs(blocks) * np.exp2(-e.astype(np.float64))[:, None]
        g = X.GRID[X.e2m1_nearest(t)].reshape(t.shape)
        return ((g - t) ** 2).sum(axis=1)
    s0, s1 = scaled_err(e0), scaled_err(e0 + 1)
    up = (4.0 * s1 < s0) & (e0 < 127)
    band = 1.5 * 11.0 * U * (4.0 * s1 + s0) + 32 * 2.0 ** -140
    # exact ties (4 S_{e+1} = S_e: nothing clips under e, so every error
    # scales by exactly 4, in float32 too) keep e
    certain = (4.0 * s1 == s0) | (np.abs(4.0 * s1 - s0) > band) | (e0 >= 127)
    assert ((chosen == e0) | (chosen == e0 + 1)).all()
    bad = np.nonzero(certain & (chosen != np.where(up, e0 + 1, e0)))[0]
    assert len(bad) == 0, f"{len(bad)} blocks differ from the exact argmin, first {bad[:5]}"
    assert (~certain).mean() < 0.005
    assert 0.05 < (chosen == e0 + 1).mean() < 0.95
    t = np.abs(blocks) * np.exp2(-chosen.astype(np.float64))[:, None]
    want = X.e2m1_nearest(t).reshape(t.shape)
    got = unpack(q["codes"]).reshape(-1, 32).astype(np.int64)
    np.testing.assert_array_equal(got & 7, want)
    np.testing.assert_array_equal(got >> 3, np.signbit(blocks).astype(np.int64))


def test_whole_tensor_scale_codes_are_nearest(oracle):
    """Whole-tensor scale (every block scale 1.0, S_t = T / 6): S_t is the
    correctly rounded T / 6 and every code the nearest E2M1 value of x / S_t,
    outside the float32 rounding band, on 10^5 blocks."""
    rng = np.random.default_rng(43)
    x = make_input(rng, 4000, 400, 1, 16, lo=-2, hi=2)
    q = oracle.quantize(x, NV, flags=64)
    St = np.float32(q["tensor_scale"])
    assert correctly_rounded_f32(St, Fraction(float(np.abs(x).max())) / 6)
    assert (q["scales"] == 0x38).all()
    blocks = as_blocks(x, 1)
    chosen = np.full(len(blocks), 0x38, np.int64)
    assert check_codes(blocks, as_blocks(unpack(q["codes"]), 1).astype(np.int64), chosen, St) < 1e-3
