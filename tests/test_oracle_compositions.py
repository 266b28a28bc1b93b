"""Pins of how the oracle's quantizer composes its separately pinned steps.

Random Hadamard transform ("FP4", "Inferencia e Treinamento FP4"; "Quatro
sobre seis", option list): quantizing with the transform equals quantizing a
copy of the input that was rotated 16 values at a time along the block
direction (down the columns of X for a transposed quantize), codes, scales,
tensor scale and amax alike, so the transform comes before every amax and
runs along the right axis. On inputs of small integers times a power of two
per 16 x 16 tile, the rotated copy is the dense Sylvester matrix product in
float64, exact, and independent of the oracle's butterfly.

Stochastic rounding ("FP4", "Inferencia e Treinamento FP4": stochastic
rounding for gradients): the scale is the one round-to-nearest-even picks,
and every code is the oracle's pinned e2m1_sr of fl(x * fl(1 / eff)) (NVFP4)
or x * 2^-e (MXFP4), drawn with the 16-bit random number of the element's
row-major output index L (batch items included) taken from rocRAND's
Philox4x32-10 stream. Over 2^12 offsets, the dequantized mean of a block is
the exact expectation of that rounding, which is x up to 2^-16 of a grid
step. CPU only."""
import numpy as np
import pytest

import exact_ref as X

MX, NV = 0, 1
FOS, B2D, TR, SR, RHT, SEARCH = 1, 2, 4, 8, 16, 32


def sylvester16():
    h = np.array([[1.0]])
    for _ in range(4):
        h = np.block([[h, h], [h, -h]])
    return h


def dense_rht_rows(x: np.ndarray, signs: int) -> np.ndarray:
    """Every 16-slice v of every row of x -> H16 D v / 4 in float64, H16 the
    Sylvester matrix and D the sign diagonal (bit i of `signs` negates v_i)."""
    R, C = x.shape
    d = np.array([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)])
    v = x.astype(np.float64).reshape(R, C // 16, 16) * d
    return (v @ sylvester16().T / 4.0).reshape(R, C)


def exact_input(rng, rows, cols):
    """Integers in [-40, 40] times 2^k per 16 x 16 tile (k in [-8, 8]): every
    butterfly sum is exact in float32, so the float32 transform equals the
    exact one, along rows and along columns."""
    ints = rng.integers(-40, 41, (rows, cols)).astype(np.float64)
    k = rng.integers(-8, 9, (rows // 16, cols // 16))
    return (ints * np.exp2(np.repeat(np.repeat(k, 16, axis=0), 16, axis=1))).astype(np.float32)


def same(a, b, what):
    np.testing.assert_array_equal(a["codes"], b["codes"], err_msg=f"codes {what}")
    np.testing.assert_array_equal(a["scales"], b["scales"], err_msg=f"scales {what}")
    if a["tensor_scale"] is not None:
        assert np.float32(a["tensor_scale"]).view(np.uint32) == np.float32(b["tensor_scale"]).view(np.uint32), what
        assert np.float32(a["amax"]).view(np.uint32) == np.float32(b["amax"]).view(np.uint32), what


RHT_CASES = [(MX, 0), (MX, FOS), (NV, 0), (NV, FOS), (NV, SEARCH), (NV, FOS | B2D),
             (MX, TR), (MX, FOS | TR), (NV, TR), (NV, FOS | TR), (NV, SEARCH | TR)]


@pytest.mark.parametrize("fmt,flags", RHT_CASES, ids=[f"{'nv' if f else 'mx'}-{g}" for f, g in RHT_CASES])
def test_hadamard_quantize_is_quantize_of_the_rotated_copy(oracle, fmt, flags):
    rng = np.random.default_rng(70 + flags + 100 * fmt)
    signs = int(rng.integers(0, 1 << 16))
    x = exact_input(rng, 96, 128)
    tr = bool(flags & TR)
    # rotate along the block direction: rows of X, or rows of X^T
    y64 = dense_rht_rows(x.T, signs).T if tr else dense_rht_rows(x, signs)
    y = y64.astype(np.float32)
    assert (y.astype(np.float64) == y64).all()  # the float32 copy is the exact rotation
    # the oracle's own butterfly gives the same copy on this input
    xs = np.ascontiguousarray(x.T if tr else x)
    ys = np.stack([oracle.rht16(v, signs) for v in xs.reshape(-1, 16)]).reshape(xs.shape)
    np.testing.assert_array_equal(ys, y.T if tr else y)
    a = oracle.quantize(x, fmt, flags=flags | RHT, rht_signs=signs)
    b = oracle.quantize(y, fmt, flags=flags)
    same(a, b, f"fmt={fmt} flags={flags}")


@pytest.mark.parametrize("fmt,flags", [(MX, 0), (NV, FOS), (NV, FOS | TR), (NV, B2D | FOS)])
def test_hadamard_on_general_inputs_uses_the_pinned_butterfly(oracle, fmt, flags):
    """Normal inputs with outliers (the transform is then inexact): the
    quantize equals that of the copy rotated slice by slice with the
    oracle's 16-point transform, itself pinned to the Sylvester matrix."""
    rng = np.random.default_rng(80 + flags)
    x = (rng.standard_normal((64, 192)) * np.exp(rng.uniform(-3, 3, (64, 1)))).astype(np.float32)
    x[rng.random(x.shape) < 0.01] *= 30
    signs = 0xB38E
    tr = bool(flags & TR)
    xs = np.ascontiguousarray(x.T if tr else x)
    ys = np.stack([oracle.rht16(v, signs) for v in xs.reshape(-1, 16)]).reshape(xs.shape)
    y = np.ascontiguousarray(ys.T) if tr else ys
    same(oracle.quantize(x, fmt, flags=flags | RHT, rht_signs=signs), oracle.quantize(y, fmt, flags=flags),
         f"fmt={fmt} flags={flags}")


# ---------------------------------------------------------------------------
# stochastic rounding
# ---------------------------------------------------------------------------
def rocrand_r16(philox, seed, offset, L):
    """16-bit random numbers of linear indices L (int array): output L >> 3 of
    rocRAND's stream (counter (n, 0, offset)), word (L >> 1) & 3, low half for
    even L."""
    words = philox(seed, offset, int(L.max() >> 3) + 1)
    w = words[L >> 3, (L >> 1) & 3].astype(np.uint32)
    return np.where(L & 1, w >> 16, w & 0xFFFF).astype(np.uint32)


def scaled_values(x_out: np.ndarray, fmt: int, scales: np.ndarray, St):
    """The values SR rounds: NVFP4 q = fl(x * fl(1 / eff)), eff = fl(E4M3 *
    S_t), in float32; MXFP4 x * 2^-e (exact barring underflow). Also a mask of
    NVFP4 zero blocks (eff below the smallest normal)."""
    R, C = x_out.shape
    blk = 16 if fmt == NV else 32
    s = np.repeat(scales.astype(np.int64), blk, axis=1)
    if fmt == NV:
        eff = X.E4M3[s].astype(np.float32) * np.float32(St)
        zero = eff < np.float32(X.FLT_MIN)
        r = np.float32(1.0) / np.where(zero, np.float32(1.0), eff)
        return (x_out * r).astype(np.float32), zero
    q = (x_out.astype(np.float64) * np.exp2(-(s - 127).astype(np.float64))).astype(np.float32)
    return q, np.zeros(q.shape, bool)


SR_CASES = [(NV, FOS, 0), (NV, FOS | TR, 0), (NV, FOS | B2D, 0), (NV, 0, 0), (NV, SEARCH, 0), (MX, 0, 0),
            (MX, TR, 0), (MX, FOS, 0), (NV, FOS, 2), (NV, FOS | TR, 1), (MX, 0, 2)]


@pytest.mark.parametrize("fmt,flags,item", SR_CASES,
                         ids=[f"{'nv' if f else 'mx'}-{g}-item{i}" for f, g, i in SR_CASES])
def test_sr_codes_are_e2m1_sr_of_the_scaled_value(oracle, rocrand_philox, fmt, flags, item):
    """Batch item `item` of a batch of items of this shape: its first output
    element has linear index L0 = item * R * C."""
    rng = np.random.default_rng(90 + flags + 7 * item)
    rows, cols = 64, 96
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-4, 4, (rows // 16, 1))).repeat(16, 0))
    x = x.astype(np.float32)
    x[5, :] = 0.0
    x[6, :] *= np.float32(1e-30)  # NVFP4 zero blocks
    seed, offset = 0x1234_5678_9ABC, 3
    R, C = (cols, rows) if flags & TR else (rows, cols)
    L0 = item * R * C
    q_sr = oracle.quantize(x, fmt, flags=flags | SR, seed=seed, offset=offset, L0=L0)
    q_rn = oracle.quantize(x, fmt, flags=flags, L0=L0)
    np.testing.assert_array_equal(q_sr["scales"], q_rn["scales"])  # selection from the RNE candidates
    xo = np.ascontiguousarray(x.T if flags & TR else x)
    q, zero = scaled_values(xo, fmt, q_sr["scales"], q_sr["tensor_scale"])
    L = L0 + np.arange(R * C, dtype=np.int64)
    want = oracle.e2m1_sr(q.reshape(-1), rocrand_r16(rocrand_philox, seed, offset, L)).reshape(R, C)
    want = np.where(zero, np.signbit(xo).astype(np.uint8) * 8, want)
    got = np.stack([q_sr["codes"] & 15, q_sr["codes"] >> 4], axis=-1).reshape(R, C)
    np.testing.assert_array_equal(got, want)
    assert (got != np.stack([q_rn["codes"] & 15, q_rn["codes"] >> 4], axis=-1).reshape(R, C)).any()


@pytest.mark.parametrize("fmt,flags", [(NV, FOS), (MX, 0)])
def test_sr_dequantized_mean_is_unbiased_over_offsets(oracle, fmt, flags):
    """2^12 Philox offsets on one input (fixed scales, since they come from
    the RNE choice): the mean dequantized value of each element is within 6
    standard errors of the exact expectation lo + ceil(f 2^16) / 2^16 (hi -
    lo) of the rounding of q, and that expectation is q up to 2^-16 of the
    grid step: unbiased."""
    rng = np.random.default_rng(99)
    x = (rng.standard_normal((1, 64)) * 3).astype(np.float32)
    n = 4096
    deq = np.zeros((n, 64))
    for o in range(n):
        r = oracle.quantize(x, fmt, flags=flags | SR, seed=7, offset=o)
        deq[o] = oracle.dequantize(fmt, r["codes"], r["scales"], r["tensor_scale"])[0]
    base = oracle.quantize(x, fmt, flags=flags)
    q, _ = scaled_values(x, fmt, base["scales"], base["tensor_scale"])
    blk = 16 if fmt == NV else 32
    s = np.repeat(base["scales"].astype(np.int64), blk, axis=1)[0]
    eff = (X.E4M3[s].astype(np.float32) * np.float32(base["tensor_scale"])).astype(np.float64) if fmt == NV \
        else np.exp2((s - 127).astype(np.float64))
    a = np.abs(q[0].astype(np.float64))
    sat = a >= 6.0  # saturates: always 6
    lo_i = np.clip(np.searchsorted(X.GRID, a, side="right") - 1, 0, 6)
    lo, hi = X.GRID[lo_i], X.GRID[lo_i + 1]
    f = np.where(sat, 0.0, (a - lo) / (hi - lo))
    p_up = np.ceil(f * 65536) / 65536
    mag = np.where(sat, 6.0, lo + p_up * (hi - lo))
    expect = np.sign(q[0]) * mag * eff
    sigma = (hi - lo) * eff * np.sqrt(p_up * (1 - p_up))
    # dequantized values are fl(g eff): one float32 rounding off the exact g eff
    assert (np.abs(deq.mean(axis=0) - expect) <= 6 * sigma / np.sqrt(n) + 6.0 * eff * 2.0 ** -24).all()
    unsat = ~sat
    assert (np.abs(expect - q[0] * eff)[unsat] <= ((hi - lo) * eff * 2.0 ** -16)[unsat] + 1e-12).all()
    assert unsat.sum() >= 60
    assert len({tuple(d) for d in deq[:64]}) > 32  # the offset changes the draws
