"""Reference values for the oracle's scale and code decisions, computed from
the definitions with no code shared with the oracle or the kernels:

* E4M3 values come from torch's float8_e4m3fn decoding; the nearest code is
  found against the midpoints of that table, ties to the even code.
* E2M1 nearest values by distance to the magnitudes of the "FP4" page
  ("Como funciona FP4") that bracket the value, ties to the even index
  (`test_e2m1_nearest_is_exhaustive_search` checks it against a search over
  all 8).
* Squared errors in float64, in the input domain: sum of (g * eff - |x|)^2.
  g * eff is exact (2 + 24 significant bits), and the subtraction, the
  square and a sum of at most 256 terms each round at 2^-53, so the float64
  value is within 1e-13 of the exact rational one, relatively
  (`test_float64_sse_is_exact_to_1e13` checks this against fractions).

`fp32_band` bounds how far the oracle's float32 evaluation of a candidate's
error can be from that exact value, from the operations the oracle's reading
of the 4/6 criterion performs (see the function). Decisions closer than the
sum of two candidates' bands are near-ties: there, the exact-rational choice
and the float32 one may differ, and both are correct readings.
"""
from __future__ import annotations

import numpy as np
import torch

U = 2.0 ** -24                       # unit roundoff of binary32
FLT_MIN = 2.0 ** -126
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

E4M3 = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()  # codes 0..126, ascending
E4M3_MID = (E4M3[:-1] + E4M3[1:]) / 2.0


def e4m3_rne(s: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code to s (float64, >= 0; values above 448 give 448),
    ties to the even code."""
    s = np.minimum(np.asarray(s, np.float64), 448.0)
    k = np.clip(np.searchsorted(E4M3, s, side="right") - 1, 0, 125)   # E4M3[k] <= s
    mid = E4M3_MID[k]
    up = (s > mid) | ((s == mid) & (k % 2 == 1))
    return np.where(s >= 448.0, 126, k + up).astype(np.int64)


def e4m3_near_midpoint(s: np.ndarray, rel: float) -> np.ndarray:
    """True where s lies within rel * s of a rounding midpoint of E4M3."""
    s = np.minimum(np.asarray(s, np.float64), 448.0)
    k = np.clip(np.searchsorted(E4M3_MID, s), 0, len(E4M3_MID) - 1)
    d = np.minimum(np.abs(s - E4M3_MID[k]), np.abs(s - E4M3_MID[np.maximum(k - 1, 0)]))
    return d <= rel * s


def e2m1_nearest(t: np.ndarray) -> np.ndarray:
    """Index (0..7) of the E2M1 magnitude nearest to t >= 0, ties to the even
    index. The nearest magnitude is one of the two that bracket t (the last
    two above 6), so their distances decide."""
    t = np.asarray(t, np.float64).reshape(-1)
    hi = np.clip(np.searchsorted(GRID, t, side="left"), 1, 7)   # GRID[hi - 1] < t <= GRID[hi], or t > 6
    lo = hi - 1
    dl, dh = t - GRID[lo], np.abs(GRID[hi] - t)
    return np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(lo % 2 == 0, lo, hi))).astype(np.int64)


def e2m1_near_midpoint(t: np.ndarray, rel: float) -> np.ndarray:
    """True where t lies within rel * t of a midpoint between neighbouring
    magnitudes (where a relative perturbation of rel may change the
    nearest value)."""
    mids = (GRID[:-1] + GRID[1:]) / 2.0
    t = np.asarray(t, np.float64)
    k = np.clip(np.searchsorted(mids, t), 1, len(mids) - 1)   # the two midpoints around t
    return np.minimum(np.abs(t - mids[k - 1]), np.abs(t - mids[k])) <= rel * t


def block_terms(xb: np.ndarray, eff: np.ndarray):
    """xb [n, k] blocks of input values, eff [n] effective scales (>= FLT_MIN).
    Returns t = |x| / eff [n, k], the nearest magnitudes g [n, k] and the
    exact-to-1e-13 squared error sum((g eff - |x|)^2) [n]."""
    ax = np.abs(np.asarray(xb, np.float64))
    eff = np.asarray(eff, np.float64)[:, None]
    t = ax / eff
    g = GRID[e2m1_nearest(t)].reshape(t.shape)
    sse = ((g * eff - ax) ** 2).sum(axis=1)
    return t, g, sse


def fp32_band(t: np.ndarray, g: np.ndarray, eff: np.ndarray, k_sum: float, rel_q: float = 2.01 * U) -> np.ndarray:
    """Bound on |float32 error of a candidate - exact error| for blocks whose
    elements are scaled as q = fl(x * fl(1 / eff)) (|q - t| <= rel_q * t,
    plus 2^-149 where q is subnormal), whose squared distances to the
    nearest magnitude (a 1-Lipschitz function of q) are summed by float32
    operations with k_sum roundings along any path (an 8-term FMA chain, the
    adds that join chains, the tree over a tile's rows), then multiplied by
    fl(eff * eff) (two more roundings). Times 1.5 for second-order terms."""
    eff = np.asarray(eff, np.float64)
    d = np.abs(g - t)
    delta = rel_q * t + 2.0 ** -149
    s = (d ** 2).sum(axis=1)
    e_q = (2.0 * d * delta + delta ** 2).sum(axis=1)
    return 1.5 * eff ** 2 * (e_q + k_sum * U * s + 2.01 * U * s)
