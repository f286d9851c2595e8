"""The output parity bar: the library's 16-bit outputs against the oracle's.

No GPU and none of the method's arithmetic here: the oracle (oracle/) gives
the exact output, its rounding to the 16-bit format (out_bits), the row
normaliser (l, the float sum of the unquantised p~) and the unrounded
255 * p~ that each p8 rounds (e255); this module only compares.

The bar, per output element:
  * in a row where no 255 * p~ lies within TIE of a rounding tie, the
    library's bits are at most 1 ulp from the oracle's out_bits (the kernel
    forms the same integer A; its float32 row sum and last multiply differ
    from the oracle's float64 ones by far less than one 16-bit ulp);
  * in a row with such near-tie keys (float32 scores in the kernel, float64
    in the oracle, may round one of those p8 the other way), the distance to
    the oracle's exact output is at most one 16-bit spacing plus what those
    keys can move it: each changes A_c by v8_jc, i.e. the output by
    |v8_jc| scale_c / (255 l). The allowance used, (|v8_jc| scale_c +
    |O_c|) / (255 l - n), is that bound widened so that it also holds for
    the integer normaliser (sum p8, which such a key moves by 1).
The looser bound of the method's statement, 2e-2 * max|V|, is reported and
checked beside it.
"""
from __future__ import annotations

import numpy as np

from workloads import F16, from_bits

# How close to a rounding tie (in units of p8) a 255 * p~ must lie for the
# kernel's float32 scores to be allowed to round it the other way: the
# float32 error of the exponent argument is below 1e-6 (in log2 units) and
# of v_exp_f32 about one float ulp, so 255 * p~ moves by at most ~2e-4.
TIE = 2e-3


def _order(bits: np.ndarray) -> np.ndarray:
    """16-bit sign-magnitude patterns -> integers in value order (+0 == -0)."""
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Number of 16-bit steps between two arrays of the same format."""
    return np.abs(_order(a_bits) - _order(b_bits))


def spacing(x: np.ndarray, dtype: int) -> np.ndarray:
    """One ulp of the 16-bit format at |x| (the subnormal step below the
    normal range)."""
    mant, emin = (10, -14) if dtype == F16 else (7, -126)
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - mant).astype(np.int64))


def tie_allowance(ref, vq: np.ndarray, vscale: np.ndarray):
    """(allowance [nbh,nrows,d], near-tie count [nbh,nrows]) for an oracle
    result with e255. vq: int8 [nbh, N, d] and vscale [nbh, d] of the
    result's heads."""
    e = ref.e255
    frac = e - np.floor(e)
    near = np.abs(frac - 0.5) < TIE
    n = near.sum(-1)                                     # [nbh, nrows]
    den = np.maximum(255.0 * ref.l - n, 1.0)
    av = np.abs(vq.astype(np.float64)) * vscale[:, None, :].astype(np.float64)  # [nbh, N, d]
    move = np.einsum("hrn,hnd->hrd", near.astype(np.float64), av)
    allow = (move + n[..., None] * np.abs(ref.out)) / den[..., None]
    return allow, n


def check_output(got_bits: np.ndarray, ref, vq: np.ndarray, vscale: np.ndarray, dtype: int,
                 vmax: float, label: str = "", loose: float = 2e-2) -> dict:
    """Assert the bar above for got_bits (uint16 [nbh, nrows, d]) against
    an oracle result computed with want_e255; returns the statistics."""
    got_bits = np.ascontiguousarray(got_bits, np.uint16)
    got = from_bits(got_bits, dtype).astype(np.float64)
    dist = ulp_distance(got_bits, ref.out_bits)
    allow, n = tie_allowance(ref, vq, vscale)
    clean = (n == 0)[..., None] & np.ones_like(dist, dtype=bool)
    dev = np.abs(got - ref.out)
    room = allow + spacing(np.maximum(np.abs(got), np.abs(ref.out)), dtype)
    bad_clean = clean & (dist > 1)
    bad_tie = ~clean & (dev > room)
    stats = {
        "identical": float((dist == 0).mean()),
        "within_1ulp": float((dist <= 1).mean()),
        "rows_with_near_ties": int((n > 0).sum()),
        "rows": int(n.size),
        "max_ulp_clean_rows": int(dist[clean].max()) if clean.any() else 0,
        "max_dev_over_room": float((dev / room).max()),
        "max_err_over_vmax": float(dev.max() / vmax),
    }
    print(f"{label}: bit-identical {stats['identical']:.4f}, within 1 ulp {stats['within_1ulp']:.4f}, "
          f"rows with near-tie p8 {stats['rows_with_near_ties']}/{stats['rows']}, "
          f"max ulp (rows without) {stats['max_ulp_clean_rows']}, max dev/bound {stats['max_dev_over_room']:.3f}, "
          f"max|err|/max|V| {stats['max_err_over_vmax']:.2e}")
    assert np.isfinite(got).all(), label
    assert not bad_clean.any(), (label, int(bad_clean.sum()), "elements > 1 ulp in rows without near ties")
    assert not bad_tie.any(), (label, int(bad_tie.sum()), "elements beyond the near-tie bound")
    assert stats["max_err_over_vmax"] <= loose, (label, stats["max_err_over_vmax"])
    return stats


def violations(got_bits: np.ndarray, ref, vq: np.ndarray, vscale: np.ndarray, dtype: int) -> float:
    """Fraction of elements that break the bar (0.0 for a passing output)."""
    got = from_bits(np.ascontiguousarray(got_bits, np.uint16), dtype).astype(np.float64)
    dist = ulp_distance(got_bits, ref.out_bits)
    allow, n = tie_allowance(ref, vq, vscale)
    clean = (n == 0)[..., None]
    room = allow + spacing(np.maximum(np.abs(got), np.abs(ref.out)), dtype)
    bad = np.where(clean, dist > 1, np.abs(got - ref.out) > room)
    return float(bad.mean())
