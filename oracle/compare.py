"""Comparison of library outputs with the oracle's (test infrastructure).

Rules (the tolerances the fused epilogue is held to):
  * bf16: at most ``max_ulp`` (1) units in the last place apart, measured on
    the ordered bf16 bit patterns (so +0 and -0 are the same point); given the
    oracle's unrounded value as well, a value one unit away must be the other
    bf16 neighbour of that exact value (the two bracket it), and every value
    must lie within 2^-8 of the exact value, relative, plus 2^-16 for the
    kernel's own fp32 roundings (where the exact value is a normal bf16
    number): the correctly rounded value is within half a unit, 2^-8, and the
    kernel's fp32 arithmetic can only pick the other neighbour of an exact
    value that lies next to the midpoint between the two;
  * fp32 scales: relative difference at most 1e-6 (both exactly 0 for zero
    rows);
  * e4m3 codes: identical, except (i) codes of the same sign one step apart
    where the oracle flags the exact value as lying near a rounding midpoint,
    and (ii) 0x00 against 0x80. Both exceptions are counted and reported.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def _bf16_order(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _bf16_nan(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)


@dataclass
class Bf16Report:
    n: int
    n_diff: int          # elements not bit-identical (after +0/-0 folding)
    max_ulp: int
    max_rel: float       # against the oracle's rounded bf16 value
    max_rel_exact: float = float("nan")   # against the oracle's unrounded value, if given

    def __str__(self):
        ex = "" if self.max_rel_exact != self.max_rel_exact else \
            f", max rel to the exact value {self.max_rel_exact:.3g}"
        if self.n_diff == 0:
            return f"bf16: {self.n} values, all bit-identical{ex}"
        return (f"bf16: {self.n} values, {self.n_diff} differ by <= {self.max_ulp} ulp, "
                f"max rel {self.max_rel:.3g}{ex}")


REL_EXACT = 2.0 ** -8 + 2.0 ** -16
SMALLEST_NORMAL = 2.0 ** -126


def compare_bf16(got: np.ndarray, want: np.ndarray, max_ulp: int = 1, what: str = "bf16",
                 exact: np.ndarray = None, rtol_exact: float = REL_EXACT) -> Bf16Report:
    got = np.asarray(got, np.uint16).reshape(-1)
    want = np.asarray(want, np.uint16).reshape(-1)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    gn, wn = _bf16_nan(got), _bf16_nan(want)
    bad_nan = gn != wn
    if bad_nan.any():
        i = int(np.nonzero(bad_nan)[0][0])
        raise AssertionError(f"{what}: NaN mismatch at {i}: got {got[i]:#06x} want {want[i]:#06x}")
    ok = ~gn
    d = np.abs(_bf16_order(got[ok]) - _bf16_order(want[ok]))
    worst = int(d.max()) if d.size else 0
    if worst > max_ulp:
        idx = np.nonzero(ok)[0][int(d.argmax())]
        raise AssertionError(f"{what}: {int((d > max_ulp).sum())} values more than {max_ulp} ulp "
                             f"apart; worst at flat index {idx}: got {got[idx]:#06x} "
                             f"want {want[idx]:#06x} ({worst} ulp)")
    gf = (got[ok].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wf = (want[ok].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(wf != 0, np.abs(gf - wf) / np.abs(wf), np.abs(gf))
    rel_exact = float("nan")
    if exact is not None:
        ex = np.asarray(exact, np.float64).reshape(-1)
        assert ex.shape == got.shape, f"{what}: exact shape {ex.shape} vs {got.shape}"
        ex = ex[ok]
        # a value one unit from the correctly rounded one must lie on the other
        # side of the exact value: the two bf16 values bracket it
        step = _bf16_order(got[ok]) - _bf16_order(want[ok])
        side = np.sign(ex - wf)
        wrong = (step != 0) & (step != side)
        if wrong.any():
            i = np.nonzero(ok)[0][int(np.nonzero(wrong)[0][0])]
            raise AssertionError(f"{what}: at flat index {i} got {got[i]:#06x}, which with "
                                 f"{want[i]:#06x} does not bracket the exact value "
                                 f"{float(np.asarray(exact).reshape(-1)[i])!r}")
        with np.errstate(divide="ignore", invalid="ignore"):
            re = np.where(ex != 0, np.abs(gf - ex) / np.abs(ex), np.abs(gf))
        normal = np.abs(ex) >= SMALLEST_NORMAL
        if np.any(re[normal] > rtol_exact):
            j = int(np.argmax(np.where(normal, re, 0.0)))
            i = np.nonzero(ok)[0][j]
            raise AssertionError(f"{what}: at flat index {i} got {got[i]:#06x}, {re[j]:.3g} "
                                 f"from the exact value {ex[j]!r} (bound {rtol_exact:.4g})")
        rel_exact = float(re[normal].max()) if normal.any() else 0.0
    return Bf16Report(int(got.size), int((d > 0).sum()), worst,
                      float(rel.max()) if rel.size else 0.0, rel_exact)


def compare_scales(got: np.ndarray, want: np.ndarray, rtol: float = 1e-6, what: str = "scale"
                   ) -> float:
    got = np.asarray(got, np.float64).reshape(-1)
    want = np.asarray(want, np.float64).reshape(-1)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    zero = want == 0
    if np.any(got[zero] != 0):
        raise AssertionError(f"{what}: nonzero where the oracle has 0")
    rel = np.abs(got[~zero] - want[~zero]) / np.abs(want[~zero])
    worst = float(rel.max()) if rel.size else 0.0
    if worst > rtol:
        i = np.nonzero(~zero)[0][int(rel.argmax())]
        raise AssertionError(f"{what}: rel diff {worst:.3g} > {rtol} at {i}: got {got[i]!r} "
                             f"want {want[i]!r}")
    return worst


@dataclass
class Fp8Report:
    n: int
    n_tie: int           # off by one code at a flagged near-tie
    n_signed_zero: int   # 0x00 vs 0x80

    def __str__(self):
        return (f"e4m3: {self.n} codes, {self.n_tie} off-by-one at near-ties, "
                f"{self.n_signed_zero} signed-zero differences")


def compare_e4m3(got: np.ndarray, want: np.ndarray, near_tie: np.ndarray, what: str = "e4m3"
                 ) -> Fp8Report:
    got = np.asarray(got, np.uint8).reshape(-1).astype(np.int32)
    want = np.asarray(want, np.uint8).reshape(-1).astype(np.int32)
    near_tie = np.asarray(near_tie, bool).reshape(-1)
    assert got.shape == want.shape == near_tie.shape
    diff = got != want
    szero = diff & (((got == 0x00) & (want == 0x80)) | ((got == 0x80) & (want == 0x00)))
    same_sign = (got & 0x80) == (want & 0x80)
    step = np.abs((got & 0x7F) - (want & 0x7F)) == 1
    tie = diff & same_sign & step & near_tie
    fail = diff & ~szero & ~tie
    if fail.any():
        i = int(np.nonzero(fail)[0][0])
        raise AssertionError(f"{what}: {int(fail.sum())} codes differ outside near-ties; first at "
                             f"flat index {i}: got {got[i]:#04x} want {want[i]:#04x} "
                             f"(near_tie={bool(near_tie[i])})")
    return Fp8Report(int(got.size), int(tie.sum()), int(szero.sum()))
