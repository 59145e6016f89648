"""Comparison of a quantizer's output with the oracle's (test infrastructure).

Acceptance, per matrix and kernel:
  * E8M0 scales: bit-exact everywhere;
  * E2M1 codes: exact except where the exact value y / 2^e lies within the
    transform's error bound of a rounding midpoint (several codes are then
    correct); such a code must keep the sign and differ by one grid step, or
    be a zero code whose sign differs for a value within the bound of zero;
    at least 99.99% of all codes must be exact;
  * front-ends without accumulation (plain, SmoothQuant, identity K): every
    code exact.
The error bound is TOL * (block amax) on the pre-quantization value, TOL = 1e-5.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import E2M1_GRID, unpack_codes

TOL = 1e-5
MIDPOINTS = (E2M1_GRID[:-1] + E2M1_GRID[1:]) / 2.0


@dataclass
class Report:
    n_codes: int = 0
    n_scales: int = 0
    scale_mismatch: int = 0
    code_mismatch: int = 0
    code_unexplained: int = 0
    details: list = field(default_factory=list)

    @property
    def exact_fraction(self) -> float:
        return 1.0 - self.code_mismatch / max(self.n_codes, 1)

    def ok(self, exact: bool = False) -> bool:
        if self.scale_mismatch or self.code_unexplained:
            return False
        if exact:
            return self.code_mismatch == 0
        return self.exact_fraction >= 0.9999

    def __str__(self) -> str:
        return (f"codes {self.n_codes} mismatched {self.code_mismatch} (unexplained {self.code_unexplained}, "
                f"exact {100 * self.exact_fraction:.5f}%), scales {self.n_scales} mismatched {self.scale_mismatch}"
                + (f"; first: {self.details[:4]}" if self.details else ""))


def compare(codes: np.ndarray, scales: np.ndarray, ref_codes: np.ndarray, ref_scales: np.ndarray,
            ref_yhat_rows=None, tol: float = TOL) -> Report:
    """Compare packed codes [T, d/2] and scales [T, d/32] with the oracle's.

    ref_yhat_rows(rows) -> (yhat [len(rows), d] fp64, y32 [len(rows), d]) gives
    the oracle's pre-rounding values for the rows that have code mismatches;
    without it every code mismatch counts as unexplained."""
    r = Report(n_codes=codes.size * 2, n_scales=scales.size)
    smis = scales != ref_scales
    r.scale_mismatch = int(smis.sum())
    if r.scale_mismatch:
        t, j = np.nonzero(smis)
        r.details += [("scale", int(a), int(b), int(scales[a, b]), int(ref_scales[a, b])) for a, b in zip(t[:8], j[:8])]
    cmis_rows = np.nonzero(np.any(codes != ref_codes, axis=1))[0]
    if len(cmis_rows) == 0:
        return r
    c = unpack_codes(codes[cmis_rows])
    rc = unpack_codes(ref_codes[cmis_rows])
    bad = c != rc
    r.code_mismatch = int(bad.sum())
    if ref_yhat_rows is None:
        r.code_unexplained = r.code_mismatch
        return r
    yhat, y32 = ref_yhat_rows(cmis_rows)
    d = yhat.shape[1]
    amax = np.abs(y32.astype(np.float64)).reshape(len(cmis_rows), d // 32, 32).max(axis=2)
    e = ref_scales[cmis_rows].astype(np.int64) - 127
    ti, ci = np.nonzero(bad)
    for t, ch in zip(ti, ci):
        j = ch // 32
        g, gr = int(c[t, ch]), int(rc[t, ch])
        v = yhat[t, ch] / 2.0 ** e[t, j]
        err = tol * amax[t, j] / 2.0 ** e[t, j]
        same_sign = (g >> 3) == (gr >> 3)
        step = abs((g & 7) - (gr & 7)) == 1
        lo = min(g & 7, gr & 7)
        mid = MIDPOINTS[lo] if lo < 7 else np.inf
        near_mid = abs(abs(v) - mid) <= err
        # +0 and -0 codes both decode to zero; the sign is undetermined when the
        # exact value is within the error bound of zero
        zero_sign = (g & 7) == 0 and (gr & 7) == 0 and abs(v) <= err
        if not ((same_sign and step and near_mid) or zero_sign):
            r.code_unexplained += 1
            if len(r.details) < 16:
                r.details.append(("code", int(cmis_rows[t]), int(ch), g, gr, float(v)))
    return r


def transform_error(y_gpu: np.ndarray, yhat: np.ndarray, y32: np.ndarray) -> float:
    """max over elements of |y_gpu - yhat| / (block amax of the oracle's y)."""
    T, d = y_gpu.shape
    amax = np.abs(y32.astype(np.float64)).reshape(T, d // 32, 32).max(axis=2)
    amax = np.repeat(amax, 32, axis=1)
    err = np.abs(y_gpu.astype(np.float64) - yhat)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(amax > 0, err / amax, np.where(err > 0, np.inf, 0.0))
    return float(rel.max()) if rel.size else 0.0
