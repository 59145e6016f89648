"""Seeded construction of blocks whose exact transformed amax lies within
2^-20 of a power of two (test helper: numpy and the oracle, no HIP code).

The E8M0 scale of a block is decided by the exponent of its amax (OCP
Microscaling v1.0, the Pith review's reference [10]).  A kernel that
computes the transform in fp32 in another order than the exact sum gets the
amax right only to within its rounding error, so where the exact amax sits
just above or just below a power of two it can pick the neighbouring scale.
These blocks put the exact amax (the oracle's fp64 sum of exact products,
rounded to fp32) on either side of a power of two, between 2^-30 and 2^-20
of it relative: far inside any fp32 evaluation's error, so a kernel passes
only if it decides such scales from exact values.  Some of the blocks just
below a power of two round up onto it in fp32, which decides their scale
too.

Construction: draw a bf16 block, pick the column with the largest |y|, then
replace four inputs one after the other so that each removes most of what
remains between that column and the chosen target (each step leaves about
2^-9 of the previous remainder, the bf16 rounding of the new input).  The
exact values are recomputed after every step with the oracle's arithmetic
(fp64 sequential sums of exact products), blocks whose chosen column is not
the amax any more are drawn again, and near_matrix_* return only blocks the
oracle itself confirms.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

WINDOW = 2.0 ** -20


def _bf16(v: np.ndarray) -> np.ndarray:
    """bf16 values (as fp64) nearest to v, via fp32."""
    return synth.bf16_to_f32(synth.f32_to_bf16(np.asarray(v, dtype=np.float32))).astype(np.float64)


def _kron_y(x: np.ndarray, K: np.ndarray) -> np.ndarray:
    """Every output column: fp64 sum from +0 in input order of x[r] K[r][c] (exact products)."""
    s = np.zeros(K.shape[1])
    for r in range(K.shape[0]):
        s = s + x[r] * K[r]
    return s


def _had_y(x: np.ndarray, B: int) -> np.ndarray:
    """Columns 0..31 of a block-Hadamard of size B: fp64 signed sum in input order, / sqrt(B)."""
    r = np.arange(B)[:, None]
    c = np.arange(32)[None, :]
    sgn = np.where(np.bitwise_count(r & c) % 2 == 1, -1.0, 1.0)
    s = np.zeros(32)
    for i in range(B):
        s = s + sgn[i] * x[i]
    return s / np.sqrt(float(B))


def side_of(amax: float) -> tuple[int, float]:
    """(p, rel): the power of two 2^p nearest to amax and amax / 2^p - 1."""
    p = int(np.round(np.log2(amax)))
    return p, amax / 2.0 ** p - 1.0


def _tune(x: np.ndarray, coef, ycol, rng, tuning: np.ndarray, side: int):
    """Move column ycol(x) onto a target 2^p (1 + side * delta) by replacing the
    tuning inputs; coef[r] is input r's weight in that column."""
    y = ycol(x)
    p, _ = side_of(abs(y))
    delta = 2.0 ** -rng.uniform(20.2, 30.0)
    target = np.sign(y) * 2.0 ** p * (1.0 + side * delta)
    x = x.copy()
    x[tuning] = 0.0
    for r in tuning:
        x[r] = _bf16(np.atleast_1d((target - ycol(x)) / coef[r]))[0]
    return x


def kron_near_block(K32: np.ndarray, rng, side: int, tries: int = 200):
    """bf16 bits [32] of a block whose exact amax (K32: the fp32 block) is within
    WINDOW of a power of two, above it (side +1) or below it (side -1); None if
    no draw succeeded."""
    K = K32.astype(np.float64)
    for _ in range(tries):
        x = _bf16(rng.standard_normal(32) * np.exp2(rng.integers(-3, 3, 32)))
        c = int(np.argmax(np.abs(_kron_y(x, K))))
        tuning = np.argsort(-np.abs(K[:, c]))[:4]
        x = _tune(x, K[:, c], lambda v: _kron_y(v, K)[c], rng, tuning, side)
        y = _kron_y(x, K)
        if int(np.argmax(np.abs(y))) != c or not np.all(np.isfinite(x)):
            continue
        _, rel = side_of(abs(y[c]))
        if 0 < side * rel <= WINDOW:
            return synth.f32_to_bf16(x.astype(np.float32))
    return None


def had_near_block(B: int, rng, side: int, tries: int = 200):
    """bf16 bits [B] of a Hadamard block of size B whose first 32 outputs have an
    exact amax within WINDOW of a power of two (side as above)."""
    for _ in range(tries):
        x = _bf16(rng.standard_normal(B) * np.exp2(rng.integers(-2, 2, B)))
        c = int(np.argmax(np.abs(_had_y(x, B))))
        sgn = np.where(np.bitwise_count(np.arange(B) & c) % 2 == 1, -1.0, 1.0) / np.sqrt(float(B))
        tuning = rng.choice(B, 4, replace=False)
        x = _tune(x, sgn, lambda v: _had_y(v, B)[c], rng, tuning, side)
        y = _had_y(x, B)
        if int(np.argmax(np.abs(y))) != c or not np.all(np.isfinite(x)):
            continue
        _, rel = side_of(abs(y[c]))
        if 0 < side * rel <= WINDOW:
            return synth.f32_to_bf16(x.astype(np.float32))
    return None


def near_matrix_kron(T: int, nb: int, seed: int, sigma: float = 0.1):
    """X [T, 32 nb] bf16 bits and P [nb, 5, 3]: every block near a power of two,
    sides alternating.  Returns (X, P, near) with near [T, nb] the blocks the
    oracle confirms (exact amax within WINDOW of a power of two)."""
    rng = np.random.default_rng(seed)
    P = synth.random_params(nb, seed=seed, sigma_lb=sigma, sigma_a=sigma)
    K32, _ = oracle.build_blocks(P, nb)
    X = np.zeros((T, 32 * nb), dtype=np.uint16)
    for t in range(T):
        for j in range(nb):
            b = kron_near_block(K32[j], rng, 1 if (t + j) % 2 == 0 else -1)
            X[t, 32 * j:32 * j + 32] = b if b is not None else synth.f32_to_bf16(rng.standard_normal(32).astype(np.float32))
    ref = oracle.quantize_rows(oracle.KRON, X, P, want_y=True)
    return X, P, confirmed(ref["yhat"])


def near_matrix_hadamard(T: int, d: int, B: int, seed: int):
    """X [T, d] bf16 bits: the first 32-channel block of every Hadamard block of
    size B near a power of two (sides alternating); (X, near) as above."""
    rng = np.random.default_rng(seed)
    X = np.zeros((T, d), dtype=np.uint16)
    for t in range(T):
        for k in range(d // B):
            b = had_near_block(B, rng, 1 if (t + k) % 2 == 0 else -1)
            X[t, B * k:B * k + B] = b if b is not None else synth.f32_to_bf16(rng.standard_normal(B).astype(np.float32))
    ref = oracle.quantize_rows_hadamard(X, B, want_y=True)
    return X, confirmed(ref["yhat"])


def confirmed(yhat: np.ndarray) -> np.ndarray:
    """[T, nb] bool: blocks whose exact amax (fp64, before the fp32 rounding) is
    within WINDOW of a power of two, on either side."""
    T, d = yhat.shape
    amax = np.abs(yhat).reshape(T, d // 32, 32).max(axis=2)
    with np.errstate(divide="ignore"):
        p = np.round(np.log2(np.where(amax > 0, amax, 1.0)))
    rel = amax / 2.0 ** p - 1.0
    return (amax > 0) & (np.abs(rel) <= WINDOW) & (rel != 0)
