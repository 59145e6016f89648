"""Seeded synthetic inputs for the KroQuant activation quantizer.

Only input construction lives here (see ``synth.c``): bf16 activation
matrices with the widths of the DiT linear layers the KroQuant paper measures
(PixArt-Sigma, SANA, FLUX.1-schnell; Pith review of arXiv 2607.21446,
"Summary"), Kronecker-factor parameters drawn around the identity, and
SmoothQuant-style channel multipliers.  No quantizer arithmetic: the CPU
oracle and the HIP library both consume these buffers and share nothing else.

The activations stand in for DiT activations on MJHQ-30K / SDCI prompts,
which are not available here: Gaussian (or GELU-shaped, or heavy-tailed)
values, a few outlier channels with a large multiplier, and an AdaLN-like
per-token scale (1 + s).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkqsynth.so")
_lib = None

BASE_NORMAL, BASE_GELU, BASE_STUDENT_T3 = 0, 1, 2


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        i64, u64, dbl, vp, ci = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        lib.synth_matrix.argtypes = [vp, i64, i64, u64, u64, ci, i64, dbl, dbl, dbl, ci, vp]
        lib.synth_matrix.restype = ci
        lib.synth_params.argtypes = [vp, i64, u64, u64, dbl, dbl, ci]
        lib.synth_params.restype = ci
        lib.synth_smooth_mult.argtypes = [vp, i64, i64, vp]
        lib.synth_smooth_mult.restype = ci
        lib.synth_u64.argtypes = [u64, u64, u64]
        lib.synth_u64.restype = u64
        lib.synth_uniform.argtypes = [u64, u64, u64]
        lib.synth_uniform.restype = dbl
        lib.synth_normal.argtypes = [u64, u64, u64]
        lib.synth_normal.restype = dbl
        lib.synth_adaln.argtypes = [vp, vp, i64, i64, u64, u64, dbl, dbl, dbl]
        lib.synth_adaln.restype = ci
        _lib = lib
    return _lib


@dataclass(frozen=True)
class MatrixSpec:
    """One activation matrix X[T][d] (bf16) plus its per-block parameters."""

    name: str
    T: int
    d: int
    seed: int
    matrix_id: int
    kind: int
    outlier_frac: float
    outlier_mult: float
    token_sigma: float
    zero_frac: float = 0.0
    special_blocks: bool = False
    sigma_lb: float = 0.1
    sigma_a: float = 0.1
    shared_k: bool = False  # one K for every block (parameter stride 0)

    @property
    def nb(self) -> int:
        return self.d // 32

    @property
    def n_outliers(self) -> int:
        return int(round(self.outlier_frac * self.d)) if self.outlier_frac < 1 else int(self.outlier_frac)

    def with_rows(self, T: int) -> "MatrixSpec":
        return MatrixSpec(**{**self.__dict__, "T": T})


def _spec(name, T, d, seed, mid, kind, frac, mult, tsig, **kw):
    return MatrixSpec(name, T, d, seed, mid, kind, frac, mult, tsig, **kw)


# The five workloads.  Outlier counts are round(fraction * d); config 0 fixes 12.
CONFIGS: dict[int, list[MatrixSpec]] = {
    0: [_spec("tiny", 256, 1152, 0, 1, BASE_NORMAL, 12, 50.0, 0.5, special_blocks=True)],
    1: [
        _spec("pixart_x1", 8192, 1152, 1, 1, BASE_NORMAL, 0.01, 50.0, 0.5),
        _spec("pixart_x2", 8192, 4608, 1, 2, BASE_GELU, 0.01, 50.0, 0.5),
    ],
    2: [
        _spec("sana_x1", 4096, 2240, 2, 1, BASE_NORMAL, 0.02, 80.0, 0.5),
        _spec("sana_x2", 4096, 5600, 2, 2, BASE_GELU, 0.02, 80.0, 0.5),
        _spec("sana_x1_sharedk", 4096, 2240, 2, 1, BASE_NORMAL, 0.02, 80.0, 0.5, shared_k=True),
        _spec("sana_x2_sharedk", 4096, 5600, 2, 2, BASE_GELU, 0.02, 80.0, 0.5, shared_k=True),
    ],
    3: [
        _spec("flux_x1", 4608, 3072, 3, 1, BASE_NORMAL, 0.005, 100.0, 1.0),
        _spec("flux_x2", 4608, 12288, 3, 2, BASE_NORMAL, 0.005, 100.0, 1.0),
    ],
    4: [_spec("stress", 18432, 12288, 4, 1, BASE_STUDENT_T3, 0.01, 200.0, 0.0, zero_frac=0.01)],
}

STRESS_CALLS = 57  # config 4 is timed as this many back-to-back calls


def all_specs() -> list[MatrixSpec]:
    return [s for c in sorted(CONFIGS) for s in CONFIGS[c]]


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def matrix(spec: MatrixSpec, threads: int | None = None, with_outliers: bool = False):
    """X as a uint16 array [T, d] of bf16 bit patterns (and the outlier channel list)."""
    lib = _load()
    X = np.empty((spec.T, spec.d), dtype=np.uint16)
    outl = np.empty(max(spec.n_outliers, 1), dtype=np.int64)
    rc = lib.synth_matrix(
        X.ctypes.data, spec.T, spec.d, spec.seed, spec.matrix_id, spec.kind, spec.n_outliers,
        spec.outlier_mult, spec.token_sigma, spec.zero_frac, threads or default_threads(), outl.ctypes.data,
    )
    if rc != 0:
        raise RuntimeError(f"synth_matrix failed ({rc}) for {spec}")
    if with_outliers:
        return X, outl[: spec.n_outliers].copy()
    return X


def params(spec: MatrixSpec) -> np.ndarray:
    """Kronecker-factor parameters float32 [nb, 5, 3], (l, a, b) per factor.

    With ``spec.shared_k`` only one block's worth ([1, 5, 3]) is returned: the
    caller passes parameter stride 0 so every block uses it."""
    lib = _load()
    nb = 1 if spec.shared_k else spec.nb
    P = np.empty((nb, 5, 3), dtype=np.float32)
    rc = lib.synth_params(P.ctypes.data, nb, spec.seed, spec.matrix_id, spec.sigma_lb, spec.sigma_a,
                          1 if spec.special_blocks else 0)
    if rc != 0:
        raise RuntimeError("synth_params failed")
    return P


def random_params(nb: int, seed: int, matrix_id: int = 9, sigma_lb: float = 0.1, sigma_a: float = 0.1) -> np.ndarray:
    lib = _load()
    P = np.empty((nb, 5, 3), dtype=np.float32)
    if lib.synth_params(P.ctypes.data, nb, seed, matrix_id, sigma_lb, sigma_a, 0) != 0:
        raise RuntimeError("synth_params failed")
    return P


def random_matrix(T: int, d: int, seed: int, kind: int = BASE_NORMAL, n_outliers: int = 0, mult: float = 50.0,
                  token_sigma: float = 0.5, zero_frac: float = 0.0, matrix_id: int = 7) -> np.ndarray:
    spec = MatrixSpec("adhoc", T, d, seed, matrix_id, kind, n_outliers, mult, token_sigma, zero_frac)
    return matrix(spec)


def adaln_vectors(n_samples: int, d: int, seed: int, matrix_id: int = 11, sigma: float = 0.5,
                  amplified_frac: float = 0.01, amp: float = 20.0):
    """AdaLN (scale, shift), float32 [n_samples, d] each: N(0, sigma) values, and a
    fixed 1% of channels whose scale is raised by ``amp`` (amplified channels)."""
    lib = _load()
    sc = np.empty((n_samples, d), dtype=np.float32)
    sh = np.empty((n_samples, d), dtype=np.float32)
    if lib.synth_adaln(sc.ctypes.data, sh.ctypes.data, n_samples, d, seed, matrix_id, sigma, amplified_frac, amp) != 0:
        raise RuntimeError("synth_adaln failed")
    return sc, sh


def smooth_mult(X: np.ndarray) -> np.ndarray:
    """Channel multipliers m[d] = 1/sqrt(max_t |X[:, c]|) (1 for an all-zero column)."""
    lib = _load()
    X = np.ascontiguousarray(X, dtype=np.uint16)
    T, d = X.shape
    m = np.empty(d, dtype=np.float32)
    if lib.synth_smooth_mult(X.ctypes.data, T, d, m.ctypes.data) != 0:
        raise RuntimeError("synth_smooth_mult failed")
    return m


def bf16_to_f32(X: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (X.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


def u64(seed: int, stream: int, i: int) -> int:
    return int(_load().synth_u64(seed, stream, i))
