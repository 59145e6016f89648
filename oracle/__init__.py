"""CPU oracle for the KroQuant online activation quantizer (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the product path.  The C
source (``kq_oracle.c``) is a plain single-threaded fp64 implementation of the
method as the pages define it; it shares no code with the HIP library.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against something other than itself (closed forms, numpy/scipy library
routines, brute force, hand-worked values).  See that file's docstrings.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkqoracle.so")

KRON, PLAIN, SMOOTH, HADAMARD = 0, 1, 2, 3
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no FMA contraction)."""
    import subprocess

    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall",
           os.path.join(_HERE, "kq_oracle.c"), "-o", LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, ci, f, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
        L.kqo_factor.argtypes = [f, f, f, vp]
        L.kqo_factor_inverse.argtypes = [f, f, f, vp]
        L.kqo_kron_dense.argtypes = [vp, vp]
        L.kqo_kron_butterfly.argtypes = [vp, vp]
        L.kqo_kron_inverse.argtypes = [vp, vp]
        L.kqo_block_f32.argtypes = [vp, vp]
        L.kqo_build_blocks.argtypes = [vp, i64, i64, vp, vp, ci]
        L.kqo_e2m1_index.argtypes = [d]
        L.kqo_e2m1_index.restype = ci
        L.kqo_e8m0.argtypes = [f]
        L.kqo_e8m0.restype = ctypes.c_uint8
        L.kqo_quantize_block.argtypes = [vp, vp, vp]
        L.kqo_quantize_rows.argtypes = [ci, vp, i64, i64, vp, i64, vp, i64, i64, vp, vp, vp, vp]
        L.kqo_quantize_rows.restype = ci
        L.kqo_quantize_f32_rows.argtypes = [vp, i64, i64, vp, vp]
        L.kqo_quantize_f32_rows.restype = ci
        L.kqo_fwht32.argtypes = [vp]
        L.kqo_det.argtypes = [vp, ci]
        L.kqo_det.restype = d
        L.kqo_build_blocks_inverse_t.argtypes = [vp, i64, i64, vp, vp, ci]
        L.kqo_dequant_rows.argtypes = [vp, vp, i64, i64, vp]
        L.kqo_quantize_rows_blocks.argtypes = [vp, i64, i64, vp, i64, i64, i64, vp, vp, vp, vp]
        L.kqo_quantize_rows_blocks.restype = ci
        L.kqo_quantize_rows_hadamard.argtypes = [vp, i64, i64, ci, i64, i64, vp, vp, vp, vp]
        L.kqo_quantize_rows_hadamard.restype = ci
        L.kqo_build_blocks16.argtypes = [vp, i64, vp]
        L.kqo_row_stats.argtypes = [vp, i64, i64, d, vp]
        L.kqo_row_stats.restype = ci
        L.kqo_adaln_rows.argtypes = [vp, i64, i64, vp, vp, vp, i64, vp]
        L.kqo_adaln_rows.restype = ci
        _lib = L
    return _lib


def _p15(P) -> np.ndarray:
    P = np.ascontiguousarray(P, dtype=np.float32).reshape(-1)
    assert P.size == 15
    return P


def factor(l: float, a: float, b: float) -> np.ndarray:
    G = np.empty(4, dtype=np.float64)
    lib().kqo_factor(l, a, b, G.ctypes.data)
    return G.reshape(2, 2)


def factor_inverse(l: float, a: float, b: float) -> np.ndarray:
    G = np.empty(4, dtype=np.float64)
    lib().kqo_factor_inverse(l, a, b, G.ctypes.data)
    return G.reshape(2, 2)


def kron_dense(P) -> np.ndarray:
    P = _p15(P)
    K = np.empty(1024, dtype=np.float64)
    lib().kqo_kron_dense(P.ctypes.data, K.ctypes.data)
    return K.reshape(32, 32)


def kron_butterfly(P) -> np.ndarray:
    P = _p15(P)
    K = np.empty(1024, dtype=np.float64)
    lib().kqo_kron_butterfly(P.ctypes.data, K.ctypes.data)
    return K.reshape(32, 32)


def kron_inverse(P) -> np.ndarray:
    P = _p15(P)
    K = np.empty(1024, dtype=np.float64)
    lib().kqo_kron_inverse(P.ctypes.data, K.ctypes.data)
    return K.reshape(32, 32)


def block_f32(P) -> np.ndarray:
    P = _p15(P)
    K = np.empty(1024, dtype=np.float32)
    lib().kqo_block_f32(P.ctypes.data, K.ctypes.data)
    return K.reshape(32, 32)


def build_blocks(P, nb: int, pstride: int = 15, n_split: int = 3):
    """(K32 [nb,32,32] fp32 row-major (r, c), Kbf [nb,n_split,32,32] bf16 bits transposed (c, r))."""
    P = np.ascontiguousarray(P, dtype=np.float32).reshape(-1)
    K32 = np.empty((nb, 32, 32), dtype=np.float32)
    Kbf = np.empty((nb, n_split, 32, 32), dtype=np.uint16)
    lib().kqo_build_blocks(P.ctypes.data, nb, pstride, K32.ctypes.data, Kbf.ctypes.data, n_split)
    return K32, Kbf


def e2m1_index(m: float) -> int:
    return int(lib().kqo_e2m1_index(float(m)))


def e8m0(amax: float) -> int:
    return int(lib().kqo_e8m0(float(amax)))


def quantize_block(y) -> tuple[np.ndarray, int]:
    y = np.ascontiguousarray(y, dtype=np.float32).reshape(32)
    codes = np.zeros(16, dtype=np.uint8)
    sc = np.zeros(1, dtype=np.uint8)
    lib().kqo_quantize_block(y.ctypes.data, codes.ctypes.data, sc.ctypes.data)
    return codes, int(sc[0])


def quantize_f32_rows(Y: np.ndarray):
    """MXFP4 codes and scales of fp32 values Y [n, d] (no transform)."""
    Y = np.ascontiguousarray(Y, dtype=np.float32)
    n, d = Y.shape
    codes = np.zeros((n, d // 2), dtype=np.uint8)
    scales = np.zeros((n, d // 32), dtype=np.uint8)
    if lib().kqo_quantize_f32_rows(Y.ctypes.data, n, d, codes.ctypes.data, scales.ctypes.data) != 0:
        raise ValueError("oracle rejected its arguments")
    return codes, scales


def fwht32(v) -> np.ndarray:
    v = np.array(v, dtype=np.float64).reshape(32).copy()
    lib().kqo_fwht32(v.ctypes.data)
    return v


def det(A) -> float:
    A = np.ascontiguousarray(A, dtype=np.float64)
    return float(lib().kqo_det(A.ctypes.data, A.shape[0]))


def quantize_rows(front: int, X: np.ndarray, P=None, pstride: int = 15, m=None, row0: int = 0, row1=None,
                  want_y: bool = False, threads: int = 1):
    """Run the oracle over rows [row0, row1) of X (uint16 bf16 bits [T, d]).

    Returns dict(codes [n, d/2] u8, scales [n, d/32] u8, and with want_y: y32
    [n, d] f32, yhat [n, d] f64).  ``threads`` > 1 splits rows across Python
    threads, each calling the same single-threaded C routine."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    T, d = X.shape
    row1 = T if row1 is None else row1
    n = row1 - row0
    codes = np.zeros((n, d // 2), dtype=np.uint8)
    scales = np.zeros((n, d // 32), dtype=np.uint8)
    y32 = np.zeros((n, d), dtype=np.float32) if want_y else None
    yhat = np.zeros((n, d), dtype=np.float64) if want_y else None
    Pc = None if P is None else np.ascontiguousarray(P, dtype=np.float32)
    mc = None if m is None else np.ascontiguousarray(m, dtype=np.float32)
    L = lib()

    def run(a: int, b: int) -> int:
        if a >= b:
            return 0
        off = a - row0
        return L.kqo_quantize_rows(
            front, X.ctypes.data, T, d, None if Pc is None else Pc.ctypes.data, pstride,
            None if mc is None else mc.ctypes.data, a, b,
            codes[off:].ctypes.data, scales[off:].ctypes.data,
            None if y32 is None else y32[off:].ctypes.data, None if yhat is None else yhat[off:].ctypes.data)

    if threads <= 1 or n < 2 * threads:
        rc = run(row0, row1)
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
    else:
        step = (n + threads - 1) // threads
        with ThreadPoolExecutor(threads) as ex:
            rcs = list(ex.map(lambda i: run(row0 + i * step, min(row1, row0 + (i + 1) * step)), range(threads)))
        if any(rcs):
            raise ValueError("oracle rejected its arguments")
    out = {"codes": codes, "scales": scales}
    if want_y:
        out["y32"], out["yhat"] = y32, yhat
    return out


def build_blocks_inverse_t(P, nb: int, pstride: int = 15, n_split: int = 3):
    """Blocks of the weight fold: (K^-T as fp32 [nb,32,32] (r, c), its bf16 split [nb,n_split,32,32] (c, r))."""
    P = np.ascontiguousarray(P, dtype=np.float32).reshape(-1)
    K32 = np.empty((nb, 32, 32), dtype=np.float32)
    Kbf = np.empty((nb, n_split, 32, 32), dtype=np.uint16)
    lib().kqo_build_blocks_inverse_t(P.ctypes.data, nb, pstride, K32.ctypes.data, Kbf.ctypes.data, n_split)
    return K32, Kbf


def quantize_rows_blocks(X: np.ndarray, K32: np.ndarray, want_y: bool = False, threads: int = 1):
    """KroQuant front-end + MXFP4 with given fp32 blocks K32 [nb, 32, 32] (r, c) (e.g. the weight
    fold's K^-T).  Returns dict(codes, scales[, y32, yhat]) like quantize_rows."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    K32 = np.ascontiguousarray(K32, dtype=np.float32)
    T, d = X.shape
    kstride = 0 if K32.shape[0] == 1 and d > 32 else 1024
    codes = np.zeros((T, d // 2), dtype=np.uint8)
    scales = np.zeros((T, d // 32), dtype=np.uint8)
    y32 = np.zeros((T, d), dtype=np.float32) if want_y else None
    yhat = np.zeros((T, d), dtype=np.float64) if want_y else None
    L = lib()

    def run(a: int, b: int) -> int:
        if a >= b:
            return 0
        return L.kqo_quantize_rows_blocks(X.ctypes.data, T, d, K32.ctypes.data, kstride, a, b,
                                          codes[a:].ctypes.data, scales[a:].ctypes.data,
                                          None if y32 is None else y32[a:].ctypes.data,
                                          None if yhat is None else yhat[a:].ctypes.data)

    if threads <= 1 or T < 2 * threads:
        rcs = [run(0, T)]
    else:
        step = (T + threads - 1) // threads
        with ThreadPoolExecutor(threads) as ex:
            rcs = list(ex.map(lambda i: run(i * step, min(T, (i + 1) * step)), range(threads)))
    if any(rcs):
        raise ValueError("oracle rejected its arguments")
    out = {"codes": codes, "scales": scales}
    if want_y:
        out["y32"], out["yhat"] = y32, yhat
    return out


def quantize_rows_hadamard(X: np.ndarray, B: int, want_y: bool = False):
    """Block-Hadamard front-end of size B (32..512) + MXFP4: dict(codes, scales[, y32, yhat])."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    T, d = X.shape
    out = {"codes": np.zeros((T, d // 2), np.uint8), "scales": np.zeros((T, d // 32), np.uint8)}
    if want_y:
        out["y32"] = np.zeros((T, d), np.float32)
        out["yhat"] = np.zeros((T, d), np.float64)
    rc = lib().kqo_quantize_rows_hadamard(X.ctypes.data, T, d, int(B), 0, T, out["codes"].ctypes.data,
                                          out["scales"].ctypes.data,
                                          out["y32"].ctypes.data if want_y else None,
                                          out["yhat"].ctypes.data if want_y else None)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def build_blocks16(P16) -> np.ndarray:
    """16-wide, 4-factor blocks as block-diagonal fp32 32x32 blocks [nb16/2, 32, 32] (P16: [nb16, 4, 3])."""
    P16 = np.ascontiguousarray(P16, dtype=np.float32)
    nb16 = P16.shape[0]
    if nb16 % 2:
        raise ValueError("nb16 must be even")
    K = np.empty((nb16 // 2, 32, 32), dtype=np.float32)
    lib().kqo_build_blocks16(P16.ctypes.data, nb16, K.ctypes.data)
    return K


def dequant_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 codes [n, d/2] + scales [n, d/32] -> fp64 values [n, d]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    n, d = codes.shape[0], codes.shape[1] * 2
    out = np.empty((n, d), dtype=np.float64)
    lib().kqo_dequant_rows(codes.ctypes.data, scales.ctypes.data, n, d, out.ctypes.data)
    return out


def gemm_mx(a_codes, a_scales, b_codes, b_scales) -> np.ndarray:
    """Y = deq(A) deq(B)^T in fp64 (A [M, K] and B [N, K] as MXFP4 codes and scales).
    The dequantized products are exact in fp64; the sum is a BLAS fp64 matmul."""
    return dequant_rows(a_codes, a_scales) @ dequant_rows(b_codes, b_scales).T


def row_stats(X: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """LayerNorm statistics float32 [T, 2] = (mean, rstd) per row (fp64 sums, channel order)."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    T, d = X.shape
    st = np.zeros((T, 2), dtype=np.float32)
    if lib().kqo_row_stats(X.ctypes.data, T, d, float(eps), st.ctypes.data) != 0:
        raise ValueError("oracle rejected its arguments")
    return st


def adaln_rows(X: np.ndarray, stats=None, mscale=None, mshift=None, tokens_per_sample: int | None = None) -> np.ndarray:
    """The modulated activation as bf16 bits [T, d] (fp32 steps: centre, scale by rstd,
    times (1 + scale), plus shift; then round to bf16)."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    T, d = X.shape
    tps = T if tokens_per_sample is None else int(tokens_per_sample)
    cvt = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float32)
    st, ms, mh = cvt(stats), cvt(mscale), cvt(mshift)
    out = np.zeros((T, d), dtype=np.uint16)
    rc = lib().kqo_adaln_rows(X.ctypes.data, T, d, None if st is None else st.ctypes.data,
                              None if ms is None else ms.ctypes.data, None if mh is None else mh.ctypes.data,
                              max(tps, 1), out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out


# E2M1 magnitudes by code index (OCP MX v1.0 FP4 E2M1)
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """[.., d/2] packed bytes -> [.., d] 4-bit codes (even element in the low nibble)."""
    lo = codes & 0x0F
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
