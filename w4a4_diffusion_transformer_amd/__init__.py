"""Python binding of libkq, the gfx950 KroQuant online activation quantizer.

Thin ctypes layer over the C ABI declared in ``include/kq.h``: each function
has the C entry point's name and only marshals arguments (tensor -> device
pointer, current torch stream -> hipStream_t) and turns a status code into an
exception.  All computation happens in the HIP kernels.  PyTorch supplies
device memory and streams.  There is no fallback: if ``libkq.so`` is missing
or a tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "KQError", "KQ_AUTO", "KQ_MFMA_DENSE", "KQ_MFMA_OTF", "KQ_BUTTERFLY",
    "KQ_FRONT_KRON", "KQ_FRONT_PLAIN", "KQ_FRONT_SMOOTH", "KQ_FRONT_HADAMARD",
    "lib", "kq_abi_version", "kq_status_str", "kq_build_blocks", "kq_quantize", "kq_quantize_ex",
    "kq_mx_quantize", "kq_smooth_quantize", "kq_hadamard_quantize", "kq_transform_f32",
    "alloc_outputs", "LIB_PATH", "kq_auto_variant", "variant_name", "kq_row_stats", "kq_quantize_adaln",
    "kq_build_blocks_inverse_t", "kq_gemm_mx", "kq_hadamard_quantize_ex", "kq_build_blocks16", "kq_tune",
    "kq_tune_reset", "kq_stream_probe",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkq.so")

KQ_AUTO, KQ_MFMA_DENSE, KQ_MFMA_OTF, KQ_BUTTERFLY = 0, 1, 2, 3
KQ_FRONT_KRON, KQ_FRONT_PLAIN, KQ_FRONT_SMOOTH, KQ_FRONT_HADAMARD = 0, 1, 2, 3
VARIANTS = {"auto": KQ_AUTO, "mfma_dense": KQ_MFMA_DENSE, "mfma_otf": KQ_MFMA_OTF, "butterfly": KQ_BUTTERFLY}

_lib = None


class KQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {kq_status_str(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libkq.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build the HIP library first (__graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.kq_abi_version.argtypes = []
        L.kq_abi_version.restype = ci
        L.kq_status_str.argtypes = [ci]
        L.kq_status_str.restype = ctypes.c_char_p
        L.kq_build_blocks.argtypes = [vp, i64, vp, vp, ci, vp]
        L.kq_quantize.argtypes = [vp, i64, i64, vp, vp, vp, vp]
        L.kq_quantize_ex.argtypes = [vp, i64, i64, vp, i64, vp, ci, vp, vp, vp]
        L.kq_mx_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
        L.kq_stream_probe.argtypes = [vp, i64, i64, vp, vp, vp]
        L.kq_smooth_quantize.argtypes = [vp, i64, i64, vp, vp, vp, vp]
        L.kq_hadamard_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
        L.kq_transform_f32.argtypes = [ci, vp, i64, i64, vp, i64, vp, ci, vp, vp, vp, vp, vp]
        L.kq_auto_variant.argtypes = [i64, i64, ci, ci]
        L.kq_auto_variant.restype = ci
        L.kq_row_stats.argtypes = [vp, i64, i64, ctypes.c_float, vp, vp]
        L.kq_build_blocks_inverse_t.argtypes = [vp, i64, vp, vp, ci, vp]
        L.kq_gemm_mx.argtypes = [vp, vp, i64, vp, vp, i64, i64, vp, vp, vp]
        L.kq_hadamard_quantize_ex.argtypes = [vp, i64, i64, ci, vp, vp, vp]
        L.kq_build_blocks16.argtypes = [vp, i64, vp, vp, ci, vp]
        L.kq_tune.argtypes = [vp, i64, i64, vp, vp, vp, vp, ci, ctypes.POINTER(ci), vp]
        L.kq_tune_reset.argtypes = []
        L.kq_tune_reset.restype = None
        L.kq_quantize_adaln.argtypes = [vp, i64, i64, vp, vp, vp, i64, vp, i64, vp, ci, vp, vp, vp]
        for name in ("kq_build_blocks", "kq_quantize", "kq_quantize_ex", "kq_mx_quantize", "kq_stream_probe",
                     "kq_smooth_quantize",
                     "kq_hadamard_quantize", "kq_transform_f32", "kq_row_stats", "kq_quantize_adaln",
                     "kq_build_blocks_inverse_t", "kq_gemm_mx", "kq_hadamard_quantize_ex", "kq_build_blocks16", "kq_tune"):
            getattr(L, name).restype = ci
        _lib = L
    return _lib


def kq_abi_version() -> int:
    return int(lib().kq_abi_version())


def kq_auto_variant(tokens: int, d: int, has_params: bool = True, has_split: bool = False) -> int:
    return int(lib().kq_auto_variant(tokens, d, int(has_params), int(has_split)))


def variant_name(v: int) -> str:
    return {v_: k for k, v_ in VARIANTS.items()}[int(v)]


def kq_status_str(status: int) -> str:
    return lib().kq_status_str(int(status)).decode()


def _ptr(t, what: str, dtype=None):
    """Device pointer of a tensor (or None / a raw integer address)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{what}: tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")
    if dtype is not None and t.dtype not in dtype:
        raise TypeError(f"{what}: dtype {t.dtype} not in {dtype}")
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8,)
_F32 = (torch.float32,)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int, where: str):
    if status != 0:
        raise KQError(status, where)


def _shape(X):
    if X.dim() != 2:
        raise ValueError("X must be 2-D [tokens, d]")
    return X.shape[0], X.shape[1]


def alloc_outputs(X: torch.Tensor):
    """Empty (codes [T, d/2] uint8, scales [T, d/32] uint8) on X's device."""
    T, d = _shape(X)
    return (torch.empty((T, d // 2), dtype=torch.uint8, device=X.device),
            torch.empty((T, d // 32), dtype=torch.uint8, device=X.device))


def kq_build_blocks(K_params, nb: int, K_f32=None, K_bf16=None, n_split: int = 3, stream=None):
    _check(lib().kq_build_blocks(_ptr(K_params, "K_params", _F32), nb, _ptr(K_f32, "K_f32", _F32),
                                 _ptr(K_bf16, "K_bf16", _BF16), n_split, _stream(stream)), "kq_build_blocks")
    return K_f32, K_bf16


def kq_quantize(X, K_params, out_codes, out_scales, stream=None):
    T, d = _shape(X)
    _check(lib().kq_quantize(_ptr(X, "X", _BF16), T, d, _ptr(K_params, "K_params", _F32),
                             _ptr(out_codes, "out_codes", _U8), _ptr(out_scales, "out_scales", _U8),
                             _stream(stream)), "kq_quantize")
    return out_codes, out_scales


def kq_quantize_ex(X, K_params, params_block_stride: int, K_bf16, variant: int, out_codes, out_scales,
                   stream=None):
    T, d = _shape(X)
    _check(lib().kq_quantize_ex(_ptr(X, "X", _BF16), T, d, _ptr(K_params, "K_params", _F32),
                                params_block_stride, _ptr(K_bf16, "K_bf16", _BF16), int(variant),
                                _ptr(out_codes, "out_codes", _U8), _ptr(out_scales, "out_scales", _U8),
                                _stream(stream)), "kq_quantize_ex")
    return out_codes, out_scales


def kq_mx_quantize(X, out_codes, out_scales, stream=None):
    T, d = _shape(X)
    _check(lib().kq_mx_quantize(_ptr(X, "X", _BF16), T, d, _ptr(out_codes, "out_codes", _U8),
                                _ptr(out_scales, "out_scales", _U8), _stream(stream)), "kq_mx_quantize")
    return out_codes, out_scales


def kq_stream_probe(X, out_codes, out_scales, stream=None):
    """Measurement only: the default quantizer's memory traffic with no arithmetic (outputs are a digest)."""
    T, d = _shape(X)
    _check(lib().kq_stream_probe(_ptr(X, "X", _BF16), T, d, _ptr(out_codes, "out_codes", _U8),
                                 _ptr(out_scales, "out_scales", _U8), _stream(stream)), "kq_stream_probe")
    return out_codes, out_scales


def kq_smooth_quantize(X, ch_mult, out_codes, out_scales, stream=None):
    T, d = _shape(X)
    _check(lib().kq_smooth_quantize(_ptr(X, "X", _BF16), T, d, _ptr(ch_mult, "ch_mult", _F32),
                                    _ptr(out_codes, "out_codes", _U8), _ptr(out_scales, "out_scales", _U8),
                                    _stream(stream)), "kq_smooth_quantize")
    return out_codes, out_scales


def kq_hadamard_quantize(X, out_codes, out_scales, stream=None):
    T, d = _shape(X)
    _check(lib().kq_hadamard_quantize(_ptr(X, "X", _BF16), T, d, _ptr(out_codes, "out_codes", _U8),
                                      _ptr(out_scales, "out_scales", _U8), _stream(stream)),
           "kq_hadamard_quantize")
    return out_codes, out_scales


def kq_transform_f32(front: int, X, K_params=None, params_block_stride: int = 15, K_bf16=None,
                     variant: int = KQ_AUTO, ch_mult=None, Y=None, out_codes=None, out_scales=None, stream=None):
    T, d = _shape(X)
    _check(lib().kq_transform_f32(int(front), _ptr(X, "X", _BF16), T, d, _ptr(K_params, "K_params", _F32),
                                  params_block_stride, _ptr(K_bf16, "K_bf16", _BF16), int(variant),
                                  _ptr(ch_mult, "ch_mult", _F32), _ptr(Y, "Y", _F32),
                                  _ptr(out_codes, "out_codes", _U8), _ptr(out_scales, "out_scales", _U8),
                                  _stream(stream)), "kq_transform_f32")
    return Y, out_codes, out_scales


def kq_row_stats(X, eps: float, row_stats, stream=None):
    """LayerNorm (mean, rstd) per row into row_stats (float32 [tokens, 2])."""
    T, d = _shape(X)
    _check(lib().kq_row_stats(_ptr(X, "X", _BF16), T, d, float(eps), _ptr(row_stats, "row_stats", _F32),
                              _stream(stream)), "kq_row_stats")
    return row_stats


def kq_quantize_adaln(X, row_stats, mod_scale, mod_shift, tokens_per_sample: int, K_params, out_codes, out_scales,
                      params_block_stride: int = 15, K_bf16=None, variant: int = KQ_AUTO, stream=None):
    """Fused LayerNorm-normalise + AdaLN-modulate + transform + MXFP4 (any of the first three inputs may be None)."""
    T, d = _shape(X)
    _check(lib().kq_quantize_adaln(_ptr(X, "X", _BF16), T, d, _ptr(row_stats, "row_stats", _F32),
                                   _ptr(mod_scale, "mod_scale", _F32), _ptr(mod_shift, "mod_shift", _F32),
                                   int(tokens_per_sample), _ptr(K_params, "K_params", _F32), params_block_stride,
                                   _ptr(K_bf16, "K_bf16", _BF16), int(variant), _ptr(out_codes, "out_codes", _U8),
                                   _ptr(out_scales, "out_scales", _U8), _stream(stream)), "kq_quantize_adaln")
    return out_codes, out_scales


def kq_build_blocks_inverse_t(K_params, nb: int, K_f32=None, K_bf16=None, n_split: int = 3, stream=None):
    """Blocks K^-T of the weight fold (fp32 [nb,32,32] and/or transposed bf16 split [nb,n_split,32,32])."""
    _check(lib().kq_build_blocks_inverse_t(_ptr(K_params, "K_params", _F32), nb, _ptr(K_f32, "K_f32", _F32),
                                           _ptr(K_bf16, "K_bf16", _BF16), n_split, _stream(stream)),
           "kq_build_blocks_inverse_t")
    return K_f32, K_bf16


def kq_gemm_mx(a_codes, a_scales, b_codes, b_scales, y_f32=None, y_bf16=None, stream=None):
    """Y = deq(A) deq(B)^T: A codes [M, K/2] + scales [M, K/32], B codes [N, K/2] + scales [N, K/32]."""
    M, N = a_codes.shape[0], b_codes.shape[0]
    K = a_codes.shape[1] * 2
    if b_codes.shape[1] * 2 != K:
        raise ValueError("A and B must have the same K")
    _check(lib().kq_gemm_mx(_ptr(a_codes, "a_codes", _U8), _ptr(a_scales, "a_scales", _U8), M,
                            _ptr(b_codes, "b_codes", _U8), _ptr(b_scales, "b_scales", _U8), N, K,
                            _ptr(y_f32, "y_f32", _F32), _ptr(y_bf16, "y_bf16", _BF16), _stream(stream)),
           "kq_gemm_mx")
    return y_f32, y_bf16


def kq_hadamard_quantize_ex(X, block: int, out_codes, out_scales, stream=None):
    """Block-Hadamard (size 32..512) front-end + MXFP4."""
    T, d = _shape(X)
    _check(lib().kq_hadamard_quantize_ex(_ptr(X, "X", _BF16), T, d, int(block), _ptr(out_codes, "out_codes", _U8),
                                         _ptr(out_scales, "out_scales", _U8), _stream(stream)), "kq_hadamard_quantize_ex")
    return out_codes, out_scales


def kq_build_blocks16(K_params16, nb16: int, K_f32=None, K_bf16=None, n_split: int = 3, stream=None):
    """16-wide 4-factor blocks as block-diagonal 32x32 dense blocks (fp32 and/or transposed bf16 split)."""
    _check(lib().kq_build_blocks16(_ptr(K_params16, "K_params16", _F32), nb16, _ptr(K_f32, "K_f32", _F32),
                                   _ptr(K_bf16, "K_bf16", _BF16), n_split, _stream(stream)), "kq_build_blocks16")
    return K_f32, K_bf16


def kq_tune(X, K_params, K_bf16, out_codes, out_scales, reps: int = 10, stream=None) -> int:
    """Time the variants the inputs allow, record the fastest for KQ_AUTO at this shape; returns it."""
    T, d = _shape(X)
    chosen = ctypes.c_int(0)
    _check(lib().kq_tune(_ptr(X, "X", _BF16), T, d, _ptr(K_params, "K_params", _F32), _ptr(K_bf16, "K_bf16", _BF16),
                         _ptr(out_codes, "out_codes", _U8), _ptr(out_scales, "out_scales", _U8), int(reps),
                         ctypes.byref(chosen), _stream(stream)), "kq_tune")
    return chosen.value


def kq_tune_reset() -> None:
    lib().kq_tune_reset()
