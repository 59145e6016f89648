"""The C ABI without a GPU: the library loads, exports what include/kq.h
declares, and rejects bad arguments before making any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kq.h")
LIB = os.path.join(ROOT, "w4a4_diffusion_transformer_amd", "libkq.so")

KQ_OK, KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_VARIANT, KQ_ERR_HIP, KQ_ERR_ALIAS = range(7)


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libkq.so not built")
    L = ctypes.CDLL(LIB)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.kq_quantize.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    L.kq_quantize_ex.argtypes = [vp, i64, i64, vp, i64, vp, ci, vp, vp, vp]
    L.kq_build_blocks.argtypes = [vp, i64, vp, vp, ci, vp]
    L.kq_mx_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
    L.kq_smooth_quantize.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    L.kq_hadamard_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
    L.kq_transform_f32.argtypes = [ci, vp, i64, i64, vp, i64, vp, ci, vp, vp, vp, vp, vp]
    L.kq_row_stats.argtypes = [vp, i64, i64, ctypes.c_float, vp, vp]
    L.kq_quantize_adaln.argtypes = [vp, i64, i64, vp, vp, vp, i64, vp, i64, vp, ci, vp, vp, vp]
    L.kq_status_str.restype = ctypes.c_char_p
    return L


def test_header_declares_expected_entry_points():
    names = declared()
    for n in ("kq_build_blocks", "kq_quantize", "kq_quantize_ex", "kq_mx_quantize", "kq_smooth_quantize",
              "kq_hadamard_quantize", "kq_transform_f32", "kq_status_str", "kq_abi_version", "kq_row_stats",
              "kq_quantize_adaln"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in declared():
        assert n in exported, n
        assert hasattr(lib, n)


def test_version_and_status_strings(lib):
    hdr = open(HEADER).read()
    assert lib.kq_abi_version() == int(re.search(r"#define KQ_ABI_VERSION (\d+)", hdr).group(1))
    for s in range(7):
        assert lib.kq_status_str(s)
    assert lib.kq_status_str(99) == b"unknown status"


A = 0x100000  # aligned fake device addresses: every call below must return before touching HIP
B = 0x200000
C = 0x300000
D = 0x400000


def test_quantize_argument_checks(lib):
    assert lib.kq_quantize(A, 4, 48, B, C, D, None) == KQ_ERR_SHAPE
    assert lib.kq_quantize(A, 4, 0, B, C, D, None) == KQ_ERR_SHAPE
    assert lib.kq_quantize(A, -1, 64, B, C, D, None) == KQ_ERR_SHAPE
    assert lib.kq_quantize(A, 1 << 28, 64, B, C, D, None) == KQ_ERR_SHAPE
    assert lib.kq_quantize(A, 4, (1 << 24) + 32, B, C, D, None) == KQ_ERR_SHAPE
    assert lib.kq_quantize(None, 4, 64, B, C, D, None) == KQ_ERR_NULL
    assert lib.kq_quantize(A, 4, 64, None, C, D, None) == KQ_ERR_NULL
    assert lib.kq_quantize(A, 4, 64, B, None, D, None) == KQ_ERR_NULL
    assert lib.kq_quantize(A, 4, 64, B, C, None, None) == KQ_ERR_NULL
    assert lib.kq_quantize(A + 2, 4, 64, B, C, D, None) == KQ_ERR_ALIGN
    assert lib.kq_quantize(A, 4, 64, B + 2, C, D, None) == KQ_ERR_ALIGN
    assert lib.kq_quantize(A, 4, 64, B, C + 8, D, None) == KQ_ERR_ALIGN
    assert lib.kq_quantize(A, 4, 64, B, A, D, None) == KQ_ERR_ALIAS
    assert lib.kq_quantize(A, 4, 64, B, C, C + 64, None) == KQ_ERR_ALIAS  # scales inside codes
    assert lib.kq_quantize(A, 4, 64, B, C, B + 4, None) == KQ_ERR_ALIAS  # scales over the parameters
    assert lib.kq_quantize(A, 0, 64, B, C, D, None) == KQ_OK
    assert lib.kq_quantize(None, 0, 64, None, None, None, None) == KQ_OK


def test_quantize_ex_variant_checks(lib):
    assert lib.kq_quantize_ex(A, 4, 64, B, 7, None, 0, C, D, None) == KQ_ERR_SHAPE
    assert lib.kq_quantize_ex(A, 4, 64, B, 15, None, 9, C, D, None) == KQ_ERR_VARIANT
    assert lib.kq_quantize_ex(A, 4, 64, B, 15, None, 1, C, D, None) == KQ_ERR_VARIANT  # dense needs K_bf16
    assert lib.kq_quantize_ex(A, 4, 64, None, 15, B, 2, C, D, None) == KQ_ERR_VARIANT  # otf needs params
    assert lib.kq_quantize_ex(A, 4, 64, None, 15, None, 0, C, D, None) == KQ_ERR_VARIANT
    assert lib.kq_quantize_ex(A, 4, 64, None, 15, B + 8, 1, C, D, None) == KQ_ERR_ALIGN


def test_comparison_entry_checks(lib):
    assert lib.kq_mx_quantize(A, 4, 33, C, D, None) == KQ_ERR_SHAPE
    assert lib.kq_mx_quantize(A, 4, 64, C, C, None) == KQ_ERR_ALIAS
    assert lib.kq_smooth_quantize(A, 4, 64, None, C, D, None) == KQ_ERR_NULL
    assert lib.kq_smooth_quantize(A, 4, 64, B + 4, C, D, None) == KQ_ERR_ALIGN
    assert lib.kq_hadamard_quantize(A, 4, 64, None, D, None) == KQ_ERR_NULL
    assert lib.kq_transform_f32(0, A, 4, 64, B, 15, None, 0, None, None, C, D, None) == KQ_ERR_NULL
    assert lib.kq_transform_f32(7, A, 4, 64, B, 15, None, 0, None, D + 4096, C, D, None) == KQ_ERR_VARIANT
    assert lib.kq_transform_f32(1, A, 4, 64, None, 15, None, 0, None, A, C, D, None) == KQ_ERR_ALIAS


def test_auto_variant_rule(lib):
    lib.kq_auto_variant.restype = ctypes.c_int
    lib.kq_auto_variant.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
    assert lib.kq_auto_variant(4608, 12288, 1, 0) in (1, 2, 3)
    assert lib.kq_auto_variant(4608, 12288, 0, 1) == 1
    assert lib.kq_auto_variant(4608, 12288, 0, 0) == 0


def test_build_blocks_checks(lib):
    assert lib.kq_build_blocks(B, 0, C, None, 3, None) == KQ_ERR_SHAPE
    assert lib.kq_build_blocks(B, 4, None, C, 4, None) == KQ_ERR_SHAPE
    assert lib.kq_build_blocks(B, 4, None, None, 3, None) == KQ_ERR_NULL
    assert lib.kq_build_blocks(None, 4, C, None, 3, None) == KQ_ERR_NULL
    assert lib.kq_build_blocks(B, 4, C, D + 2, 3, None) == KQ_ERR_ALIGN
    assert lib.kq_build_blocks(B, 4, B, None, 3, None) == KQ_ERR_ALIAS


def test_binding_raises_without_gpu_tensors():
    import torch

    import w4a4_diffusion_transformer_amd as kq

    X = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kq.kq_mx_quantize(X, X, X)


E = 0x500000
F = 0x600000
G = 0x700000


def test_row_stats_argument_checks(lib):
    assert lib.kq_row_stats(A, 4, 48, 1e-6, B, None) == KQ_ERR_SHAPE
    assert lib.kq_row_stats(A, 4, 64, -1.0, B, None) == KQ_ERR_SHAPE
    assert lib.kq_row_stats(A, 4, 64, float("nan"), B, None) == KQ_ERR_SHAPE
    assert lib.kq_row_stats(A, 0, 64, 1e-6, None, None) == KQ_OK
    assert lib.kq_row_stats(None, 4, 64, 1e-6, B, None) == KQ_ERR_NULL
    assert lib.kq_row_stats(A, 4, 64, 1e-6, None, None) == KQ_ERR_NULL
    assert lib.kq_row_stats(A + 2, 4, 64, 1e-6, B, None) == KQ_ERR_ALIGN
    assert lib.kq_row_stats(A, 4, 64, 1e-6, B + 4, None) == KQ_ERR_ALIGN


def test_stream_probe_argument_checks(lib):
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.kq_stream_probe.argtypes = [vp, i64, i64, vp, vp, vp]
    p = lib.kq_stream_probe
    assert p(A, 4, 48, C, D, None) == KQ_ERR_SHAPE
    assert p(A, -1, 64, C, D, None) == KQ_ERR_SHAPE
    assert p(None, 4, 64, C, D, None) == KQ_ERR_NULL
    assert p(A, 4, 64, C, None, None) == KQ_ERR_NULL
    assert p(A + 2, 4, 64, C, D, None) == KQ_ERR_ALIGN
    assert p(A, 4, 64, C + 8, D, None) == KQ_ERR_ALIGN
    assert p(A, 4, 64, A + 16, D, None) == KQ_ERR_ALIAS
    assert p(A, 0, 64, None, None, None) == KQ_OK
    assert lib.kq_row_stats(A, 4, 64, 1e-6, A + 8, None) == KQ_ERR_ALIAS


def test_quantize_adaln_argument_checks(lib):
    q = lib.kq_quantize_adaln
    # tokens_per_sample must be positive and a multiple of 32 unless it covers every row
    assert q(A, 100, 64, B, C, D, 0, E, 15, None, 0, F, G, None) == KQ_ERR_SHAPE
    assert q(A, 100, 64, B, C, D, 40, E, 15, None, 0, F, G, None) == KQ_ERR_SHAPE
    assert q(A, 100, 64, B, C, D, 64, E, 7, None, 0, F, G, None) == KQ_ERR_SHAPE
    assert q(A, 100, 64, B, C, D, 64, E, 15, None, -1, F, G, None) == KQ_ERR_VARIANT
    assert q(A, 100, 64, B, C, D, 64, E, 15, None, 9, F, G, None) == KQ_ERR_VARIANT
    assert q(A, 0, 64, None, None, None, 64, None, 15, None, 0, None, None, None) == KQ_OK
    assert q(A, 100, 64, B, C, D, 64, None, 15, None, 0, F, G, None) == KQ_ERR_VARIANT
    assert q(A, 100, 64, B, C, D, 64, E, 15, None, 1, F, G, None) == KQ_ERR_VARIANT
    assert q(None, 100, 64, B, C, D, 64, E, 15, None, 0, F, G, None) == KQ_ERR_NULL
    assert q(A, 100, 64, B + 4, C, D, 64, E, 15, None, 0, F, G, None) == KQ_ERR_ALIGN
    assert q(A, 100, 64, B, C + 2, D, 64, E, 15, None, 0, F, G, None) == KQ_ERR_ALIGN
    # the modulation vectors are read 16 bytes at a time
    assert q(A, 100, 64, B, C + 4, D, 64, E, 15, None, 0, F, G, None) == KQ_ERR_ALIGN
    assert q(A, 100, 64, B, C, D + 8, 64, E, 15, None, 0, F, G, None) == KQ_ERR_ALIGN
    # an output overlapping the statistics or a modulation vector
    assert q(A, 100, 64, B, C, D, 64, E, 15, None, 0, B + 64, G, None) == KQ_ERR_ALIAS
    assert q(A, 100, 64, B, C, D, 64, E, 15, None, 0, F, D + 16, None) == KQ_ERR_ALIAS


def test_variant_entry_checks(lib):
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.kq_hadamard_quantize_ex.argtypes = [vp, i64, i64, ci, vp, vp, vp]
    lib.kq_build_blocks16.argtypes = [vp, i64, vp, vp, ci, vp]
    h = lib.kq_hadamard_quantize_ex
    for block in (16, 48, 1024, 0, -32):
        assert h(A, 4, 1024, block, C, D, None) == KQ_ERR_SHAPE
    assert h(A, 4, 1152, 256, C, D, None) == KQ_ERR_SHAPE  # d not a multiple of the block
    assert h(A, 0, 1024, 512, None, None, None) == KQ_OK
    assert h(None, 4, 1024, 512, C, D, None) == KQ_ERR_NULL
    b = lib.kq_build_blocks16
    assert b(A, 3, B, None, 3, None) == KQ_ERR_SHAPE  # odd block count
    assert b(A, 0, B, None, 3, None) == KQ_ERR_SHAPE
    assert b(A, 4, None, C, 4, None) == KQ_ERR_SHAPE
    assert b(None, 4, B, None, 3, None) == KQ_ERR_NULL
    assert b(A, 4, None, None, 3, None) == KQ_ERR_NULL
    assert b(A + 2, 4, B, None, 3, None) == KQ_ERR_ALIGN
    assert b(A, 4, A + 64, None, 3, None) == KQ_ERR_ALIAS


def test_tune_argument_checks(lib):
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.kq_tune.argtypes = [vp, i64, i64, vp, vp, vp, vp, ci, ctypes.POINTER(ci), vp]
    lib.kq_tune_reset.restype = None
    chosen = ctypes.c_int(-1)
    t = lib.kq_tune
    assert t(A, 4, 48, B, None, C, D, 5, ctypes.byref(chosen), None) == KQ_ERR_SHAPE
    assert t(A, 4, 64, B, None, C, D, 0, ctypes.byref(chosen), None) == KQ_ERR_SHAPE
    assert t(A, 4, 64, None, None, C, D, 5, ctypes.byref(chosen), None) == KQ_ERR_VARIANT
    assert t(None, 4, 64, B, None, C, D, 5, ctypes.byref(chosen), None) == KQ_ERR_NULL
    assert t(A + 2, 4, 64, B, None, C, D, 5, ctypes.byref(chosen), None) == KQ_ERR_ALIGN
    assert t(A, 4, 64, B, None, A + 16, D, 5, ctypes.byref(chosen), None) == KQ_ERR_ALIAS
    assert t(A, 0, 64, B, None, C, D, 5, ctypes.byref(chosen), None) == KQ_OK
    assert chosen.value == 3  # no tuning recorded: the default rule (the butterfly kernel)
    lib.kq_tune_reset()
