"""Exact E8M0 scales where the transform's rounding would decide them, and the
hardware E2M1 convert against the oracle's rounding rule, on an MI355X.

1. Blocks whose exact amax lies within 2^-20 of a power of two, on both sides
   (tests/near_blocks.py, confirmed by the oracle): every KroQuant variant and
   the block-Hadamard front-end at every block size must return the oracle's
   scale bytes exactly.  An fp32 transform alone gets a share of these wrong
   (tests/test_near_blocks.py shows one order of summation that does); the
   kernels decide them from exact values.
2. The scaled FP4 convert the kernels use for E2M1 rounding, through the
   SmoothQuant front-end with x = 2^k (so y = m[c] 2^k exactly): fp32 values
   swept through every rounding midpoint of the E2M1 grid (every fp32 within
   2^12 ulps of each midpoint) and random fp32 values, at scale bytes from 0
   to 251, codes and scales bit-exact against the oracle's OCP MX v1.0 rule
   (Pith review, reference [10]).
"""
import numpy as np
import pytest
import torch

import near_blocks as nbk
import oracle
import synth
from oracle.compare import compare

kq = pytest.importorskip("w4a4_diffusion_transformer_amd")

pytestmark = pytest.mark.gpu

VARIANTS = {"mfma_dense": 1, "mfma_otf": 2, "butterfly": 3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kq.lib()
    yield


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


@pytest.fixture(scope="module")
def kron_near():
    cases = {}
    for name, (T, nb, seed, sigma) in {"sigma0.1": (24, 36, 11, 0.1), "sigma0.5": (8, 96, 12, 0.5)}.items():
        X, P, near = nbk.near_matrix_kron(T, nb, seed, sigma)
        ref = oracle.quantize_rows(oracle.KRON, X, P, want_y=True)
        cases[name] = (X, P, near, ref)
    return cases


@pytest.mark.parametrize("case", ["sigma0.1", "sigma0.5"])
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_kron_scales_exact_near_powers_of_two(kron_near, case, variant):
    X, P, near, ref = kron_near[case]
    assert near.sum() >= 0.95 * near.size
    Xd, Pd = dev(X), dev(P)
    nb = P.shape[0]
    Kbf = None
    if variant == "mfma_dense":
        Kbf = torch.empty((nb, 3, 32, 32), dtype=torch.int16, device="cuda:0")
        kq.kq_build_blocks(Pd, nb, None, Kbf, 3)
    Pin = None if variant == "mfma_dense" else Pd
    for want_y in (False, True):
        codes, scales = kq.alloc_outputs(Xd)
        if want_y:
            Y = torch.empty(X.shape, dtype=torch.float32, device="cuda:0")
            kq.kq_transform_f32(kq.KQ_FRONT_KRON, Xd, Pin, 15, Kbf, VARIANTS[variant], None, Y, codes, scales)
        else:
            kq.kq_quantize_ex(Xd, Pin, 15, Kbf, VARIANTS[variant], codes, scales)
        torch.cuda.synchronize()
        c, s = codes.cpu().numpy(), scales.cpu().numpy()
        np.testing.assert_array_equal(s, ref["scales"], err_msg=f"{variant} {case} want_y={want_y}")

        def yh(rows):
            return ref["yhat"][rows], ref["y32"][rows]

        rep = compare(c, s, ref["codes"], ref["scales"], yh)
        print(f"{variant} {case}: {int(near.sum())} blocks within 2^-20 of a power of two; {rep}")
        assert rep.code_unexplained == 0, str(rep)
        if want_y:
            # the quantizer applied to the kernel's own y gives its codes and scales
            c2, s2 = oracle.quantize_f32_rows(Y.cpu().numpy())
            np.testing.assert_array_equal(s2, s)
            np.testing.assert_array_equal(c2, c)


@pytest.mark.parametrize("B", [32, 64, 128, 256, 512])
def test_hadamard_scales_exact_near_powers_of_two(B):
    X, near = nbk.near_matrix_hadamard(16, 2048, B, seed=100 + B)
    assert near[:, ::B // 32].sum() >= 0.95 * near[:, ::B // 32].size
    ref = oracle.quantize_rows_hadamard(X, B, want_y=True)
    Xd = dev(X)
    codes, scales = kq.alloc_outputs(Xd)
    kq.kq_hadamard_quantize_ex(Xd, B, codes, scales)
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    np.testing.assert_array_equal(s, ref["scales"])

    def yh(rows):
        return ref["yhat"][rows], ref["y32"][rows]

    rep = compare(c, s, ref["codes"], ref["scales"], yh)
    assert rep.code_unexplained == 0, str(rep)


@pytest.mark.parametrize("B", [64, 512])
def test_hadamard_exact_path_wide_exponent_range(B):
    """Near-power-of-two Hadamard blocks whose inputs also hold values of about 2^-100: the exponent
    range then exceeds what makes every fp64 partial sum exact, so the kernel takes the sequential
    fp64 sum over the Hadamard block instead of the fp64 butterflies; scales must still equal the
    oracle's, and codes differ only at classified ties."""
    X, near = nbk.near_matrix_hadamard(16, 2048, B, seed=300 + B)
    X = X.copy()
    tiny = synth.f32_to_bf16(np.array([2.0 ** -100, -(2.0 ** -100)], dtype=np.float32))
    X[:, 5::97] = tiny[0]  # one or two tiny inputs in every Hadamard block, far from the block amax
    X[:, 11::131] = tiny[1]
    ref = oracle.quantize_rows_hadamard(X, B, want_y=True)
    Xd = dev(X)
    codes, scales = kq.alloc_outputs(Xd)
    kq.kq_hadamard_quantize_ex(Xd, B, codes, scales)
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    np.testing.assert_array_equal(s, ref["scales"])

    def yh(rows):
        return ref["yhat"][rows], ref["y32"][rows]

    rep = compare(c, s, ref["codes"], ref["scales"], yh)
    assert rep.code_unexplained == 0, str(rep)


def convert_sweep_values(rng) -> np.ndarray:
    """fp32 values in (-8, 8): every fp32 within 2^12 ulps of each E2M1 midpoint
    (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5), each grid value +- a few ulps, and
    random fp32 bit patterns in (0, 8); signs alternate."""
    parts = []
    for mid in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):
        b = np.float32(mid).view(np.uint32).astype(np.int64)
        parts.append(np.arange(b - 4096, b + 4096, dtype=np.int64).astype(np.uint32).view(np.float32))
    for g in (0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0):
        b = np.float32(g).view(np.uint32).astype(np.int64)
        parts.append(np.arange(b - 8, b + 8, dtype=np.int64).astype(np.uint32).view(np.float32))
    top = np.float32(8.0).view(np.uint32)
    parts.append(rng.integers(1, int(top), 200000, dtype=np.uint32).view(np.float32))
    v = np.concatenate(parts)
    v = v[(v > 0) & (v < 8)]
    v[1::2] = -v[1::2]
    return v


def test_fp4_convert_matches_the_e2m1_rule_at_every_scale():
    rng = np.random.default_rng(5)
    v = convert_sweep_values(rng)
    nblk = (len(v) + 30) // 31
    m = np.zeros(32 * nblk, dtype=np.float32)
    mb = m.reshape(nblk, 32)
    mb[:, 0] = 4.0  # sets every block's scale to 2^k on a row with x = 2^k
    flat = np.zeros(nblk * 31, dtype=np.float32)
    flat[:len(v)] = v
    mb[:, 1:] = flat.reshape(nblk, 31)
    # rows x = 2^k: scale bytes 0 (k = -127, -128 and below share byte 0) .. 251 (k = 124)
    ks = [-133, -128, -127, -126, -125, -124, -100, -60, -20, -3, -1, 0, 1, 2, 7, 30, 70, 110, 123, 124]
    X = synth.f32_to_bf16(np.array([[2.0 ** k] for k in ks], dtype=np.float64).astype(np.float32)
                          * np.ones((1, m.size), dtype=np.float32))
    ref = oracle.quantize_rows(oracle.SMOOTH, X, m=m)
    Xd, md = dev(X), dev(m)
    codes, scales = kq.alloc_outputs(Xd)
    kq.kq_smooth_quantize(Xd, md, codes, scales)
    torch.cuda.synchronize()
    s = scales.cpu().numpy()
    assert s[ks.index(124)].max() == 251 and s[ks.index(-127)].max() == 0
    np.testing.assert_array_equal(s, ref["scales"])
    np.testing.assert_array_equal(codes.cpu().numpy(), ref["codes"])
