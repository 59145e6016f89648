"""Pins for the CPU oracle: each check ties it to something other than itself.

The pages (the Pith review of arXiv 2607.21446 and the AIssential summary)
print no worked numeric example and ship no parameters, so the oracle is
pinned by what they and the mathematics fix:
  * the factor is an LU product with determinant 1 and a closed-form inverse
    (review, Sec. 3.2 Eq. (6) and the axiom ledger);
  * K = G1 (x) ... (x) G5: checked against numpy.kron, against sequential
    butterfly stages (mixed-product property), det K = 1, K^-1 K = I;
  * the Hadamard matrix is a Kronecker product of five identical 2x2 factors
    (review, core claim): checked against scipy.linalg.hadamard;
  * y = x K in the row-vector convention of Eq. (1): checked against a numpy
    fp64 matmul;
  * the E2M1/E8M0 rules (OCP MX v1.0, the review's reference [10]): brute-force
    nearest search over every fp32 magnitude below 8, hand-worked values in
    tests/golden/, and the defining property of the shared scale.
"""
import ctypes
import json
import os
import subprocess

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def rand_params(n, seed=11, sigma=0.3):
    return synth.random_params(n, seed=seed, sigma_lb=sigma, sigma_a=sigma)


def lu_factor_numpy(l, a, b):
    """G = L @ U built from the two printed factors, in fp64."""
    l, a, b = float(np.float32(l)), float(np.float32(a)), float(np.float32(b))
    L = np.array([[1.0, 0.0], [l, 1.0]])
    U = np.array([[a, b], [0.0, 1.0 / a]])
    return L @ U


# ---------------------------------------------------------------- factor


def test_factor_is_lu_product_with_unit_det():
    P = rand_params(40).reshape(-1, 3)
    for l, a, b in P:
        G = oracle.factor(l, a, b)
        np.testing.assert_allclose(G, lu_factor_numpy(l, a, b), rtol=1e-15, atol=1e-15)
        assert abs(np.linalg.det(G) - 1.0) < 1e-13
        Gi = oracle.factor_inverse(l, a, b)
        np.testing.assert_allclose(Gi @ G, np.eye(2), atol=1e-13)
        np.testing.assert_allclose(G @ Gi, np.eye(2), atol=1e-13)


def test_factor_identity_and_hadamard_like():
    np.testing.assert_array_equal(oracle.factor(0.0, 1.0, 0.0), np.eye(2))
    s = np.float32(1 / np.sqrt(2))
    G = oracle.factor(1.0, s, -s)
    # H2 diag(1, -1) / sqrt(2) = [[1, -1], [1, 1]] / sqrt(2)
    np.testing.assert_allclose(G, np.array([[1, -1], [1, 1]]) / np.sqrt(2), atol=1e-7)


# ---------------------------------------------------------------- Kronecker


def test_kron_matches_numpy_kron():
    P = rand_params(12, seed=3)
    for j in range(P.shape[0]):
        Gs = [lu_factor_numpy(*P[j, k]) for k in range(5)]
        ref = Gs[0]
        for G in Gs[1:]:
            ref = np.kron(ref, G)
        K = oracle.kron_dense(P[j])
        np.testing.assert_allclose(K, ref, rtol=1e-14, atol=1e-15 * np.abs(ref).max())


def test_kron_dense_equals_sequential_butterflies():
    P = rand_params(12, seed=5)
    for j in range(P.shape[0]):
        Kd, Kb = oracle.kron_dense(P[j]), oracle.kron_butterfly(P[j])
        assert np.abs(Kd - Kb).max() <= 1e-12 * np.abs(Kd).max()


def test_kron_det_and_inverse():
    P = rand_params(8, seed=7)
    for j in range(P.shape[0]):
        K = oracle.kron_dense(P[j])
        assert abs(np.linalg.det(K) - 1.0) < 1e-9
        assert abs(oracle.det(K) - 1.0) < 1e-9
        Ki = oracle.kron_inverse(P[j])
        assert np.abs(Ki @ K - np.eye(32)).max() < 1e-12
        K32 = oracle.block_f32(P[j]).astype(np.float32)
        Ki32 = Ki.astype(np.float32)
        assert np.abs(Ki32 @ K32 - np.eye(32, dtype=np.float32)).max() < 1e-5


def test_kron_identity_factors_give_identity():
    P = np.tile(np.array([0.0, 1.0, 0.0], dtype=np.float32), (5, 1))
    np.testing.assert_array_equal(oracle.kron_dense(P), np.eye(32))


def test_kron_hadamard_factors_give_signed_hadamard():
    """Five identical Hadamard-like factors give H32 D32 / sqrt(32), D32 = diag((-1)^popcount(c))."""
    s = np.float32(1 / np.sqrt(2))
    P = np.tile(np.array([1.0, s, -s], dtype=np.float32), (5, 1))
    H = scipy.linalg.hadamard(32).astype(np.float64)
    D = np.diag([(-1.0) ** bin(c).count("1") for c in range(32)])
    np.testing.assert_allclose(oracle.kron_dense(P), H @ D / np.sqrt(32), atol=1e-6)


def test_fwht_matches_scipy_hadamard():
    H = scipy.linalg.hadamard(32)
    np.testing.assert_array_equal(H @ H.T, 32 * np.eye(32))
    rng = np.random.default_rng(0)
    for _ in range(10):
        v = rng.integers(-1000, 1000, 32).astype(np.float64)
        np.testing.assert_array_equal(oracle.fwht32(v), v @ H)


# ---------------------------------------------------------------- dense blocks


def test_build_blocks_k32_and_split():
    P = rand_params(16, seed=13)
    K32, Kbf = oracle.build_blocks(P, 16)
    for j in range(16):
        np.testing.assert_array_equal(K32[j], oracle.kron_dense(P[j]).astype(np.float32))
        # split terms are RNE bf16 roundings (torch's float32 -> bfloat16 conversion) of the running rest
        rest = torch.from_numpy(K32[j].T.copy())
        total = torch.zeros_like(rest)
        for s in range(3):
            h = rest.to(torch.bfloat16)
            np.testing.assert_array_equal(Kbf[j, s], h.view(torch.int16).numpy().view(np.uint16))
            total = total + h.float()
            rest = rest - h.float()
        # three bf16 terms represent the fp32 block exactly
        np.testing.assert_array_equal(total.numpy(), K32[j].T)


def test_build_blocks_shared_stride_zero():
    P = rand_params(1, seed=17)
    K32, _ = oracle.build_blocks(P, 5, pstride=0)
    for j in range(5):
        np.testing.assert_array_equal(K32[j], K32[0])


# ---------------------------------------------------------------- E2M1 / E8M0


@pytest.fixture(scope="module")
def bruteforce_lib(tmp_path_factory):
    out = tmp_path_factory.mktemp("pins") / "libe2m1bf.so"
    src = os.path.join(ROOT, "tests", "pins", "e2m1_bruteforce.c")
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", src, "-o", str(out), "-lm"], check=True)
    L = ctypes.CDLL(str(out))
    L.e2m1_compare_range.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                     ctypes.POINTER(ctypes.c_uint32)]
    L.e2m1_compare_range.restype = ctypes.c_int64
    L.e2m1_nearest_even.argtypes = [ctypes.c_double]
    L.e2m1_nearest_even.restype = ctypes.c_int
    return L


def test_e2m1_exhaustive_against_bruteforce(bruteforce_lib):
    """Every positive fp32 below 8 (exponent field < 130), plus a stride over [8, max]."""
    fn = ctypes.cast(oracle.lib().kqo_e2m1_index, ctypes.c_void_p)
    first = ctypes.c_uint32(0)
    bad = bruteforce_lib.e2m1_compare_range(fn, 0, 130 << 23, 1, ctypes.byref(first))
    assert bad == 0, f"first mismatch at bits {first.value:#010x}"
    # fp64 distances stay exact while m < 2^50; check that range on a stride
    bad = bruteforce_lib.e2m1_compare_range(fn, 130 << 23, (127 + 50) << 23, 4099, ctypes.byref(first))
    assert bad == 0, f"first mismatch at bits {first.value:#010x}"
    # beyond it the direct search cannot resolve |m - 4| vs |m - 6|; saturation to 6 is the rule itself
    for bits in range((127 + 50) << 23, 0x7F800000, 1 << 20):
        m = float(np.array([bits], dtype=np.uint32).view(np.float32)[0])
        assert oracle.e2m1_index(m) == 7


def load_golden():
    with open(os.path.join(GOLDEN, "e2m1_e8m0_handworked.json")) as f:
        return json.load(f)


def _amax_of(case):
    if "amax_bits" in case:
        return float(np.array([int(case["amax_bits"], 16)], dtype=np.uint32).view(np.float32)[0])
    return float(np.float32(case["amax"]))


def test_e8m0_handworked():
    for case in load_golden()["scale_cases"]:
        assert oracle.e8m0(_amax_of(case)) == case["byte"], case


def test_e2m1_handworked(bruteforce_lib):
    for case in load_golden()["element_cases"]:
        v = float(np.float32(case["v"]))
        assert oracle.e2m1_index(v) == case["index"], case
        assert bruteforce_lib.e2m1_nearest_even(v) == case["index"], case


def test_e8m0_defining_property():
    """2^e is the power of two with amax / 2^e in [4, 8) whenever no clamp applies."""
    rng = np.random.default_rng(1)
    bits = rng.integers(0x00800000, 0x7F800000, 200000, dtype=np.uint32)
    amax = bits.view(np.float32)
    for a in amax[:20000]:
        byte = oracle.e8m0(float(a))
        e = byte - 127
        r = float(a) / 2.0 ** e
        if e > -127:
            assert 4.0 <= r < 8.0, (a, byte)
        else:
            assert r < 8.0


def test_quantize_block_handworked():
    g = load_golden()["block_case"]
    codes, scale = oracle.quantize_block(np.array(g["y"], dtype=np.float32))
    assert scale == g["scale"]
    assert codes.tobytes().hex() == g["codes_hex"].replace(" ", "")


def test_quantize_block_codes_are_nearest_grid_points():
    """For random blocks: every decoded element is the grid point nearest to y / 2^e (ties to even code)."""
    rng = np.random.default_rng(2)
    for _ in range(300):
        y = (rng.standard_normal(32) * 10.0 ** rng.uniform(-6, 6)).astype(np.float32)
        if rng.random() < 0.3:
            y[rng.integers(0, 32)] *= 50
        codes, scale = oracle.quantize_block(y)
        e = scale - 127
        v = y.astype(np.float64) / 2.0 ** e
        cds = oracle.unpack_codes(codes[None])[0]
        idx = cds & 7
        dist = np.abs(np.abs(v)[:, None] - oracle.E2M1_GRID[None, :])
        best = dist.min(axis=1)
        assert np.all(dist[np.arange(32), idx] == best)
        tie = (dist == best[:, None]).sum(axis=1) > 1
        assert np.all(idx[tie] % 2 == 0)
        assert np.all((cds >> 3) == np.signbit(y))


# ---------------------------------------------------------------- whole path


@pytest.fixture(scope="module")
def tiny():
    spec = synth.CONFIGS[0][0]
    return synth.matrix(spec), synth.params(spec)


def test_transform_matches_numpy_row_vector_matmul(tiny):
    X, P = tiny
    o = oracle.quantize_rows(oracle.KRON, X, P, want_y=True)
    x = synth.bf16_to_f32(X).astype(np.float64)
    K32, _ = oracle.build_blocks(P, P.shape[0])
    for j in range(P.shape[0]):
        ref = x[:, 32 * j:32 * j + 32] @ K32[j].astype(np.float64)
        got = o["yhat"][:, 32 * j:32 * j + 32]
        bound = 1e-14 * (np.abs(x[:, 32 * j:32 * j + 32]) @ np.abs(K32[j].astype(np.float64)))
        assert np.all(np.abs(got - ref) <= bound + 1e-300)
        np.testing.assert_array_equal(o["y32"][:, 32 * j:32 * j + 32], got.astype(np.float32))


def test_identity_block_equals_plain(tiny):
    X, P = tiny
    k = oracle.quantize_rows(oracle.KRON, X, P)
    p = oracle.quantize_rows(oracle.PLAIN, X)
    np.testing.assert_array_equal(k["codes"][:, :16], p["codes"][:, :16])
    np.testing.assert_array_equal(k["scales"][:, 0], p["scales"][:, 0])


def test_hadamard_block_equals_signed_fwht(tiny):
    """Block 1 of the tiny config uses the Hadamard-like factors: y = D32 * WHT(x) / sqrt(32)."""
    X, P = tiny
    k = oracle.quantize_rows(oracle.KRON, X, P, want_y=True)
    h = oracle.quantize_rows(oracle.HADAMARD, X, want_y=True)
    D = np.array([(-1.0) ** bin(c).count("1") for c in range(32)])
    yk = k["yhat"][:, 32:64]
    yh = h["yhat"][:, 32:64] * D
    amax = np.abs(yh).max(axis=1, keepdims=True)
    assert np.all(np.abs(yk - yh) <= 1e-6 * amax)
    # the scales agree except where the block amax sits within that error of a power of two
    sk, sh = k["scales"][:, 1], h["scales"][:, 1]
    am = amax[:, 0]
    near = np.abs(np.log2(am) - np.round(np.log2(am))) < 1e-5
    assert np.all((sk == sh) | near)


def test_hadamard_front_end_matches_scipy(tiny):
    X, _ = tiny
    h = oracle.quantize_rows(oracle.HADAMARD, X, want_y=True)
    x = synth.bf16_to_f32(X).astype(np.float64)
    H = scipy.linalg.hadamard(32).astype(np.float64)
    for j in range(X.shape[1] // 32):
        ref = x[:, 32 * j:32 * j + 32] @ H / np.sqrt(32)
        np.testing.assert_allclose(h["yhat"][:, 32 * j:32 * j + 32], ref, rtol=1e-13,
                                   atol=1e-13 * np.abs(ref).max())


def test_plain_and_smooth_front_ends_exact(tiny):
    X, _ = tiny
    x = synth.bf16_to_f32(X)
    p = oracle.quantize_rows(oracle.PLAIN, X, want_y=True)
    np.testing.assert_array_equal(p["y32"], x)
    m = synth.smooth_mult(X)
    s = oracle.quantize_rows(oracle.SMOOTH, X, m=m, want_y=True)
    np.testing.assert_array_equal(s["y32"], x * m[None, :])  # numpy float32 multiply: one IEEE rounding


def test_block_locality(tiny):
    """Perturbing block j+1 leaves block j bit-identical (block-diagonal T; review, Sec. 3.2 Eq. (4))."""
    X, P = tiny
    base = oracle.quantize_rows(oracle.KRON, X, P)
    X2 = X.copy()
    X2[:, 32 * 5:32 * 6] ^= 0x0101
    pert = oracle.quantize_rows(oracle.KRON, X2, P)
    np.testing.assert_array_equal(base["codes"][:, :16 * 5], pert["codes"][:, :16 * 5])
    np.testing.assert_array_equal(base["codes"][:, 16 * 6:], pert["codes"][:, 16 * 6:])
    np.testing.assert_array_equal(np.delete(base["scales"], 5, axis=1), np.delete(pert["scales"], 5, axis=1))
    assert not np.array_equal(base["codes"][:, 16 * 5:16 * 6], pert["codes"][:, 16 * 5:16 * 6])


def test_whole_path_codes_are_nearest_and_scales_satisfy_property(tiny):
    X, P = tiny
    o = oracle.quantize_rows(oracle.KRON, X, P, want_y=True)
    y = o["y32"].astype(np.float64)
    T, d = y.shape
    yb = y.reshape(T, d // 32, 32)
    amax = np.abs(yb).max(axis=2)
    e = o["scales"].astype(np.int64) - 127
    r = amax / 2.0 ** e
    assert np.all((r >= 4) & (r < 8) | (amax == 0))
    v = yb / 2.0 ** e[:, :, None]
    idx = oracle.unpack_codes(o["codes"]).reshape(T, d // 32, 32) & 7
    dist = np.abs(np.abs(v)[..., None] - oracle.E2M1_GRID)
    assert np.all(np.take_along_axis(dist, idx[..., None].astype(np.int64), -1)[..., 0] == dist.min(-1))


def test_shared_k_stride_zero(tiny):
    X, P = tiny
    one = P[2:3].copy()
    a = oracle.quantize_rows(oracle.KRON, X, one, pstride=0)
    b = oracle.quantize_rows(oracle.KRON, X, np.repeat(one, X.shape[1] // 32, axis=0), pstride=15)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_array_equal(a["scales"], b["scales"])


def test_rejects_bad_arguments(tiny):
    X, P = tiny
    with pytest.raises(ValueError):
        oracle.quantize_rows(oracle.KRON, X[:, :40], P)
    with pytest.raises(ValueError):
        oracle.quantize_rows(oracle.SMOOTH, X)


def test_threaded_rows_match_single(tiny):
    X, P = tiny
    a = oracle.quantize_rows(oracle.KRON, X, P, threads=1)
    b = oracle.quantize_rows(oracle.KRON, X, P, threads=4)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_array_equal(a["scales"], b["scales"])
