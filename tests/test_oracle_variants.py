"""Pins of the oracle's variants: block-Hadamard front-ends of size 32..512
and 16-wide, 4-factor KroQuant blocks.

Checked against scipy's Hadamard matrices, the B = 32 front-end, exact
orthogonality, numpy's Kronecker product, determinants, and identities.
"""
import numpy as np
import pytest
from scipy.linalg import hadamard

import oracle
import synth


@pytest.mark.parametrize("B", [32, 64, 128, 256, 512])
def test_hadamard_b_matches_scipy(B):
    X = synth.random_matrix(6, 1024, seed=B, n_outliers=4, mult=30.0)
    out = oracle.quantize_rows_hadamard(X, B, want_y=True)
    H = hadamard(B).astype(np.float64)
    xf = synth.bf16_to_f32(X).astype(np.float64)
    ref = np.concatenate([xf[:, b:b + B] @ H for b in range(0, 1024, B)], axis=1) / np.sqrt(B)
    np.testing.assert_allclose(out["yhat"], ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    np.testing.assert_array_equal(out["y32"], out["yhat"].astype(np.float32))
    # the MXFP4 step is the shared one
    c2, s2 = oracle.quantize_f32_rows(out["y32"])
    np.testing.assert_array_equal(out["codes"], c2)
    np.testing.assert_array_equal(out["scales"], s2)


def test_hadamard_32_equals_existing_front_end():
    X = synth.random_matrix(9, 288, seed=3, n_outliers=2, mult=30.0)
    a = oracle.quantize_rows_hadamard(X, 32, want_y=True)
    b = oracle.quantize_rows(oracle.HADAMARD, X, want_y=True)
    for k in ("codes", "scales", "y32", "yhat"):
        np.testing.assert_array_equal(a[k], b[k])


def test_hadamard_b_is_orthonormal_energy_preserving():
    X = synth.random_matrix(4, 512, seed=4)
    y = oracle.quantize_rows_hadamard(X, 512, want_y=True)["yhat"]
    xf = synth.bf16_to_f32(X).astype(np.float64)
    np.testing.assert_allclose((y ** 2).sum(axis=1), (xf ** 2).sum(axis=1), rtol=1e-12)


def test_hadamard_rejects_bad_sizes():
    X = synth.random_matrix(2, 96, seed=5)
    for B in (16, 48, 1024):
        with pytest.raises(ValueError):
            oracle.quantize_rows_hadamard(X, B)
    with pytest.raises(ValueError):
        oracle.quantize_rows_hadamard(X, 64)  # 96 % 64 != 0


def test_blocks16_match_numpy_kron_and_are_block_diagonal():
    rng = np.random.default_rng(6)
    P16 = np.stack([np.stack([rng.normal(0, 0.3), np.exp(rng.normal(0, 0.3)), rng.normal(0, 0.3)]) for _ in range(4 * 6)])
    P16 = P16.reshape(6, 4, 3).astype(np.float32)
    K = oracle.build_blocks16(P16)
    assert K.shape == (3, 32, 32)
    for j in range(3):
        for h in range(2):
            G = [oracle.factor(*P16[2 * j + h, k]) for k in range(4)]
            ref = np.kron(np.kron(np.kron(G[0], G[1]), G[2]), G[3])
            blk = K[j, 16 * h:16 * h + 16, 16 * h:16 * h + 16].astype(np.float64)
            assert np.abs(blk - ref).max() <= 2e-7 * np.abs(ref).max()
            assert abs(np.linalg.det(ref) - 1.0) < 1e-9
        assert not K[j, :16, 16:].any() and not K[j, 16:, :16].any()


def test_blocks16_identity_factors_give_plain_mx():
    P16 = np.zeros((8, 4, 3), dtype=np.float32)
    P16[:, :, 1] = 1.0
    K = oracle.build_blocks16(P16)
    np.testing.assert_array_equal(K, np.broadcast_to(np.eye(32, dtype=np.float32), K.shape))
    X = synth.random_matrix(5, 128, seed=7, n_outliers=1, mult=20.0)
    a = oracle.quantize_rows_blocks(X, K)
    b = oracle.quantize_rows(oracle.PLAIN, X)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_array_equal(a["scales"], b["scales"])
