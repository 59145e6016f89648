"""The offline calibration (w4a4_diffusion_transformer_amd.calibrate), on the CPU.

Pins: the fake quantizer against the oracle's MXFP4, the differentiable
Kronecker blocks and their inverse-transpose against the oracle, Eq. (1) with
quantization switched off, orthonormality of the Hadamard-like start, and the
straight-through gradient against central differences of its surrogate.
Then a short calibration run must lower its objective.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from w4a4_diffusion_transformer_amd import calibrate as cal


def test_fake_quant_equals_oracle_mxfp4():
    rng = np.random.default_rng(1)
    Y = (rng.standard_t(3, size=(64, 256)) * 4).astype(np.float32)
    Y[3, 32:64] = 0.0                      # an all-zero block
    Y[5, :32] *= np.float32(1e-38)         # a block whose scale byte clamps at 0
    codes, scales = oracle.quantize_f32_rows(Y)
    ref = oracle.dequant_rows(codes, scales)
    got = cal.mx_fake_quant(torch.from_numpy(Y)).double().numpy()
    np.testing.assert_array_equal(got, ref)


def test_blocks_match_oracle():
    P = synth.random_params(4, seed=2, sigma_lb=0.3, sigma_a=0.3)
    th = torch.from_numpy(P).double()
    G = cal.factors(th)
    K = cal.kron_blocks(G).numpy()
    Kit = cal.kron_blocks(cal.inverse_transpose(G)).numpy()
    for j in range(4):
        np.testing.assert_allclose(K[j], oracle.kron_dense(P[j]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(Kit[j], oracle.kron_inverse(P[j]).T, rtol=0, atol=1e-13)


def test_eq1_without_quantization_is_exact():
    X, W = cal.synthetic_layer(64, 128, 48, (3, 40), 30.0, seed=3)
    th = torch.from_numpy(synth.random_params(4, seed=4, sigma_lb=0.3, sigma_a=0.3))
    out, _, _ = cal.losses(th.double(), X.double(), W.double(), quantize=False)
    assert float(out) < 1e-24


def test_hadamard_start_is_orthonormal():
    K = cal.kron_blocks(cal.factors(cal.hadamard_init(3).double())).numpy()
    for j in range(3):
        np.testing.assert_allclose(K[j] @ K[j].T, np.eye(32), atol=1e-6)


def test_ste_gradient_matches_surrogate_finite_differences():
    X, W = cal.synthetic_layer(32, 64, 16, (1, 40), 20.0, seed=5)
    X, W = X.double(), W.double()
    th0 = cal.hadamard_init(2).double()
    th0 += 0.05 * torch.from_numpy(np.random.default_rng(6).normal(size=th0.shape))
    th = th0.clone().requires_grad_(True)
    out, _, _ = cal.losses(th, X, W)
    out.backward()
    g = th.grad.clone()
    # surrogate: the quantization residuals at th0 held fixed, from the oracle's quantizer
    with torch.no_grad():
        G0 = cal.factors(th0)
        Xt0 = cal.apply_blocks(X, cal.kron_blocks(G0))
        Wt0 = cal.apply_blocks(W, cal.kron_blocks(cal.inverse_transpose(G0)))
        deq = lambda A: oracle.dequant_rows(*oracle.quantize_f32_rows(A.float().numpy()))
        c1 = torch.from_numpy(deq(Xt0)) - Xt0
        c2 = torch.from_numpy(deq(Wt0)) - Wt0
    ref = X @ W.T

    def f(t):
        G = cal.factors(t)
        Xt = cal.apply_blocks(X, cal.kron_blocks(G)) + c1
        Wt = cal.apply_blocks(W, cal.kron_blocks(cal.inverse_transpose(G))) + c2
        return float(((Xt @ Wt.T - ref) ** 2).sum() / (ref ** 2).sum())

    h = 1e-6
    fd = torch.zeros_like(th0)
    for idx in np.ndindex(*th0.shape):
        tp, tm = th0.clone(), th0.clone()
        tp[idx] += h
        tm[idx] -= h
        fd[idx] = (f(tp) - f(tm)) / (2 * h)
    err = float((g - fd).abs().max() / fd.abs().max())
    assert err < 1e-5, err


def test_short_calibration_lowers_the_objective():
    X, W = cal.synthetic_layer(256, 128, 64, (5, 20), 50.0, seed=7)
    theta, hist = cal.calibrate(X, W, steps=30)
    assert hist[-1] < hist[0]
    assert cal.error_kroquant(theta, X, W) <= cal.error_kroquant(cal.hadamard_init(4), X, W)
    assert np.isfinite(cal.error_kroquant_permuted(theta, X, W))
    assert cal.error_smooth(X, W) > 0 and cal.error_plain(X, W) > 0
