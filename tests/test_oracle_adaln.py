"""Pins of the oracle's producer step (LayerNorm statistics and AdaLN modulation).

Each test checks the oracle against something other than its own code:
hand-worked values (tests/golden/adaln_handworked.json), exact rational
arithmetic, the defining property of a normalised row, identities, and
torch's float32 -> bfloat16 conversion for the final rounding.
"""
import json
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _bf16_bits(values):
    return synth.f32_to_bf16(np.asarray(values, dtype=np.float32))


def test_handworked_cases():
    cases = json.load(open(os.path.join(HERE, "golden", "adaln_handworked.json")))["cases"]
    for cse in cases:
        X = _bf16_bits(cse["x"]).reshape(1, -1)
        st = oracle.row_stats(X, eps=cse["eps"])
        assert st[0, 0] == np.float32(cse["mean"]) and st[0, 1] == np.float32(cse["rstd"]), cse
        out = oracle.adaln_rows(X, st, np.array([cse["scale"]], np.float32), np.array([cse["shift"]], np.float32))
        assert np.array_equal(out[0], _bf16_bits(cse["out"])), cse


def test_row_stats_match_exact_rational_arithmetic():
    """mean and var are exact rationals of the bf16 inputs; rstd to 40 digits; all rounded once to fp32."""
    getcontext().prec = 40
    X = synth.random_matrix(6, 96, seed=11, n_outliers=3, mult=40.0)
    eps = 1e-6
    st = oracle.row_stats(X, eps=eps)
    xf = synth.bf16_to_f32(X).astype(np.float64)
    for t in range(X.shape[0]):
        vals = [Fraction(float(v)) for v in xf[t]]
        mean = sum(vals) / len(vals)
        var = sum((v - mean) ** 2 for v in vals) / len(vals)
        rstd = 1 / (Decimal(var.numerator) / Decimal(var.denominator) + Decimal(eps)).sqrt()
        assert st[t, 0] == np.float32(float(mean))
        exp_rstd = np.float32(float(rstd))
        assert abs(int(st[t, 1].view(np.int32)) - int(exp_rstd.view(np.int32))) <= 1


def test_normalised_rows_have_zero_mean_unit_variance():
    X = synth.random_matrix(16, 1152, seed=12, n_outliers=12, mult=50.0)
    st = oracle.row_stats(X, eps=0.0)
    out = synth.bf16_to_f32(oracle.adaln_rows(X, st)).astype(np.float64)
    assert np.all(np.abs(out.mean(axis=1)) < 1e-2)
    assert np.all(np.abs(out.var(axis=1) - 1.0) < 1e-2)


def test_identity_modulation_and_no_stats():
    X = synth.random_matrix(8, 64, seed=13)
    z = np.zeros((1, 64), np.float32)
    assert np.array_equal(oracle.adaln_rows(X, None, z, z), X)
    assert np.array_equal(oracle.adaln_rows(X), X)


def test_samples_select_their_own_vectors():
    X = synth.random_matrix(12, 64, seed=14)
    rng = np.random.default_rng(0)
    sc = rng.normal(0, 0.5, (3, 64)).astype(np.float32)
    sh = rng.normal(0, 0.5, (3, 64)).astype(np.float32)
    st = oracle.row_stats(X)
    whole = oracle.adaln_rows(X, st, sc, sh, tokens_per_sample=4)
    for s in range(3):
        part = oracle.adaln_rows(X[4 * s:4 * s + 4], st[4 * s:4 * s + 4], sc[s:s + 1], sh[s:s + 1])
        assert np.array_equal(whole[4 * s:4 * s + 4], part)


def test_final_rounding_matches_torch_bfloat16():
    X = synth.random_matrix(8, 128, seed=15, n_outliers=2, mult=30.0)
    st = oracle.row_stats(X)
    rng = np.random.default_rng(1)
    sc = rng.normal(0, 0.5, (1, 128)).astype(np.float32)
    sh = rng.normal(0, 0.5, (1, 128)).astype(np.float32)
    xf = synth.bf16_to_f32(X)
    v = (xf - st[:, :1]) * st[:, 1:]
    v = v * (np.float32(1) + sc)
    v = v + sh
    assert v.dtype == np.float32
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.adaln_rows(X, st, sc, sh), ref)


def test_rejects_bad_arguments():
    X = synth.random_matrix(2, 32, seed=16)
    with pytest.raises(ValueError):
        oracle.row_stats(X, eps=-1.0)
