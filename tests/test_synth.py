"""The seeded input generators: determinism and the workload shapes they promise."""
import hashlib

import numpy as np

import synth


def test_deterministic_and_thread_independent():
    spec = synth.CONFIGS[0][0]
    a = synth.matrix(spec, threads=1)
    b = synth.matrix(spec, threads=7)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(synth.params(spec), synth.params(spec))


def test_row_subset_is_prefix():
    spec = synth.CONFIGS[3][1]
    full = synth.matrix(spec.with_rows(64))
    part = synth.matrix(spec.with_rows(16))
    np.testing.assert_array_equal(full[:16], part)


def test_outliers_and_token_scale():
    spec = synth.CONFIGS[1][1].with_rows(2048)
    X, outl = synth.matrix(spec, with_outliers=True)
    assert len(outl) == spec.n_outliers == 46 and len(set(outl.tolist())) == 46
    x = np.abs(synth.bf16_to_f32(X).astype(np.float64))
    col = x.mean(axis=0)
    normal = np.setdiff1d(np.arange(spec.d), outl)
    ratio = col[outl].mean() / col[normal].mean()
    assert 35 < ratio < 65  # multiplier 50


def test_stress_zero_groups_and_heavy_tail():
    spec = synth.CONFIGS[4][0].with_rows(256)
    X = synth.matrix(spec)
    g = X.reshape(256, -1, 32)
    zero = np.all(g == 0, axis=2).mean()
    assert 0.005 < zero < 0.015
    x = synth.bf16_to_f32(X).astype(np.float64)
    normal = x[:, np.abs(x).mean(axis=0) < 5]
    kurt = ((normal - normal.mean()) ** 4).mean() / normal.var() ** 2
    assert kurt > 6  # Student-t(3) is heavy tailed (a Gaussian has 3)


def test_params_layout_and_special_blocks():
    P = synth.params(synth.CONFIGS[0][0])
    assert P.shape == (36, 5, 3) and P.dtype == np.float32
    np.testing.assert_array_equal(P[0], np.tile([0.0, 1.0, 0.0], (5, 1)))
    assert np.all(P[1, :, 0] == 1.0) and np.all(P[1, :, 2] == -P[1, :, 1])
    rest = P[2:]
    assert np.all(rest[:, :, 1] > 0)
    assert abs(rest[:, :, 0].std() - 0.1) < 0.03 and abs(np.log(rest[:, :, 1]).std() - 0.1) < 0.03


def test_shapes_of_all_configs():
    sizes = {s.name: (s.T, s.d) for s in synth.all_specs()}
    assert sizes["tiny"] == (256, 1152)
    assert sizes["pixart_x2"] == (8192, 4608)
    assert sizes["sana_x2"] == (4096, 5600) and 5600 // 32 == 175
    assert sizes["flux_x2"] == (4608, 12288)
    assert sizes["stress"] == (18432, 12288)


def test_bf16_round_trip():
    x = np.array([1.0, -2.5, 3.14159, 1e-3, 65504.0], dtype=np.float32)
    b = synth.f32_to_bf16(x)
    y = synth.bf16_to_f32(b)
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -8)


def test_tiny_hash_is_stable():
    X = synth.matrix(synth.CONFIGS[0][0])
    h = hashlib.sha256(X.tobytes()).hexdigest()
    assert h == hashlib.sha256(synth.matrix(synth.CONFIGS[0][0], threads=3).tobytes()).hexdigest()
