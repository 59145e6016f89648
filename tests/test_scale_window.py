"""The exact-scale window of the default (block-per-lane) kernel, proved for the workloads.

The kernel quantizes a block again from exact values when its fp32 amax lies
within 2^-16 of a power of two; elsewhere it keeps the fp32 transform's
exponent.  That is sound for a block when the transform's error cannot move
its amax across a power of two.  A bound from the kernel's rounding steps:
every value passes through 25 relative roundings of 2^-24 at most (five
shear pairs, one rounding each and one more for the coefficient a b; the
diagonal's reciprocals, products and multiply), and the exact sum the oracle
and the exact path form (fp64, entries of K rounded to fp32) is within one
more rounding of x K.  With A = |D||U||L| (each factor's shears and
diagonal in absolute values) and N_A = prod_k max row sum of A_k,

    |y_kernel - y_exact| <= 27.2 u N_A max|x|,   u = 2^-24,

so the window is sound for a block when w = (27.2 N_A max|x| / amax + 1.1) u
(1.1 u: the final fp32 rounding of the exact amax) stays within 2^-16.

These tests emulate the kernel's fp32 steps in numpy (shear pairs G5 first,
then the diagonal; coefficients l, fl(a b), fl(1/a) and their tree products,
as the kernel forms them), check the bound against the oracle's exact sums
for factors near and far from the identity, and check w <= 2^-16 for every
block of sampled rows of the PixArt, SANA, FLUX and stress workloads.  The
tiny config's block 1 (Hadamard-butterfly factors) is outside the proof; its
scales are checked on the GPU like every other block's.  Parity of the kernel
itself is the GPU tests' job."""
import numpy as np
import pytest

import oracle
import synth

U = 2.0 ** -24


def fma32(a, b, c):
    # a b is exact in fp64; the sum rounds once in fp64 and again to fp32
    # (within 2^-24 (1 + 2^-29) of the fused result, inside the bound's margin)
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def emulate_kernel(x, P):
    """x [T, 32 nb] float32, P [nb, 5, 3] (l, a, b): the kernel's fp32 y."""
    T, d = x.shape
    nb = d // 32
    y = x.reshape(T, nb, 32).astype(np.float32).copy()
    l, a, b = P[:, :, 0], P[:, :, 1], P[:, :, 2]
    ss = (a * b).astype(np.float32)
    for k in range(4, -1, -1):
        bit = 1 << (4 - k)
        lo = [c for c in range(32) if not c & bit]
        for c in lo:
            y[:, :, c] = fma32(np.broadcast_to(l[:, k], (T, nb)), y[:, :, c | bit], y[:, :, c])
        for c in lo:
            y[:, :, c | bit] = fma32(np.broadcast_to(ss[:, k], (T, nb)), y[:, :, c], y[:, :, c | bit])
    ia = (np.float32(1.0) / a).astype(np.float32)

    def ent(c, k):
        return np.where((c >> (4 - k)) & 1, ia[:, k], a[:, k])

    dg = np.empty((nb, 32), np.float32)
    for c in range(32):
        v = (ent(c, 0) * ent(c, 1)).astype(np.float32)
        for k in (2, 3, 4):
            v = (v * ent(c, k)).astype(np.float32)
        dg[:, c] = v
    return (y * dg[None]).astype(np.float32).reshape(T, d)


def norm_a(P):
    """N_A per block column: prod_k max row sum of |D_k||U_k||L_k| = [[|a|, |a||l|], [|b|, (1 + |a b||l|) / |a|]]."""
    l, a, b = (np.abs(P[:, :, i].astype(np.float64)) for i in range(3))
    return np.prod(np.maximum(a * (1 + l), b + (1 + a * b * l) / a), axis=1)


def bf16_to_f32(X):
    return (X.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("sigma_lb,sigma_a", [(0.1, 0.1), (0.3, 0.3), (1.0, 0.5), (2.0, 1.0)])
def test_rounding_bound_holds(sigma_lb, sigma_a):
    T, nb = 256, 48
    X = synth.random_matrix(T, 32 * nb, seed=int(sigma_lb * 10 + sigma_a * 100), n_outliers=3, mult=50.0)
    P = synth.random_params(nb, seed=int(sigma_lb * 7 + sigma_a * 3 + 1), sigma_lb=sigma_lb, sigma_a=sigma_a)
    x = bf16_to_f32(X)
    yhat = oracle.quantize_rows(oracle.KRON, X, P, want_y=True)["yhat"]
    y = emulate_kernel(x, P).astype(np.float64)
    err = np.abs(y - yhat).reshape(T, nb, 32).max(axis=2)
    mx = np.abs(x.astype(np.float64)).reshape(T, nb, 32).max(axis=2)
    bound = 27.2 * U * norm_a(P)[None] * mx
    assert np.all(err <= bound), float(np.max(err / np.maximum(bound, 1e-300)))


def test_bound_catches_a_wrong_norm():
    """The bound is not vacuous: with N_A replaced by 1 (the factors' growth
    ignored) wide factors break it."""
    T, nb = 256, 48
    X = synth.random_matrix(T, 32 * nb, seed=3, n_outliers=3, mult=50.0)
    P = synth.random_params(nb, seed=4, sigma_lb=1.0, sigma_a=0.5)
    x = bf16_to_f32(X)
    yhat = oracle.quantize_rows(oracle.KRON, X, P, want_y=True)["yhat"]
    err = np.abs(emulate_kernel(x, P).astype(np.float64) - yhat).reshape(T, nb, 32).max(axis=2)
    mx = np.abs(x.astype(np.float64)).reshape(T, nb, 32).max(axis=2)
    assert np.any(err > 27.2 * U * mx)


@pytest.mark.parametrize("spec", [s for c in (1, 2, 3, 4) for s in synth.CONFIGS[c]], ids=lambda s: s.name)
def test_fixed_window_is_sound_for_the_workloads(spec):
    T = 192
    X = synth.matrix(spec)[:T]
    P = synth.params(spec)
    nb = spec.d // 32
    Pc = np.repeat(P.reshape(-1, 5, 3), nb, axis=0) if spec.shared_k else P.reshape(nb, 5, 3)
    yhat = oracle.quantize_rows(oracle.KRON, X, P, 0 if spec.shared_k else 15, want_y=True)["yhat"]
    mx = np.abs(bf16_to_f32(X).astype(np.float64)).reshape(T, nb, 32).max(axis=2)
    amax = np.abs(yhat).reshape(T, nb, 32).max(axis=2)
    live = amax >= 2.0 ** -97
    w = (27.2 * norm_a(Pc)[None] * mx / np.where(live, amax, 1) + 1.1) * U * 1.01
    assert np.all(w[live] <= 2.0 ** -16), f"{spec.name}: window 2^{np.log2(w[live].max()):.2f}"
