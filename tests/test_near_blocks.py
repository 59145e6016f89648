"""CPU checks of the near-power-of-two blocks (tests/near_blocks.py) that the
exact-scale GPU tests feed to every kernel: the oracle puts their exact amax
within 2^-20 of a power of two on both sides, and an fp32 evaluation of the
same transform in another summation order picks a different E8M0 scale for
some of them, so a kernel that does not decide such scales exactly fails."""
import numpy as np

import near_blocks as nbk
import oracle
import synth


def test_kron_blocks_straddle_powers_of_two():
    X, P, near = nbk.near_matrix_kron(8, 36, seed=11)
    assert near.all()
    ref = oracle.quantize_rows(oracle.KRON, X, P, want_y=True)
    amax = np.abs(ref["yhat"]).reshape(8, 36, 32).max(axis=2)
    p = np.round(np.log2(amax))
    rel = amax / 2.0 ** p - 1.0
    assert (rel > 0).sum() >= 100 and (rel < 0).sum() >= 100
    # the oracle's scale follows the fp32 amax: exponent of 2^p above, of 2^(p-1) below
    # unless the fp32 rounding lands on 2^p itself
    a32 = np.abs(ref["y32"].astype(np.float64)).reshape(8, 36, 32).max(axis=2)
    e = ref["scales"].astype(np.int64) - 127 + 2
    np.testing.assert_array_equal(e, np.where(a32 >= 2.0 ** p, p, p - 1))
    assert ((rel < 0) & (a32 == 2.0 ** p)).sum() > 0
    # the same blocks evaluated in fp32 with another order of summation (numpy's fp32 matmul)
    K32, _ = oracle.build_blocks(P, 36)
    xs = synth.bf16_to_f32(X).reshape(8, 36, 32)
    y = np.einsum("tjr,jrc->tjc", xs.astype(np.float32), K32.astype(np.float32))
    e32 = np.floor(np.log2(np.abs(y).max(axis=2))).astype(np.int64)
    assert (e32 != e).sum() > 0


def test_hadamard_blocks_straddle_powers_of_two():
    for B in (32, 64, 128, 256, 512):
        X, near = nbk.near_matrix_hadamard(4, 1024, B, seed=B)
        assert near[:, ::B // 32].all(), B
