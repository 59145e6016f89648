"""Pins of the parity classifier (oracle/compare.py) with injected errors.

Every GPU parity verdict goes through compare(): scales must match bit for
bit, and a code that differs from the oracle's is accepted only as a rounding
tie of the transform (same sign, one E2M1 grid step apart, the exact value
y / 2^e within tol * amax / 2^e of the midpoint between the two grid values)
or as a zero code whose sign is undetermined (exact value within that bound
of zero); at least 99.99% of all codes must be exact.  These rules follow the
OCP Microscaling v1.0 E2M1 / E8M0 definitions the Pith review cites as its
reference [10] and the 1e-5-of-the-block-amax transform tolerance.

Each case below starts from the oracle's own output for a plain-MXFP4 matrix
(y = x, so the exact value of every element is known), injects one kind of
error and checks the verdict.  A classifier with a plausible mistake (a
midpoint taken at the wrong index, the rounded instead of the exact value
near the midpoint, a sign flip accepted at a large value, unexplained codes
ignored by ok(), an off-by-one threshold) fails one of them.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle.compare import TOL, compare, transform_error


def pack(nib: np.ndarray) -> np.ndarray:
    """[T, d] 4-bit codes -> [T, d/2] bytes, even channel in the low nibble."""
    nib = nib.astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def plain_case(rows: np.ndarray):
    """Oracle output of the plain front-end for fp32 rows that are exact in bf16,
    and the (yhat, y32) callable: for y = x both are x itself."""
    X = synth.f32_to_bf16(rows.astype(np.float32))
    ref = oracle.quantize_rows(oracle.PLAIN, X)
    xs = synth.bf16_to_f32(X).astype(np.float64)

    def yh(sel):
        return xs[sel], xs[sel].astype(np.float32)

    return ref["codes"], ref["scales"], yh


def block(vals, scale_pow: int = 0) -> np.ndarray:
    """One 32-channel block: element 0 = 6 * 2^k (scale 2^k), then vals * 2^k, zero-padded."""
    b = np.zeros(32, dtype=np.float64)
    b[0] = 6.0
    b[1:1 + len(vals)] = vals
    return b * 2.0 ** scale_pow


def nibbles(codes: np.ndarray) -> np.ndarray:
    return oracle.unpack_codes(codes).astype(np.uint8)


def with_code(codes, t, ch, new):
    n = nibbles(codes)
    n[t, ch] = new
    return pack(n)


def test_oracle_ties_follow_round_to_nearest_even():
    """The hand-picked values land where the E2M1 rule puts them (0.75 is the
    midpoint of grid values 0.5 and 1.0 and rounds to the even index, 1.0)."""
    codes, scales, _ = plain_case(block([0.75, 0.875, 0.1, 1e-6, -0.75, 2.5])[None])
    n = nibbles(codes)[0]
    assert scales[0, 0] == 127
    assert list(n[:7]) == [7, 2, 2, 0, 0, 0xA, 4]


def test_exact_output_accepted():
    codes, scales, yh = plain_case(np.stack([block([0.75, 0.3, -2.5]), block([1.25], 5)]))
    r = compare(codes, scales, codes, scales, yh)
    assert r.ok(exact=True) and r.code_mismatch == 0 and r.scale_mismatch == 0


@pytest.mark.parametrize("delta", [1, -1])
def test_scale_off_by_one_rejected(delta):
    codes, scales, yh = plain_case(block([0.75, 0.3])[None])
    bad = scales.copy()
    bad[0, 0] = np.uint8(int(bad[0, 0]) + delta)
    r = compare(codes, bad, codes, scales, yh)
    assert r.scale_mismatch == 1 and not r.ok()


def test_one_step_at_the_midpoint_is_a_tie():
    """0.75 (oracle code 2 = 1.0) reported as code 1 (0.5): one step, exact value on the midpoint."""
    codes, scales, yh = plain_case(block([0.75])[None])
    r = compare(with_code(codes, 0, 1, 1), scales, codes, scales, yh)
    assert r.code_mismatch == 1 and r.code_unexplained == 0 and r.scale_mismatch == 0


def test_midpoint_is_taken_between_the_two_codes():
    """A one-step difference between codes 1 and 2 is a tie only near 0.75, the
    midpoint of those two grid values; 1.25 is the midpoint of the next pair."""
    codes, scales, yh = plain_case(block([0.75])[None])
    # the same mismatch, but claim the exact value was 1.25: not near 0.75
    def yh_far(sel):
        yhat, y32 = yh(sel)
        yhat = yhat.copy()
        yhat[:, 1] = 1.25
        return yhat, yhat.astype(np.float32)
    r = compare(with_code(codes, 0, 1, 1), scales, codes, scales, yh_far)
    assert r.code_unexplained == 1 and not r.ok()


def test_one_step_far_from_the_midpoint_is_unexplained():
    """0.875 (oracle code 2) reported as code 1: one step, but 0.125 from the midpoint."""
    codes, scales, yh = plain_case(block([0.875])[None])
    r = compare(with_code(codes, 0, 1, 1), scales, codes, scales, yh)
    assert r.code_unexplained == 1 and not r.ok()


def test_two_steps_is_unexplained():
    codes, scales, yh = plain_case(block([0.75])[None])
    r = compare(with_code(codes, 0, 1, 0), scales, codes, scales, yh)  # code 2 -> code 0
    assert r.code_unexplained == 1 and not r.ok()


def test_sign_flip_of_a_nonzero_code_is_unexplained():
    codes, scales, yh = plain_case(block([0.75])[None])
    r = compare(with_code(codes, 0, 1, 0xA), scales, codes, scales, yh)  # +1.0 -> -1.0
    assert r.code_unexplained == 1 and not r.ok()
    # one grid step and on the midpoint, but the other sign: +1.0 -> -0.5
    r = compare(with_code(codes, 0, 1, 0x9), scales, codes, scales, yh)
    assert r.code_unexplained == 1 and not r.ok()


def test_two_steps_from_a_midpoint_is_unexplained():
    """0.25 is the midpoint of codes 0 and 1 (oracle: code 0); code 2 is two steps
    from code 0 although the value sits on the lower pair's midpoint."""
    codes, scales, yh = plain_case(block([0.25])[None])
    assert nibbles(codes)[0, 1] == 0
    r = compare(with_code(codes, 0, 1, 2), scales, codes, scales, yh)
    assert r.code_unexplained == 1 and not r.ok()


def test_one_unexplained_code_fails_a_large_matrix():
    """A single unexplained code among 640000 (99.9998% exact) still fails."""
    T = 10000
    rows = np.tile(np.concatenate([block([0.875] * 31), block([0.875] * 31)]), (T, 1))
    codes, scales, yh = plain_case(rows)
    r = compare(with_code(codes, 17, 33, 1), scales, codes, scales, yh)
    assert r.code_mismatch == 1 and r.code_unexplained == 1 and r.exact_fraction > 0.9999
    assert not r.ok()


def test_zero_code_sign_within_the_bound_is_a_tie():
    """A value within tol * amax of zero (amax 6, value 1e-6) may carry either sign in a zero code."""
    codes, scales, yh = plain_case(block([0.0, 1e-6])[None])
    assert nibbles(codes)[0, 2] == 0
    r = compare(with_code(codes, 0, 2, 8), scales, codes, scales, yh)
    assert r.code_mismatch == 1 and r.code_unexplained == 0 and r.scale_mismatch == 0


def test_zero_code_sign_beyond_the_bound_is_unexplained():
    """0.1 is far beyond tol * amax = 6e-5 from zero: -0 for +0.1 is wrong."""
    codes, scales, yh = plain_case(block([0.1])[None])
    assert nibbles(codes)[0, 1] == 0
    r = compare(with_code(codes, 0, 1, 8), scales, codes, scales, yh)
    assert r.code_unexplained == 1 and not r.ok()


def test_tolerance_scales_with_the_block_exponent():
    """Scale 2^5 (amax 192): the bound on y / 2^e is tol * 6; a value 3e-6 above
    the midpoint after scaling is a tie, one 2e-4 above is not."""
    codes, scales, yh = plain_case(block([0.75], 5)[None])
    assert scales[0, 0] == 132
    for off, explained in ((3e-6, True), (2e-4, False)):
        def yh_off(sel, off=off):
            yhat, _ = yh(sel)
            yhat = yhat.copy()
            yhat[:, 1] = 0.75 * (1 + off / 0.75) * 32.0
            return yhat, yhat.astype(np.float32)
        r = compare(with_code(codes, 0, 1, 1), scales, codes, scales, yh_off)
        assert (r.code_unexplained == 0) == explained, (off, r)


def test_midpoint_test_uses_the_exact_value_not_the_rounded_one():
    """With a bound far below fp32 resolution, a value whose fp32 rounding sits on
    the midpoint but whose exact value does not is not a tie."""
    codes, scales, yh = plain_case(block([0.75])[None])

    def yh_fine(sel):
        yhat, _ = yh(sel)
        yhat = yhat.copy()
        yhat[:, 1] = 0.75 * (1 + 2.0 ** -30)   # fp32 rounding: exactly 0.75
        return yhat, yhat.astype(np.float32)

    bad = with_code(codes, 0, 1, 1)
    assert compare(bad, scales, codes, scales, yh_fine, tol=1e-12).code_unexplained == 1
    assert compare(bad, scales, codes, scales, yh_fine, tol=1e-9).code_unexplained == 0


def test_mismatch_fraction_threshold():
    """ok() needs >= 99.99% exact codes even when every mismatch is a tie:
    N = 640000 codes, 64 ties -> exactly 99.99% (ok), 65 -> below (not ok)."""
    T = 10000
    rows = np.tile(np.concatenate([block([0.75] * 31), block([0.75] * 31)]), (T, 1))
    codes, scales, yh = plain_case(rows)
    n = nibbles(codes)
    assert n.size == 640000 and np.all(n[:, 1:32] == 2)
    for k, good in ((64, True), (65, False)):
        m = n.copy()
        m[np.arange(k), 1] = 1   # one tie in each of the first k rows
        r = compare(pack(m), scales, codes, scales, yh)
        assert r.code_mismatch == k and r.code_unexplained == 0
        assert r.ok() == good, (k, r)
        assert not r.ok(exact=True)


def test_mismatches_without_exact_values_are_unexplained():
    codes, scales, _ = plain_case(block([0.75])[None])
    r = compare(with_code(codes, 0, 1, 1), scales, codes, scales, None)
    assert r.code_unexplained == 1 and not r.ok()


def test_transform_error_hand_computed():
    """|y_gpu - yhat| / (block amax of the oracle's y), per block; a nonzero error
    in an all-zero block is infinite."""
    yhat = np.zeros((2, 64))
    yhat[0, :32] = np.round(np.linspace(-3.0, 4.0, 32) * 64) / 64   # amax 4, exact in fp32
    yhat[1, 32:] = np.round(np.linspace(0.5, 2.0, 32) * 64) / 64    # amax 2
    y32 = yhat.astype(np.float32)
    g = y32.copy()
    assert transform_error(g, yhat, y32) == 0.0
    g[0, 5] += np.float32(1e-4)   # 1e-4 / 4
    g[1, 40] -= np.float32(3e-5)  # 3e-5 / 2
    err = transform_error(g, yhat, y32)
    want = max(abs(float(g[0, 5]) - yhat[0, 5]) / 4.0, abs(float(g[1, 40]) - yhat[1, 40]) / 2.0)
    assert err == pytest.approx(want, rel=1e-12)
    assert 2.4e-5 < err < 2.6e-5
    g2 = y32.copy()
    g2[1, 3] = np.float32(1e-30)  # block 0 of row 1 is all zero
    assert transform_error(g2, yhat, y32) == np.inf
    assert TOL == 1e-5
