"""CPU checks of the comparison rules themselves (tests/parity.py), on planted cases."""
import numpy as np
import pytest

from parity import assert_out_close, check_idx_row, kernel_precision, order_violation

import oracle


def test_out_rule_is_relative_to_row_max():
    ref = np.array([[1.0, 0.001, -0.5], [0.0, 0.0, 0.0]])
    assert_out_close(ref + np.array([[1.9e-3, 0, 0], [0, 0, 0]]), ref)
    with pytest.raises(AssertionError):
        assert_out_close(ref + np.array([[2.1e-3, 0, 0], [0, 0, 0]]), ref)
    with pytest.raises(AssertionError):
        assert_out_close(ref + np.array([[0, 0, 0], [1e-9, 0, 0]]), ref)


def test_idx_rule_accepts_band_swaps_only():
    rng = np.random.default_rng(0)
    n, W, k = 400, 16, 64
    s = rng.random(n)
    ref = oracle.select_tokens(s, W, k)
    assert check_idx_row(ref, ref, s, n, W, k) == 0
    cand = np.arange(n - W)
    order = cand[np.lexsort((cand, -s[cand]))]
    inside, outside = order[k - 1], order[k]
    # a near-tie swap of the k-th and (k+1)-th candidate is accepted
    s2 = s.copy()
    s2[outside] = s2[inside] * (1 - 1e-7)
    ref2 = oracle.select_tokens(s2, W, k)
    swapped = np.sort(np.concatenate([ref2[ref2 >= 0][ref2[ref2 >= 0] != inside], [outside]]))
    row = np.full_like(ref2, -1)
    row[:len(swapped)] = swapped
    assert check_idx_row(row, ref2, s2, n, W, k) == 1
    # the same swap without a near tie is rejected
    with pytest.raises(AssertionError):
        check_idx_row(row, ref, s, n, W, k)
    # a missing window position is rejected
    bad = ref.copy()
    bad[np.where(bad == n - 1)[0][0]] = order[k]
    with pytest.raises(AssertionError):
        check_idx_row(np.sort(bad), ref, s, n, W, k)


def test_kernel_precision_flushes_below_float32_range():
    s = np.array([1e-72, 3e-72, 1e-40, 2e-38, 0.5])
    got = kernel_precision(s)
    assert got[0] == 0 and got[1] == 0 and got[2] == 0
    assert got[3] == np.float32(2e-38) and got[4] == 0.5


def _row(positions, S):
    row = np.full(S, -1, dtype=np.int64)
    p = np.sort(np.asarray(list(positions), dtype=np.int64))
    row[:len(p)] = p
    return row


def test_idx_rule_enforces_lower_positions_among_float32_zeros():
    """Scores far below the float32 range are all zero in the kernel's precision: the
    GPU must then take the lowest zero-score positions, whatever the float64 order."""
    rng = np.random.default_rng(3)
    n, W, k = 400, 16, 64
    w0 = n - W
    s = 10.0 ** rng.uniform(-80, -60, n)               # all flush to 0 in float32
    big = rng.choice(w0, size=40, replace=False)
    s[big] = rng.uniform(0.01, 0.02, size=40)            # 40 clear winners
    ref = oracle.select_tokens(s, W, k)
    zeros = np.setdiff1d(np.arange(w0), big)
    win = np.arange(w0, n)
    good = _row(np.concatenate([big, zeros[:24], win]), W + k)
    assert check_idx_row(good, ref, s, n, W, k) >= 1   # differs from the float64 choice
    # one zero-score pick moved to a higher position: the tie order is violated
    late = _row(np.concatenate([big, zeros[:23], zeros[30:31], win]), W + k)
    with pytest.raises(AssertionError, match="tie order"):
        check_idx_row(late, ref, s, n, W, k)
    # the float64 order among the zeros is not the kernel-precision order either
    if not np.array_equal(np.sort(ref[ref >= 0]), good[good >= 0]):
        with pytest.raises(AssertionError, match="tie order"):
            check_idx_row(ref, ref, s, n, W, k)
    # a clear winner dropped for a zero is rejected (outside the band of the k-th = 0)
    drop = _row(np.concatenate([big[1:], zeros[:25], win]), W + k)
    with pytest.raises(AssertionError):
        check_idx_row(drop, ref, s, n, W, k)


def test_idx_rule_zero_ties_with_scores_at_the_float32_edge():
    """A score at the smallest normal float32 may be flushed by the kernel: it may be
    taken or left like a zero, but a zero may not displace a clearly positive score."""
    n, W, k = 200, 8, 16
    w0 = n - W
    s = np.full(n, 1e-70)
    s[:10] = 0.05                                       # 10 winners
    s[150] = float(np.finfo(np.float32).tiny)           # at the edge
    ref = oracle.select_tokens(s, W, k)                 # float64: 0..9, 150, then 1e-70 ties
    win = np.arange(w0, n)
    flushed = _row(np.concatenate([np.arange(16), win]), W + k)      # 150 treated as zero
    assert check_idx_row(flushed, ref, s, n, W, k) >= 1
    kept = _row(np.concatenate([np.arange(15), [150], win]), W + k)  # 150 kept
    check_idx_row(kept, ref, s, n, W, k)
    wrong = _row(np.concatenate([np.arange(1, 16), [150], win]), W + k)  # drops winner 0
    with pytest.raises(AssertionError):
        check_idx_row(wrong, ref, s, n, W, k)


def test_order_violation_interval_rule():
    s32 = np.array([1.0, 1.0 + 5e-7, 0.9, 0.0, 0.0, 0.0])
    # near-equal scores may go either way; a clearly smaller one may not be preferred
    assert order_violation(np.array([True, False, False, False, False, False]), s32) is None
    assert order_violation(np.array([False, True, False, False, False, False]), s32) is None
    assert order_violation(np.array([False, False, True, False, False, False]), s32) == (2, 1)
    assert order_violation(np.array([True, False, False, True, False, False]), s32) == (3, 1)
    # among exact zeros the lower position goes first
    assert order_violation(np.array([True, True, True, True, False, False]), s32) is None
    assert order_violation(np.array([True, True, True, False, True, False]), s32) == (4, 3)
