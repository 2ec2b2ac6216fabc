"""CPU checks of the comparison rules themselves (tests/parity.py), on planted cases."""
import numpy as np
import pytest

from parity import assert_out_close, check_idx_row, kernel_precision

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
