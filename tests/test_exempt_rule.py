"""The near-tie exemption used by the GPU parity tests, on the CPU.

A row is exempt from bit-exact index parity only when its oracle k-th and (k+1)-th
scores a >= b differ, by less than 1e-5 of |a|; exact ties are never exempt (the tie rule
decides them).  An exempt GPU row must still hold k distinct ascending positions, every
position scoring above a(1 + 1e-5) and none scoring below b - 1e-5|b|.  These tests fix
the accept/reject bounds of ``row_exempt`` and ``check_selection`` on hand-built rows."""

import numpy as np
import pytest

import oracle.reference as orc
from tests.gpu_util import TIE_REL, check_selection, row_exempt


def test_tie_rel_is_the_stated_bound():
    assert TIE_REL == 1e-5


def test_row_exempt_bounds():
    # clear gap between the 2nd and 3rd largest: unique answer, not exempt
    assert row_exempt(np.array([5.0, 1.0, 4.0, 0.5]), 2) is None
    # exact tie at the boundary: the lower position wins, not exempt
    assert row_exempt(np.array([5.0, 4.0, 4.0, 0.5]), 2) is None
    # fewer than k + 1 entries: every entry is chosen, nothing to exempt
    assert row_exempt(np.array([1.0, 2.0]), 2) is None
    assert row_exempt(np.array([1.0, 2.0]), 5) is None
    # near tie: a - b = 2e-6 * a < 1e-5 * a
    a, b = 4.0, 4.0 * (1 - 2e-6)
    ex = row_exempt(np.array([5.0, a, b, 0.5]), 2)
    assert ex is not None
    hi, lo = ex
    assert hi == a + TIE_REL * a and lo == b - TIE_REL * b
    # a gap just above the bound is not exempt
    assert row_exempt(np.array([5.0, 4.0, 4.0 * (1 - 2e-5), 0.5]), 2) is None
    # negative boundary scores use |a|
    ex = row_exempt(np.array([-1.0, -1.0 - 3e-6, 7.0]), 2)
    assert ex is not None and ex[0] == -1.0 + TIE_REL and ex[1] == (-1.0 - 3e-6) - TIE_REL * (1.0 + 3e-6)


def test_check_selection_accepts_and_rejects():
    k = 2
    near = np.array([5.0, 4.0, 4.0 * (1 - 2e-6), 0.5, 3.0])
    want = orc.topk_select_row(near, k)
    assert want.tolist() == [0, 1]
    assert check_selection(want, want, near, k) is True
    # the near-tie swap is accepted (and reported as not exact)
    assert check_selection(np.array([0, 2]), want, near, k) is False
    # dropping the clear winner is rejected even on an exempt row
    with pytest.raises(AssertionError):
        check_selection(np.array([1, 2]), want, near, k)
    # picking a position far below the boundary is rejected
    with pytest.raises(AssertionError):
        check_selection(np.array([0, 3]), want, near, k)
    # a duplicate or an unsorted answer is rejected
    with pytest.raises(AssertionError):
        check_selection(np.array([2, 0]), want, near, k)
    # any difference on a row with a clear gap is rejected
    gap = np.array([5.0, 1.0, 4.0, 0.5])
    with pytest.raises(AssertionError):
        check_selection(np.array([0, 1]), orc.topk_select_row(gap, k), gap, k)
    # on an exact tie the tie rule must hold bit for bit
    tie = np.array([5.0, 4.0, 4.0, 0.5])
    with pytest.raises(AssertionError):
        check_selection(np.array([0, 2]), orc.topk_select_row(tie, k), tie, k)
