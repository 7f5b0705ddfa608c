"""The routing comparison of the GPU tests must reject every wrong row.

check_routing judges a GPU top-k row against the oracle's fp64 logits alone;
these cases plant the mistakes a selection kernel could make (a repeated
expert, a swapped pair, a better expert left out, an exact tie taken in the
wrong order, an index out of range) and check that each one fails, while the
correct rows and a genuine near-tie pass.
"""
import numpy as np
import pytest

from moe_testlib import check_routing

L = np.array([[0.5, 0.9, 0.1, 0.9, -0.3, 0.7],
              [1.0, 1.0 + 1e-15, 0.2, -1.0, 0.3, 0.0]])
SCALE = np.array([1.0, 1.0])


def _ok(rows):
    return check_routing(np.array(rows), None, L, "case", scale=SCALE)


def test_correct_rows_pass():
    # row 0: 0.9 (1) and 0.9 (3) tie exactly -> 1 before 3; row 1: 1+1e-15 beats 1.0
    _ok([[1, 3, 5], [1, 0, 4]])


def test_near_tie_may_come_either_way():
    # 1.0 and 1.0 + 1e-15 differ by far less than 1e-12 of the scale
    _ok([[1, 3, 5], [0, 1, 4]])


@pytest.mark.parametrize("rows", [
    [[1, 1, 3], [1, 0, 4]],        # repeated expert
    [[3, 1, 5], [1, 0, 4]],        # exact tie in the wrong order
    [[1, 5, 3], [1, 0, 4]],        # order broken (0.7 before 0.9)
    [[1, 3, 0], [1, 0, 4]],        # 0.5 chosen over 0.7
    [[1, 3, 5], [1, 0, 2]],        # 0.2 chosen over 0.3
    [[1, 3, 6], [1, 0, 4]],        # index out of range
])
def test_wrong_rows_fail(rows):
    with pytest.raises(AssertionError):
        _ok(rows)


def test_exact_tie_at_the_boundary_needs_the_lower_index():
    Lb = np.array([[0.9, 0.4, 0.4, 0.1]])
    check_routing(np.array([[0, 1]]), None, Lb, "b", scale=np.array([1.0]))
    with pytest.raises(AssertionError):
        check_routing(np.array([[0, 2]]), None, Lb, "b", scale=np.array([1.0]))
