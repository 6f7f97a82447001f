"""Host-side logic of the loop driver (no GPU): the error-history check."""

import pytest
import torch

from post_weight_quantization_06_amd.quantize import check_history


def _h(rows):
    return torch.tensor(rows, dtype=torch.float64)[:, None]


def test_half_step_history_passes_a_descent():
    # assign 0, refine 0, assign 1, refine 1, assign 2, refine 2 (bf16: may rise), final assign
    check_history(_h([10.0, 9.0, 8.0, 7.0, 6.0, 6.5, 6.2]))


@pytest.mark.parametrize("row,value", [(1, 10.5), (3, 8.5), (4, 7.5), (6, 6.6)])
def test_half_step_history_rejects_a_rise(row, value):
    h = _h([10.0, 9.0, 8.0, 7.0, 6.0, 6.5, 6.2])
    h[row, 0] = value
    with pytest.raises(RuntimeError, match="from history row %d to %d" % (row - 1, row)):
        check_history(h)


def test_only_the_last_refine_may_rise():
    # the bf16 refine (row 5) is above its assign (row 4): allowed; the same rise one step
    # earlier is not
    check_history(_h([10.0, 9.0, 8.0, 7.0, 6.0, 6.5, 6.2]))
    with pytest.raises(RuntimeError):
        check_history(_h([10.0, 9.0, 8.0, 8.2, 7.0, 7.5, 7.2]))


def test_slack_is_relative_plus_w2():
    # within 1e-6 of the earlier value: accepted; the W2 term widens it further
    check_history(_h([1.0, 1.0 + 0.9e-6, 1.0, 1.0, 1.0]))
    with pytest.raises(RuntimeError):
        check_history(_h([1.0, 1.0 + 2e-6, 1.0, 1.0, 1.0]))
    check_history(_h([1.0, 1.0 + 2e-6, 1.0, 1.0, 1.0]),
                  w2=torch.tensor([2e7], dtype=torch.float64))


def test_assign_only_history():
    # one row per iteration's assignment and a last row against the bf16 tables (not compared)
    check_history(_h([10.0, 9.0, 8.5, 9.0]), half_steps=False)
    with pytest.raises(RuntimeError):
        check_history(_h([10.0, 11.0, 8.0, 9.0]), half_steps=False)


def test_several_matrices_name_the_one_that_rose():
    h = torch.tensor([[3.0, 5.0], [2.0, 6.0], [1.5, 4.0], [1.4, 4.5], [1.0, 4.0]],
                     dtype=torch.float64)
    with pytest.raises(RuntimeError, match="matrix 1 from history row 0 to 1"):
        check_history(h)
