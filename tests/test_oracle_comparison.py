"""Pins of the comparison rule every sampled GPU result passes through
(oracle.excusal) and of the two batch-driver conventions that GPU parity
otherwise checks only by agreement with the kernel.

The rule: a sampled result equals the oracle's, or differs only at a draw
whose uniform lies within the window (1e-6) of an acceptance threshold or of
a CDF boundary of the final draw, with the token it took of positive mass; a
request whose top-p cut is a near tie is excused whenever it differs.  Every
record here is written out by hand with exact binary fractions, so each
expectation follows from the rule, not from the oracle's own arithmetic.
"""

import numpy as np
import pytest

import oracle
from oracle import F32, ONEHOT, PROBS

W20 = 2.0 ** -20          # an exactly representable window for the edge cases


def _rec(a, margins, k=3, w=(0.25, 0.0, 0.25, 0.5), u=0.25, t=None, near=False):
    w = np.asarray(w, dtype=np.float64)
    C = np.cumsum(w)
    W = float(C[-1])
    if t is None:
        t = int(np.nonzero(C > u * W)[0][0])
    return oracle.SampledRecord(a=a, tokens=[0] * a + [t], p_x=[0.5] * k, q_x=[0.5] * k,
                                theta=[0.5] * k, margins=list(margins), t=t, final_w=w,
                                final_C=C, final_W=W, final_u=u, near_tie=near)


# ---------------------------------------------------------------- accept decisions
def test_identical_result_matches():
    r = _rec(1, [0.1, 0.2])
    assert oracle.excusal(r, 1, r.t) == "match"


def test_gpu_accepts_where_the_oracle_rejected():
    # oracle stops at 1; the GPU accepted position 1 and went on to 2
    assert oracle.excusal(_rec(1, [0.1, 5e-7]), 2, 0) == "excused"
    assert oracle.excusal(_rec(1, [0.1, 2e-6]), 2, 0) == "fail"
    # the margin consulted is the oracle's last examined position, not the
    # GPU's count (which indexes past the examined positions here)
    assert oracle.excusal(_rec(1, [5e-7, 0.3]), 2, 0) == "fail"


def test_gpu_rejects_where_the_oracle_accepted():
    # oracle accepted 0 and stopped at 1; the GPU rejected already at 0
    assert oracle.excusal(_rec(1, [5e-7, 0.3]), 0, 0) == "excused"
    assert oracle.excusal(_rec(1, [2e-6, 5e-7]), 0, 0) == "fail"
    assert oracle.excusal(_rec(1, [0.1, 5e-7]), 0, 0) == "fail"


def test_margin_just_inside_and_outside_the_window():
    assert oracle.excusal(_rec(0, [W20 / 2]), 1, 0, window=W20) == "excused"
    assert oracle.excusal(_rec(0, [W20]), 1, 0, window=W20) == "fail"      # strict <
    assert oracle.excusal(_rec(3, [0.2, 0.2, 9.9e-7]), 2, 0) == "excused"   # all accepted
    assert oracle.excusal(_rec(3, [0.2, 0.2, 1.01e-6]), 2, 0) == "fail"


def test_out_of_range_results_always_fail():
    for near in (False, True):
        r = _rec(1, [5e-7, 5e-7], near=near)
        assert oracle.excusal(r, -1, 0) == "fail"
        assert oracle.excusal(r, 4, 0) == "fail"          # k = 3
        assert oracle.excusal(r, 1, -1) == "fail"
        assert oracle.excusal(r, 1, 4) == "fail"          # V = 4


# ---------------------------------------------------------------- final token
# w = [0.25, 0, 0.25, 0.5], C = [0.25, 0.25, 0.5, 1]: token 0 owns [0, 0.25),
# token 1 nothing, token 2 [0.25, 0.5), token 3 [0.5, 1).
def test_final_token_on_a_boundary():
    r = _rec(1, [0.1, 0.1], u=0.25)
    assert r.t == 2
    assert oracle.excusal(r, 1, 0, window=W20) == "excused"    # upper edge of token 0
    assert oracle.excusal(r, 1, 1, window=W20) == "fail"       # zero mass, empty interval
    assert oracle.excusal(r, 1, 3, window=W20) == "fail"


def test_final_token_upper_edge_is_strict():
    r = _rec(1, [0.1, 0.1], u=0.25 + W20)
    assert r.t == 2
    assert oracle.excusal(r, 1, 0, window=W20) == "fail"
    r = _rec(1, [0.1, 0.1], u=0.25 + W20 / 2)
    assert oracle.excusal(r, 1, 0, window=W20) == "excused"


def test_final_token_lower_edge_is_inclusive():
    r = _rec(1, [0.1, 0.1], u=0.5 - W20)
    assert r.t == 2
    assert oracle.excusal(r, 1, 3, window=W20) == "excused"
    r = _rec(1, [0.1, 0.1], u=0.5 - 2 * W20)
    assert oracle.excusal(r, 1, 3, window=W20) == "fail"


def test_final_token_with_the_default_window():
    assert oracle.excusal(_rec(2, [0.1, 0.1, 0.1], u=0.25 + 5e-7), 2, 0) == "excused"
    assert oracle.excusal(_rec(2, [0.1, 0.1, 0.1], u=0.25 + 2e-6), 2, 0) == "fail"
    assert oracle.excusal(_rec(2, [0.1, 0.1, 0.1], u=0.3), 2, 3) == "fail"


def test_final_token_interval_is_normalised_by_the_total():
    # w = [1, 0, 1, 2]: W = 4, intervals as above after division
    r = _rec(1, [0.1, 0.1], w=(1.0, 0.0, 1.0, 2.0), u=0.5 - W20 / 2)
    assert r.t == 2
    assert oracle.excusal(r, 1, 3, window=W20) == "excused"
    assert oracle.excusal(r, 1, 0, window=W20) == "fail"


def test_zero_mass_token_inside_a_widened_interval_fails():
    # u right at the boundary shared by token 0's end, the empty token 1 and
    # token 2's start: only tokens of positive mass may be excused
    r = _rec(1, [0.1, 0.1], u=0.25)
    assert oracle.excusal(r, 1, 1) == "fail"
    assert oracle.excusal(r, 1, 0) == "excused"


def test_near_tie_request_excused_when_it_differs():
    r = _rec(1, [0.3, 0.3], near=True)
    assert oracle.excusal(r, 3, 3) == "excused"
    assert oracle.excusal(r, 0, 1) == "excused"
    assert oracle.excusal(_rec(1, [0.3, 0.3], near=False), 3, 3) == "fail"


# ---------------------------------------------------------------- batch-driver conventions
def _single(rows, T, kind, drafts, u, q_rows=None):
    k = len(drafts)
    return oracle.verify(np.asarray(rows, dtype=np.float32), F32,
                         np.array([0, k + 1], dtype=np.int32), np.asarray(drafts, np.int32),
                         np.asarray(u, dtype=np.float32), np.array([T], dtype=np.float32),
                         draft=None if q_rows is None else np.asarray(q_rows, np.float32),
                         draft_dtype=F32, draft_kind=np.array([kind]), max_k=8)


@pytest.mark.parametrize("bad", [np.nan, np.inf, -0.125])
def test_probability_row_checked_only_where_the_request_stops(bad):
    """A probability draft's row is read in full only at the position where
    the request stops: a bad value elsewhere in that row is NONFINITE after a
    rejection there, and never looked at after an acceptance.  Uniform target
    rows (p = 1/4 each); q(x_0 = 0) = 0.5, so the acceptance threshold is 0.5."""
    rows = np.zeros((2, 4))
    q = np.array([[0.5, bad, 0.25, 0.25], [0.25, 0.25, 0.25, 0.25]])
    r = _single(rows, 1.0, PROBS, [0], [0.75, 0.625], q_rows=q)       # 0.75 >= 0.5: reject
    assert r.status[0] == oracle.ROW_NONFINITE
    assert r.accepted[0] == -1 and list(r.out_tokens) == [-1, -1]
    assert np.isnan(r.p_at_draft[0]) and np.isnan(r.q_at_draft[0])
    r = _single(rows, 1.0, PROBS, [0], [0.25, 0.625], q_rows=q)       # accept, bonus from p_1
    assert r.status[0] == oracle.ROW_OK and r.accepted[0] == 1
    assert list(r.out_tokens) == [0, 2]                                # 0.625 in [0.5, 0.75)
    assert r.p_at_draft[0] == 0.25 and r.q_at_draft[0] == 0.5


def test_greedy_rows_report_indicator_probabilities():
    """Greedy requests in the sampled entry report p_i(x_i) = 1 when x_i is the
    row's argmax and 0 otherwise, q_i(x_i) = 1, at every draft position (also
    past the first mismatch)."""
    rows = np.full((4, 5), -1.0)
    rows[0, 2] = rows[1, 0] = rows[2, 1] = rows[3, 4] = 3.0
    r = _single(rows, 0.0, ONEHOT, [2, 1, 1], [0.9] * 4)
    assert r.status[0] == oracle.ROW_OK and r.accepted[0] == 1
    assert list(r.out_tokens) == [2, 0, -1, -1]
    assert list(r.p_at_draft) == [1.0, 0.0, 1.0]
    assert list(r.q_at_draft) == [1.0, 1.0, 1.0]
