"""Pins of the oracle's presence / frequency penalties (FreeToken PR #836,
section "Design": penalties are applied per verify row, the drafts before a
row counted as already generated; its test list asks for exactly that).

The pages name the penalties but not their formula; the oracle takes the
usual additive form l' = l - (frequency * c + presence) for every token with
count c > 0, in fp64, rounded to fp32 and then to the logits' dtype.  These
pins fix that reading with hand-worked numbers and closed forms, chosen so
that the plausible mistakes fail: counting the row's own draft or all drafts,
skipping the presence term, penalizing draft rows, the wrong rounding mode,
unpenalized argmax for greedy requests."""

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import BF16, F32, LOGITS, MATCH, ONEHOT, ROW_NONFINITE, ROW_OK

B1 = np.array([0, 0], dtype=np.int32)


def _one(rows, drafts, T=1.0, kind=ONEHOT, dtype=F32, presence=0.0, frequency=0.0,
         hist=((), ()), u=None, draft=None):
    rows = np.atleast_2d(np.asarray(rows, dtype=np.float64))
    k = rows.shape[0] - 1
    tgt = rows.astype(np.float32) if dtype == F32 else oracle_bf16_bits(rows)
    ht, hc = hist
    return oracle.verify(tgt, dtype, np.array([0, k + 1]), np.asarray(drafts, np.int32),
                         uniforms=np.asarray(u if u is not None else [0.5] * (k + 1), np.float32),
                         temperature=np.array([T], np.float32), draft=draft, draft_dtype=F32,
                         draft_kind=np.array([kind], np.int32), max_k=8,
                         presence=np.array([presence], np.float32),
                         frequency=np.array([frequency], np.float32),
                         hist_offsets=np.array([0, len(ht)], np.int32),
                         hist_tokens=np.asarray(ht, np.int32), hist_counts=np.asarray(hc, np.int32))


def oracle_bf16_bits(rows):
    """Exactly representable bf16 values -> their bit patterns (the upper
    half of the fp32 pattern)."""
    f = np.asarray(rows, dtype=np.float32)
    assert np.all(f.view(np.uint32) & 0xFFFF == 0), "test values must be bf16 values"
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------- hand-worked rows
ROW = np.array([0.5, 1.0, 2.0, -1.0, 1.5, 0.0])
HIST = ([2, 4], [3, 1])
# frequency 0.5, presence 1.0; drafts x = [4, 1]
EXPECT = [
    [0.5, 1.0, -0.5, -1.0, 0.0, 0.0],     # row 0: history only (2: 3, 4: 1)
    [0.5, 1.0, -0.5, -1.0, -0.5, 0.0],    # row 1: x_0 = 4 counted (4: 2)
    [0.5, -0.5, -0.5, -1.0, -0.5, 0.0],   # row 2: x_1 = 1 counted too (1: 1)
]


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_hand_worked_rows(dtype):
    xs = np.array([4, 1])
    for j in range(3):
        got = oracle.penalize(ROW.copy(), dtype, *HIST, xs[:j], presence=1.0, frequency=0.5)
        assert got.tolist() == EXPECT[j]
    res = _one(np.tile(ROW, (3, 1)), [4, 1], dtype=dtype, presence=1.0, frequency=0.5, hist=HIST)
    assert res.status[0] == ROW_OK
    assert res.p_at_draft[0] == np.float32(scipy.special.softmax(EXPECT[0])[4])
    assert res.p_at_draft[1] == np.float32(scipy.special.softmax(EXPECT[1])[1])


def test_only_the_drafts_before_a_row_count():
    """Uniform logits, no history, drafts [1, 1], frequency 1: row 0 sees no
    count, row 1 one, row 2 two."""
    rows = np.zeros((3, 4))
    res = _one(rows, [1, 1], frequency=1.0)
    e1, e2 = np.exp(-1.0), np.exp(-2.0)
    assert res.p_at_draft[0] == np.float32(0.25)
    assert res.p_at_draft[1] == np.float32(e1 / (3 + e1))
    row2 = oracle.penalize(np.zeros(4), F32, [], [], [1, 1], presence=0.0, frequency=1.0)
    assert row2.tolist() == [0.0, -2.0, 0.0, 0.0]


def test_presence_counts_once_frequency_per_occurrence():
    got = oracle.penalize(np.zeros(5), F32, [0, 3], [4, 0], [2, 2, 2], presence=0.75,
                          frequency=0.25)
    # token 0: count 4 -> 1.0 + 0.75; token 3: count 0 -> untouched; token 2: 3 -> 0.75 + 0.75
    assert got.tolist() == [-1.75, 0.0, -1.5, 0.0, 0.0]


def test_zero_penalties_change_nothing():
    rng = np.random.default_rng(3)
    V, k = 50, 4
    rows = np.round(rng.normal(0, 2, size=(k + 1, V)), 2)
    draft = np.round(rows[:k] + rng.normal(0, 0.5, size=(k, V)), 2)
    xs = [int(np.argmax(d)) for d in draft]
    u = rng.random(k + 1).tolist()
    base = _one(rows, xs, kind=LOGITS, u=u, draft=draft.astype(np.float32))
    pen = _one(rows, xs, kind=LOGITS, u=u, draft=draft.astype(np.float32), hist=([1, 2], [5, 5]))
    assert base.accepted.tolist() == pen.accepted.tolist()
    assert base.out_tokens.tolist() == pen.out_tokens.tolist()
    assert base.p_at_draft.tolist() == pen.p_at_draft.tolist()


def test_draft_rows_are_not_penalized():
    """q(x) is the drafter's own distribution: penalties leave it alone."""
    rng = np.random.default_rng(4)
    V, k = 12, 2
    rows = np.round(rng.normal(size=(k + 1, V)), 2)
    draft = np.round(rng.normal(size=(k, V)), 2).astype(np.float32)
    xs = [3, 3]
    plain = _one(rows, xs, kind=LOGITS, draft=draft)
    pen = _one(rows, xs, kind=LOGITS, draft=draft, presence=2.0, frequency=1.0, hist=([3], [2]))
    assert pen.q_at_draft.tolist() == plain.q_at_draft.tolist()
    assert pen.p_at_draft[0] < plain.p_at_draft[0]


def test_huge_presence_blocks_every_seen_token():
    rng = np.random.default_rng(5)
    V = 16
    row = rng.normal(size=V)
    seen = [3, 7]
    for j, before in enumerate(([], [9], [9, 11])):
        pr = oracle.process(oracle.penalize(row, F32, seen, [1, 1], before, presence=1e4,
                                            frequency=0.0), 1.0).p
        blocked = seen + list(before)
        assert np.all(pr[blocked] == 0.0)
        free = np.setdiff1d(np.arange(V), blocked)
        assert abs(pr[free].sum() - 1.0) < 1e-15


def test_bf16_rounding_is_nearest_even():
    """1 - 2^-9 lies halfway between the bf16 values 1 - 2^-8 and 1: ties go to
    the even one, 1.0; 1 - 3 * 2^-10 is nearer 1 - 2^-8."""
    row = np.array([1.0, 0.0])
    assert oracle.penalize(row, BF16, [0], [1], [], 0.0, 2.0 ** -9)[0] == 1.0
    assert oracle.penalize(row, BF16, [0], [1], [], 0.0, 3 * 2.0 ** -10)[0] == 1.0 - 2.0 ** -8
    assert oracle.penalize(row, BF16, [0], [1], [], 2.0 ** -9 + 2.0 ** -12, 0.0)[0] == \
        1.0 - 2.0 ** -8
    # fp32 rows: 1 - 2^-30 rounds to 1, 1 - 2^-23 is a float
    assert oracle.penalize(row, F32, [0], [1], [], 0.0, 2.0 ** -30)[0] == 1.0
    assert oracle.penalize(row, F32, [0], [1], [], 0.0, 2.0 ** -23)[0] == 1.0 - 2.0 ** -23


def test_greedy_requests_take_the_penalized_argmax():
    rows = np.array([[1.0, 5.0, 3.0, 2.0]] * 2)
    res = _one(rows, [2], T=0.0, frequency=2.5, hist=([1], [1]))
    # row 0: [1, 2.5, 3, 2] -> 2 = x_0, accepted; row 1: 2 counted -> [1, 2.5, 0.5, 2] -> 1
    assert res.accepted[0] == 1 and res.out_tokens.tolist() == [2, 1]


def test_match_requests_sample_the_penalized_rows():
    rows = np.zeros((2, 4))
    # row 0 after presence 1e4 on tokens 0..2: all mass on 3, so any uniform draws 3
    res = _one(rows, [3], kind=MATCH, presence=1e4, hist=([0, 1, 2], [1, 1, 1]), u=[0.999, 0.3])
    assert res.accepted[0] == 1
    # row 1 also counts x_0 = 3: every token is penalized alike, uniform again
    assert res.out_tokens[1] == int(np.searchsorted(np.cumsum([0.25] * 4), 0.3 * 1.0, "right"))


def test_nonfinite_penalties_and_ignored_history():
    rows = np.zeros((2, 4))
    assert _one(rows, [1], presence=np.nan).status[0] == oracle.ROW_BAD_PARAM
    assert _one(rows, [1], frequency=np.inf).status[0] == oracle.ROW_BAD_PARAM
    # both zero: no penalty, so a NaN-free OK request
    assert _one(rows, [1]).status[0] == ROW_OK
    base = _one(rows, [1], presence=1.0, hist=([2], [1]))
    junk = _one(rows, [1], presence=1.0, hist=([2, -1, 4, 3], [1, 5, 5, -2]))
    assert base.p_at_draft.tolist() == junk.p_at_draft.tolist()
    # offsets out of order: no history at all
    res = oracle.verify(np.zeros((2, 4), np.float32), F32, np.array([0, 2]),
                        np.array([1], np.int32), uniforms=np.full(2, 0.5, np.float32),
                        temperature=np.ones(1, np.float32), draft_kind=np.zeros(1, np.int32),
                        presence=np.ones(1, np.float32), frequency=np.zeros(1, np.float32),
                        hist_offsets=np.array([1, 0], np.int32),
                        hist_tokens=np.array([1], np.int32), hist_counts=np.array([1], np.int32))
    assert res.p_at_draft[0] == np.float32(0.25)


def test_a_negative_penalty_can_overflow_to_inf():
    rows = np.array([[3.0e38, 0.0], [0.0, 0.0]])
    res = _one(rows, [0], presence=-1.0e38, hist=([0], [1]))
    assert res.status[0] == ROW_NONFINITE
