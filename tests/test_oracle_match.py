"""Pins of the prefix-match verify of argmax drafts (draft kind MATCH): every
verify row is sampled as decode samples it, with the row's own uniform, and
the drafts are accepted while each equals its row's sample (FreeToken PR #836,
Design: the rejection row and the bullet on argmax drafts).

* Law, by exact enumeration at V=8, k=2: the u-space of each row's draw is a
  finite union of inverse-CDF intervals; the oracle is evaluated at every
  interval midpoint of every row and the branch masses are summed.  The
  committed sequence must follow the target law (losslessness, the theorem of
  the Draft-Model-Sampling page, Key Topic 2) and equal, sequence by sequence,
  the law of sampled mode with one-hot drafts (the equivalence the PR page
  states).
* Pointwise: each row's sample is numpy's searchsorted over the row's running
  sum (a library routine), and one-hot target rows reduce it to greedy.
"""

import itertools

import numpy as np
import pytest

import oracle
from oracle import F32, MATCH, ONEHOT
from test_oracle_laws import FAMILIES, _check_lossless, _final_intervals, enumerate_law

V, K = 8, 2
TOL = 1e-12


def match_law(p_rows, xs):
    """Exact law of the committed sequence under oracle.match_request, by
    enumerating the product of every row's inverse-CDF intervals."""
    law = {}
    per_row = [_final_intervals(p_rows[j]) for j in range(K + 1)]
    for combo in itertools.product(*per_row):
        mass = 1.0
        u = []
        for (_, lo, hi) in combo:
            mass *= hi - lo
            u.append((lo + hi) / 2)
        rec = oracle.match_request(p_rows, xs, u)
        # the branch the midpoints stand for: accept while the row's interval is x's
        a = K
        for j in range(K):
            if combo[j][0] != xs[j]:
                a = j
                break
        assert rec.a == a and rec.t == combo[a][0], (xs, combo, rec.a, rec.t)
        key = tuple(rec.tokens)
        law[key] = law.get(key, 0.0) + mass
    return law


@pytest.mark.parametrize("name", ["random_T1", "T0.6_topk5_topp0.8", "peaked_q"])
@pytest.mark.parametrize("xs", [(0, 0), (3, 5), (7, 2), (1, 1)])
def test_match_law_is_lossless_and_equals_onehot_sampled_mode(name, xs):
    p_rows, _ = FAMILIES[name]
    law = match_law(p_rows, xs)
    _check_lossless(law, p_rows, K)
    onehot = enumerate_law(p_rows, [np.eye(V)[xs[0]], np.eye(V)[xs[1]]], iter([(xs, 1.0)]),
                           check_oracle=False)
    for key in set(law) | set(onehot):
        assert abs(law.get(key, 0.0) - onehot.get(key, 0.0)) < TOL, key
    # acceptance law: P(a >= j) = prod_{i<j} p_i(x_i)
    for j in range(K + 1):
        reach = sum(pr for seq, pr in law.items() if len(seq) >= j + 1)
        assert abs(reach - np.prod([p_rows[i][xs[i]] for i in range(j)])) < TOL


def test_each_row_sample_is_searchsorted():
    rng = np.random.default_rng(21)
    for _ in range(300):
        k = int(rng.integers(0, 6))
        n = int(rng.integers(2, 40))
        rows = [oracle.process(rng.normal(0, 2, n), 0.8).p for _ in range(k + 1)]
        u = (rng.integers(0, 1 << 24, size=k + 1) * 2.0 ** -24).tolist()
        ys = [int(np.searchsorted(np.cumsum(r), uj * np.cumsum(r)[-1], side="right"))
              for r, uj in zip(rows, u)]
        # drafts agree with the samples up to a planted position
        plant = int(rng.integers(0, k + 1))
        xs = [ys[j] if j != plant else (ys[j] + 1) % n for j in range(k)]
        rec = oracle.match_request(rows, xs, u)
        assert rec.a == min(plant, k)
        assert rec.tokens == xs[:rec.a] + [ys[rec.a]]


def test_margins_are_distances_to_the_draft_interval():
    # p = [0.25, 0.25, 0.5]: token 1 owns [0.25, 0.5)
    p = np.array([0.25, 0.25, 0.5])
    rec = oracle.match_request([p, p], [1], [0.3, 0.7])
    assert rec.a == 1 and rec.tokens == [1, 2]
    assert abs(rec.margins[0] - 0.05) < 1e-15
    rec = oracle.match_request([p, p], [1], [0.5, 0.1])        # u at the upper end: mismatch
    assert rec.a == 0 and rec.tokens == [2]
    assert rec.margins[0] == 0.0
    assert rec.final_u == 0.5 and rec.margin_final == 0.0


def _single(rows, T, drafts, u, kind=MATCH):
    k = len(drafts)
    return oracle.verify(np.asarray(rows, dtype=np.float32), F32,
                         np.array([0, k + 1], dtype=np.int32), np.asarray(drafts, np.int32),
                         np.asarray(u, dtype=np.float32), np.array([T], dtype=np.float32),
                         draft_kind=np.array([kind]), max_k=8)


def test_one_hot_targets_reduce_match_to_greedy():
    rng = np.random.default_rng(22)
    for _ in range(50):
        n, k = 12, 3
        rows = np.full((k + 1, n), -np.inf)
        g = rng.integers(0, n, size=k + 1)
        rows[np.arange(k + 1), g] = rng.normal(size=k + 1)
        xs = [int(g[j]) if rng.random() < 0.7 else int((g[j] + 1) % n) for j in range(k)]
        u = (rng.integers(0, 1 << 24, size=k + 1) * 2.0 ** -24).astype(np.float32)
        got = _single(rows, 0.9, xs, u)
        ref = _single(rows, 0.0, xs, u, kind=ONEHOT)        # greedy request
        assert got.status[0] == 0 and got.accepted[0] == ref.accepted[0]
        assert np.array_equal(got.out_tokens, ref.out_tokens)


def test_verify_reports_p_and_unit_q_for_match_requests():
    rows = np.log(np.array([[0.25, 0.25, 0.5], [0.5, 0.25, 0.25]]))
    r = _single(rows, 1.0, [1], [0.3, 0.6])
    assert r.status[0] == 0 and r.accepted[0] == 1
    assert list(r.out_tokens) == [1, 1]                  # row 1: 0.6 in [0.5, 0.75)
    assert abs(r.p_at_draft[0] - 0.25) < 1e-7 and r.q_at_draft[0] == 1.0
    r = _single(rows, 1.0, [1], [0.2, 0.6])              # row 0 samples token 0
    assert r.accepted[0] == 0 and list(r.out_tokens) == [0, -1]
