"""Pins of the steps after the verify: the drain (commit n = a + 1 tokens,
give back the unused verify slots; FreeToken PR #836, Design, drain row; the
catalog page's coupling point 1, accept all / some / none) and the acceptance
accounting (the Rust page's three counters and its adaptive lookahead,
Production Pitfalls item 3; the draft-sampling page's expected tokens per
step, Key Topic 4)."""

import numpy as np
import pytest

import oracle
from oracle import F32, LOGITS, ROW_BAD_K, ROW_NONFINITE, ROW_OK


# ---------------------------------------------------------------- drain
def test_drain_accept_all_some_none_fault_and_bad_offsets():
    # k = 3, 2, 4, 1, 2 (request 4's offsets were rejected by the verify)
    cu = np.array([0, 4, 7, 12, 14, 17])
    out = np.array([10, 11, 12, 13,   20, 21, -1,   30, -1, -1, -1, -1,   -1, -1,   -1, -1, -1])
    acc = np.array([3, 1, 0, -1, -1])
    st = np.array([ROW_OK, ROW_OK, ROW_OK, ROW_NONFINITE, ROW_BAD_K])
    committed, offsets, rollback = oracle.drain(cu, acc, st, out)
    assert committed.tolist() == [10, 11, 12, 13, 20, 21, 30]
    assert offsets.tolist() == [0, 4, 6, 7, 7, 7]
    assert rollback.tolist() == [0, 1, 4, 2, 0]


def test_drain_rejects_an_accepted_count_outside_the_request():
    cu = np.array([0, 3])
    c, o, r = oracle.drain(cu, np.array([5]), np.array([ROW_OK]), np.arange(3))
    assert c.tolist() == [] and o.tolist() == [0, 0] and r.tolist() == [3]
    # rows outside the token buffer: nothing committed, nothing given back
    c, o, r = oracle.drain(np.array([0, 5]), np.array([1]), np.array([ROW_OK]), np.arange(3))
    assert c.tolist() == [] and o.tolist() == [0, 0] and r.tolist() == [0]
    # an INTERNAL request defines only its status: its accepted count is not trusted
    c, o, r = oracle.drain(cu, np.array([1]), np.array([oracle.ROW_INTERNAL]), np.arange(3))
    assert c.tolist() == [] and o.tolist() == [0, 0] and r.tolist() == [3]


def test_drain_invariants_on_random_batches():
    rng = np.random.default_rng(3)
    for _ in range(200):
        B = int(rng.integers(1, 30))
        ks = rng.integers(0, 9, size=B)
        cu = np.concatenate([[0], np.cumsum(ks + 1)])
        acc = np.array([int(rng.integers(0, k + 1)) for k in ks])
        st = rng.choice([ROW_OK, ROW_OK, ROW_OK, ROW_NONFINITE, ROW_BAD_K], size=B)
        out = rng.integers(0, 1000, size=int(cu[-1]))
        committed, offsets, rollback = oracle.drain(cu, acc, st, out)
        n = np.diff(offsets)
        assert offsets[0] == 0 and np.all(n >= 0) and committed.shape[0] == offsets[-1]
        for b in range(B):
            if st[b] == ROW_OK:
                assert n[b] == acc[b] + 1 and rollback[b] == ks[b] - acc[b]
                assert committed[offsets[b]:offsets[b + 1]].tolist() == \
                    out[cu[b]:cu[b] + acc[b] + 1].tolist()
            elif st[b] == ROW_BAD_K:
                assert n[b] == 0 and rollback[b] == 0
            else:
                assert n[b] == 0 and rollback[b] == ks[b] + 1


def _verify_batch(L, D, xs_list, u_list, T=1.0):
    """B requests with the same rows L (k+1) and D (k), drafts and uniforms per
    request, through the oracle's verify."""
    k = D.shape[0]
    B = len(xs_list)
    cu = np.arange(0, (k + 1) * (B + 1), k + 1)
    res = oracle.verify(np.tile(L, (B, 1)).astype(np.float32), F32, cu,
                        np.concatenate(xs_list).astype(np.int32),
                        np.concatenate(u_list).astype(np.float32), np.full(B, T, np.float32),
                        draft=np.tile(D, (B, 1)).astype(np.float32), draft_dtype=F32,
                        draft_kind=np.full(B, LOGITS), max_k=k)
    return cu, res


def test_drain_at_the_zero_and_full_acceptance_edges():
    """The catalog's Acceptance bars item 3: p = q accepts every draft (n = k+1,
    nothing given back); disjoint supports accept none (n = 1, k given back)."""
    rng = np.random.default_rng(5)
    k, V, B = 4, 12, 25
    L = rng.normal(size=(k + 1, V))
    xs = [rng.integers(0, V, size=k) for _ in range(B)]
    us = [(rng.integers(0, 1 << 24, size=k + 1) * 2.0 ** -24) for _ in range(B)]
    cu, res = _verify_batch(L, L[:k], xs, us)
    _, offsets, rollback = oracle.drain(cu, res.accepted, res.status, res.out_tokens)
    assert np.all(np.diff(offsets) == k + 1) and np.all(rollback == 0)
    Ld = L.copy()
    Ld[:, 6:] = -np.inf
    D = L[:k].copy()
    D[:, :6] = -np.inf
    xs = [rng.integers(6, V, size=k) for _ in range(B)]
    cu, res = _verify_batch(Ld, D, xs, us)
    _, offsets, rollback = oracle.drain(cu, res.accepted, res.status, res.out_tokens)
    assert np.all(np.diff(offsets) == 1) and np.all(rollback == k)


# ---------------------------------------------------------------- accounting
def test_accounting_by_hand():
    # k = 4, 3, 0, 2, 2; request 3 faulted
    cu = np.array([0, 5, 9, 10, 13, 16])
    acc = np.array([1, 3, 0, -1, 0])
    st = np.array([ROW_OK, ROW_OK, ROW_OK, ROW_NONFINITE, ROW_OK])
    ema = np.array([0.5, 0.5, 0.9, 0.1, 0.8], dtype=np.float32)
    e, kn, cnt = oracle.accounting(cu, acc, st, ema, 0.5, 0.4, 2, 5, np.array([100, 200, 50, 10]))
    # a request that ended INTERNAL with a count that looks valid is not accounted
    st2 = st.copy()
    st2[1] = oracle.ROW_INTERNAL
    e2, _, cnt2 = oracle.accounting(cu, acc, st2, ema, 0.5, 0.4, 2, 5, np.zeros(4))
    assert e2[1] == ema[1] and cnt2.tolist() == [2 + 1 + 1, 4 + 0 + 2, 1, 3]
    # r = 1/4, 3/3, (k=0), (fault), 0/2
    assert e.tolist() == np.array([0.375, 0.75, 0.9, 0.1, 0.4], np.float32).tolist()
    assert kn.tolist() == [2, 5, 5, 2, 5]                  # 0.4 is not below 0.4
    assert cnt.tolist() == [100 + 2 + 4 + 1 + 1, 200 + 4 + 3 + 0 + 2, 50 + 1 + 3 + 0 + 0, 10 + 4]


def test_moving_average_closed_form_and_lookahead_switch():
    """A constant rate r drives the average to r geometrically,
    ema_n = r + (ema_0 - r)(1 - beta)^n; the lookahead drops to k_low once the
    average is below the threshold and returns to k_high after it recovers."""
    beta, thr = 0.25, 0.4
    cu = np.array([0, 6])
    ema = np.array([0.9], np.float32)
    ks = []
    for n in range(1, 13):
        ema, kn, _ = oracle.accounting(cu, np.array([1]), np.array([ROW_OK]), ema, beta, thr,
                                       2, 5, np.zeros(4))
        assert abs(float(ema[0]) - (0.2 + 0.7 * 0.75 ** n)) < 1e-6
        ks.append(int(kn[0]))
    assert ks[0] == 5 and ks[-1] == 2 and ks == sorted(ks, reverse=True)
    for _ in range(12):
        ema, kn, _ = oracle.accounting(cu, np.array([5]), np.array([ROW_OK]), ema, beta, thr,
                                       2, 5, np.zeros(4))
    assert int(kn[0]) == 5


def test_counters_reproduce_expected_tokens_per_step():
    """Key Topic 4 of the draft-sampling page: with the same acceptance rate
    alpha at every position, tokens per step average (1 - alpha^(k+1)) /
    (1 - alpha).  Oracle verify steps with x ~ q, accounted: the counters'
    generated / requests lands within 4 standard errors of the formula."""
    rng = np.random.default_rng(9)
    k, V, B, steps = 4, 8, 400, 10
    Lrow = rng.normal(0, 1.2, size=V)
    Drow = Lrow + rng.normal(0, 0.9, size=V)
    L = np.tile(Lrow, (k + 1, 1))
    D = np.tile(Drow, (k, 1))
    p = oracle.process(Lrow, 1.0).p
    q = oracle.process(Drow, 1.0).p
    alpha = oracle.acceptance_rate(p, q)
    cnt = np.zeros(4, np.int64)
    per = []
    for _ in range(steps):
        xs = [rng.choice(V, size=k, p=q) for _ in range(B)]
        us = [(rng.integers(0, 1 << 24, size=k + 1) * 2.0 ** -24) for _ in range(B)]
        cu, res = _verify_batch(L, D, xs, us)
        _, _, cnt = oracle.accounting(cu, res.accepted, res.status, np.zeros(B, np.float32),
                                      0.1, 0.4, 2, 5, cnt)
        per.extend((res.accepted + 1).tolist())
    mean = cnt[0] / cnt[3]
    se = np.std(per) / np.sqrt(len(per))
    assert cnt[3] == B * steps and cnt[1] == k * B * steps
    assert abs(mean - oracle.expected_tokens_per_step(alpha, k)) < 4 * se
    assert abs(cnt[2] / cnt[1] - (mean - 1) / k) < 1e-12
