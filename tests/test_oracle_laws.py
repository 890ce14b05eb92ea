"""Law-level pins of the oracle: exact enumeration of the committed-token
distribution at V=8, k=2 (losslessness, the theorem stated on the Draft-Model
-Sampling page, Key Topic 2, and on the Rust page, section "The Memory
Bandwidth Wall and Speculative Math"), the acceptance law and its closed form
(Key Topic 4), the one-hot invariant (FreeToken PR #836, Design: with argmax
drafts, drawing every verify row and keeping the prefix that agrees with the
drafts has the law of rejection sampling), the
greedy degenerate case (catalog page, Verification and sampling item 2) and
the 0 % / 100 % acceptance edges (catalog page, Acceptance bars item 3).

The u-space of every draw is a finite union of intervals: accept [0, theta),
reject [theta, 1), final token t [C_{t-1}/W, C_t/W).  The test enumerates
every draft tuple and every interval, checks that the oracle evaluated at the
interval midpoint takes that branch, and sums the exact branch masses.
"""

import itertools

import numpy as np
import pytest

import oracle

V, K = 8, 2
TOL = 1e-12


def _theta(px, qx):
    if qx > 0:
        return min(1.0, px / qx)
    return 1.0 if px > 0 else 0.0


def _final_intervals(w):
    C = np.cumsum(w)
    W = C[-1]
    out = []
    for t in range(len(w)):
        if w[t] > 0:
            lo = (C[t - 1] if t > 0 else 0.0) / W
            out.append((t, lo, C[t] / W))
    return out


def enumerate_law(p_rows, q_rows, drafts_iter, check_oracle=True):
    """Exact law of the committed sequence.

    drafts_iter yields (x_tuple, weight).  Returns {committed tuple: prob}.
    """
    law = {}
    k = len(q_rows)
    for xs, wx in drafts_iter:
        if wx == 0:
            continue
        reach = wx
        for a in range(k + 1):
            if a < k:
                th = _theta(p_rows[a][xs[a]], q_rows[a][xs[a]])
                pm = reach * (1.0 - th)
                if pm > 0:
                    w = np.maximum(0.0, p_rows[a] - q_rows[a])
                    if w.sum() == 0:
                        w = p_rows[a]
                    _accumulate(law, xs, a, w, pm, p_rows, q_rows, check_oracle, th)
                reach = reach * th
                if reach == 0:
                    break
            else:
                _accumulate(law, xs, k, p_rows[k], reach, p_rows, q_rows, check_oracle, None)
    return law


def _accumulate(law, xs, a, w, mass, p_rows, q_rows, check, th_reject):
    k = len(q_rows)
    for t, lo, hi in _final_intervals(w):
        law_key = tuple(xs[:a]) + (t,)
        law[law_key] = law.get(law_key, 0.0) + mass * (hi - lo)
        if check:
            u = []
            for i in range(a):
                u.append(_theta(p_rows[i][xs[i]], q_rows[i][xs[i]]) / 2)
            if a < k:
                u.append((th_reject + 1.0) / 2)
                u.extend([0.5] * (k - a - 1))
            u.append((lo + hi) / 2)
            rec = oracle.sampled_request(p_rows, q_rows, xs, u)
            assert rec.a == a and rec.t == t, (xs, a, t, rec.a, rec.t)


def _draft_tuples(q_rows):
    k = len(q_rows)
    for xs in itertools.product(range(V), repeat=k):
        w = 1.0
        for i in range(k):
            w *= q_rows[i][xs[i]]
        yield xs, w


def _check_lossless(law, p_rows, k):
    """P(a >= j, y_0..y_j = t_0..t_j) = P(a >= j, y_0..y_{j-1} = t_0..t_{j-1}) p_j(t_j)."""
    total = sum(law.values())
    assert abs(total - 1.0) < TOL
    for j in range(k + 1):
        prefix_mass = {}
        full_mass = {}
        for seq, pr in law.items():
            if len(seq) >= j + 1:
                full_mass[seq[:j + 1]] = full_mass.get(seq[:j + 1], 0.0) + pr
                prefix_mass[seq[:j]] = prefix_mass.get(seq[:j], 0.0) + pr
        for pre, m in prefix_mass.items():
            for t in range(V):
                got = full_mass.get(pre + (t,), 0.0)
                assert abs(got - m * p_rows[j][t]) < TOL, (j, pre, t, got, m * p_rows[j][t])


def _p_at_least(law, j):
    return sum(pr for seq, pr in law.items() if len(seq) >= j + 1)


def _families():
    rng = np.random.default_rng(11)
    fam = {}
    L = rng.normal(0, 1.5, size=(K + 1, V))
    D = L[:K] + rng.normal(0, 0.8, size=(K, V))
    fam["random_T1"] = ([oracle.process(r, 1.0).p for r in L],
                        [oracle.process(r, 1.0).p for r in D])
    fam["T0.6_topk5_topp0.8"] = ([oracle.process(r, 0.6, 5, 0.8).p for r in L],
                                 [oracle.process(r, 0.6, 5, 0.8).p for r in D])
    P = [oracle.process(r, 1.3).p for r in L]
    fam["p_equals_q"] = (P, [P[0], P[1]])
    Lm = L.copy()
    Lm[:, 4:] = -np.inf
    Dm = D.copy()
    Dm[:, :4] = -np.inf
    fam["disjoint"] = ([oracle.process(r, 1.0).p for r in Lm],
                       [oracle.process(r, 1.0).p for r in Dm])
    Q = rng.dirichlet(np.ones(V) * 0.3, size=K)
    fam["peaked_q"] = ([oracle.process(r, 0.9).p for r in L], list(Q))
    return fam


FAMILIES = _families()


@pytest.mark.parametrize("name", list(FAMILIES))
def test_exact_enumeration_law_is_target(name):
    p_rows, q_rows = FAMILIES[name]
    law = enumerate_law(p_rows, q_rows, _draft_tuples(q_rows))
    _check_lossless(law, p_rows, K)
    # acceptance law: P(a >= j) = prod_{i<j} alpha_i
    alphas = [oracle.acceptance_rate(p_rows[i], q_rows[i]) for i in range(K)]
    for j in range(K + 1):
        assert abs(_p_at_least(law, j) - np.prod(alphas[:j])) < TOL
    if name == "p_equals_q":
        assert abs(_p_at_least(law, K) - 1.0) < TOL          # 100 % acceptance
    if name == "disjoint":
        assert abs(_p_at_least(law, 1)) < TOL                  # 0 % acceptance


def test_expected_tokens_closed_form_iid():
    """i.i.d. rows: E[a+1] = (1 - alpha^(k+1)) / (1 - alpha)."""
    rng = np.random.default_rng(12)
    p = oracle.process(rng.normal(size=V), 1.0).p
    q = oracle.process(rng.normal(size=V), 1.0).p
    law = enumerate_law([p, p, p], [q, q], _draft_tuples([q, q]), check_oracle=False)
    mean = sum(len(seq) * pr for seq, pr in law.items())
    alpha = oracle.acceptance_rate(p, q)
    assert abs(mean - oracle.expected_tokens_per_step(alpha, K)) < TOL


@pytest.mark.parametrize("xs", [(0, 0), (3, 5), (7, 2), (1, 1)])
def test_onehot_invariant_equals_prefix_match_law(xs):
    """q = e_x: the sampled-mode law equals the law of 'y_j = invCDF_{p_j}(u_j),
    accept while y_j == x_j, commit the first mismatch or y_k'."""
    p_rows, _ = FAMILIES["random_T1"]
    q_rows = [np.eye(V)[xs[0]], np.eye(V)[xs[1]]]
    law = enumerate_law(p_rows, q_rows, iter([(xs, 1.0)]))
    _check_lossless(law, p_rows, K)
    # prefix-match scheme: enumerate the inverse-CDF interval of every row draw
    pm = {}

    def walk(j, prefix, mass):
        for t, lo, hi in _final_intervals(p_rows[j]):
            got_t, _, _ = oracle.inverse_cdf(p_rows[j], (lo + hi) / 2)
            assert got_t == t
            m = mass * (hi - lo)
            if j < K and t == xs[j]:
                walk(j + 1, prefix + (t,), m)
            else:
                pm[prefix + (t,)] = pm.get(prefix + (t,), 0.0) + m

    walk(0, (), 1.0)
    keys = set(pm) | set(law)
    for key in keys:
        assert abs(pm.get(key, 0.0) - law.get(key, 0.0)) < TOL


def test_onehot_pointwise_edges():
    rng = np.random.default_rng(13)
    p = np.zeros(V)
    p[3] = 1.0
    q = np.eye(V)[3]
    for u in rng.random(50):
        rec = oracle.sampled_request([p, p], [q], [3], [u, 0.5])
        assert rec.a == 1                               # p(x) = 1: accepted for every u
    p2 = oracle.process(rng.normal(size=V), 1.0).p
    p2[5] = 0.0
    p2 /= p2.sum()
    q5 = np.eye(V)[5]
    for u in rng.random(20):
        rec = oracle.sampled_request([p2, p2], [q5], [5], [u, 0.37])
        assert rec.a == 0                               # p(x) = 0: always rejected
        w, _ = oracle.final_weights(p2, q5, True)
        np.testing.assert_allclose(w, p2, atol=0)       # residual is p itself


def test_sampled_on_onehot_target_equals_greedy_pointwise():
    """Rows with one finite logit make p one-hot; sampled mode then equals
    greedy mode for every uniform and every draft distribution."""
    rng = np.random.default_rng(14)
    for _ in range(200):
        k = int(rng.integers(0, 4))
        g = rng.integers(0, V, size=k + 1)
        rows = np.full((k + 1, V), -np.inf)
        rows[np.arange(k + 1), g] = rng.normal(size=k + 1)
        drafts = np.where(rng.random(k) < 0.6, g[:k], rng.integers(0, V, size=k))
        p_rows = [oracle.process(r, float(rng.uniform(0.3, 2))).p for r in rows]
        q_rows = [oracle.process(rng.normal(size=V), 1.0).p for _ in range(k)]
        if rng.random() < 0.5:
            q_rows = [np.eye(V)[d] for d in drafts]
        u = rng.random(k + 1)
        rec = oracle.sampled_request(p_rows, q_rows, drafts, u)
        a, tokens, _ = oracle.greedy_request(rows, drafts)
        assert rec.a == a and rec.tokens == tokens


def test_p_equals_q_accepts_everything_pointwise():
    rng = np.random.default_rng(15)
    p = oracle.process(rng.normal(size=V), 1.0).p
    for _ in range(200):
        xs = rng.integers(0, V, size=K)
        u = np.append(rng.integers(0, 1 << 24, size=K) * 2.0 ** -24, 0.5)
        rec = oracle.sampled_request([p, p, p], [p, p], xs, u)
        assert rec.a == K
