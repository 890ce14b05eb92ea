"""Chi-square check of the oracle's sampled verify over 10^6 seeded trials.

The catalog page "Adding Speculative Decoding" (Acceptance bars, item 1)
asks for a distribution check over at least 100k tokens with chi-square
p > 0.05; this runs 10^6 trials at V=8, k=2 with drafts drawn from q by
numpy's own sampler and uniforms on the 2^-24 grid.  Checked: the first
committed token against p_0, the token at position j given a >= j against
p_j, and the histogram of a against its exact law prod alpha_i.  Seed 0 is
fixed in advance; the significance level is Bonferroni-corrected over the
five tests.
"""

import numpy as np
import pytest
import scipy.stats

import oracle

V, K, N = 8, 2, 1_000_000
ALPHA = 0.05


def _pooled_chi2(counts, expected):
    counts = np.asarray(counts, dtype=np.float64)
    expected = np.asarray(expected, dtype=np.float64)
    order = np.argsort(expected)
    c, e = [], []
    acc_c = acc_e = 0.0
    for i in order:                  # pool the smallest bins until each expects >= 5
        acc_c += counts[i]
        acc_e += expected[i]
        if acc_e >= 5:
            c.append(acc_c)
            e.append(acc_e)
            acc_c = acc_e = 0.0
    if acc_e > 0:
        if e:
            c[-1] += acc_c
            e[-1] += acc_e
        else:
            c.append(acc_c)
            e.append(acc_e)
    e = np.array(e) * (np.sum(c) / np.sum(e))
    if len(c) < 2:
        return 1.0
    return scipy.stats.chisquare(c, e).pvalue


@pytest.mark.slow
def test_chi_square_million_trials():
    rng_rows = np.random.default_rng(20240)
    L = rng_rows.normal(0, 1.5, size=(K + 1, V))
    D = L[:K] + rng_rows.normal(0, 0.9, size=(K, V))
    T = 0.9
    p_rows = [oracle.process(r, T).p for r in L]
    q_rows = [oracle.process(r, T).p for r in D]

    rng = np.random.default_rng(0)
    xs = np.stack([rng.choice(V, size=N, p=q_rows[i]) for i in range(K)], axis=1)
    us = rng.integers(0, 1 << 24, size=(N, K + 1)).astype(np.float64) * 2.0 ** -24

    a_hist = np.zeros(K + 1, dtype=np.int64)
    tok = [np.zeros(V, dtype=np.int64) for _ in range(K + 1)]
    for n in range(N):
        rec = oracle.sampled_request(p_rows, q_rows, xs[n], us[n])
        a_hist[rec.a] += 1
        for j, t in enumerate(rec.tokens):
            tok[j][t] += 1

    alphas = [oracle.acceptance_rate(p_rows[i], q_rows[i]) for i in range(K)]
    law_a = [np.prod(alphas[:j]) * (1 - alphas[j]) for j in range(K)] + [np.prod(alphas)]
    pvals = [_pooled_chi2(a_hist, np.array(law_a) * N)]
    for j in range(K + 1):
        pvals.append(_pooled_chi2(tok[j], p_rows[j] * tok[j].sum()))
    assert sum(t.sum() for t in tok) >= 100_000
    for pv in pvals:
        assert pv > ALPHA / len(pvals), pvals
