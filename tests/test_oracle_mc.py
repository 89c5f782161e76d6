"""Monte-Carlo check of the oracle's output law (chi-square), standing in for
the distribution test the aivaro.ru page suggests for its pet project
(section 11): seeded uniforms, fixed logits, emitted token at position 0
compared with the target row p_0."""

import numpy as np
from scipy.special import softmax
from scipy.stats import chisquare

import oracle


def test_first_token_law_chisquare():
    rng = np.random.default_rng(123)
    K, V, T = 4, 16, 1.0
    base = rng.normal(0, 2, (K + 1, V))
    q_rows = base[:K]
    p_rows = base + rng.normal(0, 0.8, (K + 1, V))
    q0 = softmax(q_rows[0] / T)
    p0 = softmax(p_rows[0] / T)
    N = 20000
    counts = np.zeros(V)
    qs = [softmax(q_rows[i] / T) for i in range(K)]
    for _ in range(N):
        x = [int(rng.choice(V, p=qs[i])) for i in range(K)]
        u = rng.random(K + 1)
        r = oracle.verify_sequence(q_rows, p_rows, x, u, T)
        counts[r["tokens"][0]] += 1
    stat, pval = chisquare(counts, N * p0)
    assert pval > 1e-4, (stat, pval)
    # the draft law itself differs from p0 enough that the test has power
    stat_q, pval_q = chisquare(counts, N * q0)
    assert pval_q < 1e-6
