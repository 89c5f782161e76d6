"""Exact outcome enumeration around the oracle's several-chain verification
(test helper). The oracle is a black box in its uniforms. Every test of a
candidate is a threshold in its own uniform (accepted on [0, a)), and a draw
is a non-decreasing step function of its own. The oracle reports which chain
it accepted at each position. Bisection then recovers each threshold, and
every outcome's probability is a product of interval lengths."""

import numpy as np

import oracle
from exact_paths import step_measure, threshold


def enumerate_multi(q_rows, p_rows, x, T, top_k=0, top_p=1.0):
    """Outcomes for fixed candidate tokens x [M, K]: a list of
    (probability, n, accepted prefix (list), law of the token at position n)."""
    M, K = x.shape
    V = p_rows.shape[2]
    out = []

    def run(u):
        return oracle.verify_multi_sequence(q_rows, p_rows, x, u, T, top_k, top_p)

    def rec(u, j, live, weight, prefix):
        if j == K:
            def bonus(v):
                uu = u.copy()
                uu[K, M] = v
                return run(uu)["tokens"][K]
            out.append((weight, K, prefix, step_measure(bonus, V)))
            return
        for m in live:
            def accepted(v, m=m):
                uu = u.copy()
                uu[j, m] = v
                return run(uu)["chosen"][j] == m
            a = threshold(accepted)
            if a > 0.0:
                ua = u.copy()
                ua[j, m] = 0.5 * a
                t = int(x[m, j])
                rec(ua, j + 1, [mm for mm in live if int(x[mm, j]) == t], weight * a,
                    prefix + [t])
            if a >= 1.0:
                return
            u = u.copy()
            u[j, m] = 0.5 * (a + 1.0)
            weight *= 1.0 - a

        def draw(v):
            uu = u.copy()
            uu[j, M] = v
            return run(uu)["tokens"][j]
        out.append((weight, j, prefix, step_measure(draw, V)))

    rec(np.full((K + 1, M + 1), 0.5), 0, list(range(M)), 1.0, [])
    return out
