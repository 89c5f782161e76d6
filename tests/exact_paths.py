"""Exact path-probability enumeration around the oracle (test helper).

The oracle is treated as a black box function of its uniforms. Every decision
in it is a threshold in one uniform: acceptance at position i is ``u_i < a_i``
and the resampled or bonus token is a non-decreasing step function of ``u_K``.
Bisection in float64 recovers each threshold, so the probability of every
outcome is a product of interval lengths, known to ~1e-15, with no sampling.
"""

import math

import numpy as np

import oracle


def _bisect(pred, iters=64):
    """pred True on [0, a), False on [a, 1). Returns (lo, hi) around a with
    pred(lo) True and pred(hi) False; (0, 0) if a = 0 and (1, 1) if a = 1."""
    if not pred(0.0):
        return 0.0, 0.0
    top = math.nextafter(1.0, 0.0)
    if pred(top):
        return 1.0, 1.0
    lo, hi = 0.0, top
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if pred(mid):
            lo = mid
        else:
            hi = mid
    return lo, hi


def threshold(pred, iters=64):
    """``pred`` is True on [0, a) and False on [a, 1): return a."""
    lo, hi = _bisect(pred, iters)
    return 0.5 * (lo + hi)


def step_measure(f, V):
    """Lengths of the intervals of [0, 1) on which the step function f takes
    each value (f non-decreasing in u). Returns a float64 array [V]."""
    out = np.zeros(V)
    v = 0.0
    y = f(0.0)
    while True:
        lo, hi = _bisect(lambda t, y=y: f(t) <= y)
        b = 0.5 * (lo + hi)
        out[y] += b - v
        if hi >= 1.0:
            break
        v = b
        y = f(hi)
    return out


def enumerate_sequence(q_rows, p_rows, x, T, top_k=0, top_p=1.0):
    """Outcome distribution of one sequence for a fixed draft tuple ``x``.

    Returns a list of (probability, n, token_distribution) where n is the
    number of accepted drafts and token_distribution the law of the token
    emitted at position n (resample if n < K, bonus if n == K)."""
    K = len(x)
    V = p_rows.shape[1]
    u = [0.5] * (K + 1)
    weight = 1.0
    out = []

    def run(uu):
        return oracle.verify_sequence(q_rows, p_rows, x, uu, T, top_k, top_p)

    for i in range(K):
        def accepted(v, i=i):
            uu = list(u)
            uu[i] = v
            return run(uu)["n"] > i

        a = threshold(accepted)
        if a < 1.0:
            base = list(u)
            base[i] = 0.5 * (a + 1.0)

            def tok(v, base=base, i=i):
                uu = list(base)
                uu[K] = v
                return run(uu)["tokens"][i]

            out.append((weight * (1.0 - a), i, step_measure(tok, V)))
        if a == 0.0:
            return out
        u[i] = 0.5 * a
        weight *= a

    def bonus(v):
        uu = list(u)
        uu[K] = v
        return run(uu)["tokens"][K]

    out.append((weight, K, step_measure(bonus, V)))
    return out


def marginals(q_rows, p_rows, q_probs, T, top_k=0, top_p=1.0):
    """Enumerate all draft tuples x ~ prod_i q_i(x_i) (q_probs: [K, V]).

    Returns (reach [K+1], emit [K+1, V]): reach[j] = P(n >= j) and emit[j, y] =
    P(n >= j and the token emitted at position j is y)."""
    K, V = q_probs.shape[0], p_rows.shape[1]
    reach = np.zeros(K + 1)
    emit = np.zeros((K + 1, V))
    for flat in range(V ** K):
        x = [(flat // V ** i) % V for i in range(K)]
        w = float(np.prod([q_probs[i, x[i]] for i in range(K)])) if K else 1.0
        if w == 0.0:
            continue
        for prob, n, dist in enumerate_sequence(q_rows, p_rows, x, T, top_k, top_p):
            pw = w * prob
            for j in range(n):
                reach[j] += pw
                emit[j, x[j]] += pw
            reach[n] += pw
            emit[n] += pw * dist
    return reach, emit
