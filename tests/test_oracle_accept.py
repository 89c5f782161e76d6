"""Pins of the oracle's acceptance statistics (probability that a draft passes,
expected accepted drafts per round).

- The aihero.vn page's two-token example and exercise
  (tests/golden/two_token_examples.json): the probability that a draft drawn
  from q passes is sum_x q(x) * accept(x) over the printed per-token
  acceptances, as exact fractions.
- Exact path enumeration of the verification oracle on tiny vocabularies
  (tests/exact_paths.py): the measured pass rate of every position and the
  expected number of accepted drafts, with and without filters.
- The identity sum min(p, q) = 1 - Z, Z the residual mass of the resample step.
- Unusable rows give NaN; K_b = 0 gives an expected count of 0.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact_paths import marginals

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "two_token_examples.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=["example", "exercise"])
def test_printed_examples_pass_rate(case):
    q_f = [Fraction(v) for v in case["q"]]
    want = q_f[0] * Fraction(case["accept_prob_A"]) + q_f[1] * Fraction(case["accept_prob_B"])
    assert want == (Fraction(9, 10) if case["q"][0] == "2/5" else Fraction(1, 2))
    q_l = np.log([float(v) for v in q_f])
    p_l = np.log([float(Fraction(v)) for v in case["p"]])
    q, _, _ = oracle.filtered_distribution(q_l, 1.0)
    p, _, _ = oracle.filtered_distribution(p_l, 1.0)
    assert oracle.acceptance_probability(p, q) == pytest.approx(float(want), abs=1e-12)
    # one sequence, one draft: the expected accepted count is that probability
    draft = q_l[None, :]
    target = np.stack([p_l, p_l])
    r = oracle.acceptance_stats(draft, target, B=1, K=1, V=2, dtype="f64", temperature=1.0)
    assert r["beta"][0] == pytest.approx(float(want), abs=1e-12)
    assert r["expected_accepted"][0] == pytest.approx(float(want), abs=1e-12)


def _rand_rows(rng, K, V, sd=1.0, shift=0.7):
    base = rng.normal(0, sd, (K + 1, V))
    return base[:K], base + rng.normal(0, shift, (K + 1, V))


@pytest.mark.parametrize("seed,K,V,T,top_k,top_p", [
    (30, 1, 5, 1.0, 0, 1.0), (31, 2, 4, 0.7, 0, 1.0), (32, 3, 3, 1.3, 0, 1.0),
    (33, 2, 6, 1.0, 4, 1.0), (34, 2, 5, 0.8, 0, 0.8), (35, 2, 6, 1.0, 4, 0.85)])
def test_matches_enumerated_pass_rates(seed, K, V, T, top_k, top_p):
    """The oracle's pass probability of position j is the enumerated
    P(n >= j+1 | n >= j) of the verification oracle, and its expected count is
    the enumerated E[n] = sum_{j>=1} P(n >= j)."""
    rng = np.random.default_rng(seed)
    q_rows, p_rows = _rand_rows(rng, K, V, sd=1.5, shift=1.0)
    q_probs = np.stack([oracle.filtered_distribution(q_rows[i], T, top_k, top_p)[0]
                        for i in range(K)])
    reach, _ = marginals(q_rows, p_rows, q_probs, T, top_k, top_p)
    r = oracle.acceptance_stats(q_rows, p_rows, B=1, K=K, V=V, dtype="f64", temperature=T,
                                top_k=top_k, top_p=top_p)
    for j in range(K):
        assert r["beta"][j] == pytest.approx(reach[j + 1] / reach[j], abs=1e-10)
    assert r["expected_accepted"][0] == pytest.approx(reach[1:].sum(), abs=1e-10)


def test_pass_rate_is_one_minus_residual_mass():
    rng = np.random.default_rng(36)
    for _ in range(20):
        V = int(rng.integers(2, 300))
        for top_k, top_p in ((0, 1.0), (max(1, V // 3), 1.0), (max(1, V // 2), 0.9)):
            q, _, _ = oracle.filtered_distribution(rng.normal(0, 2, V), 0.8, top_k, top_p)
            p, _, _ = oracle.filtered_distribution(rng.normal(0, 2, V), 0.8, top_k, top_p)
            _, Z, _ = oracle.inverse_cdf(oracle.residual(p, q), 0.5)
            Z = 0.0 if Z is None else Z
            assert oracle.acceptance_probability(p, q) == pytest.approx(1.0 - Z, abs=1e-12)


def test_identical_rows_always_pass_and_disjoint_rows_never():
    rng = np.random.default_rng(37)
    l = rng.normal(0, 2, 50)
    p, _, _ = oracle.filtered_distribution(l, 1.0)
    assert oracle.acceptance_probability(p, p) == pytest.approx(1.0, abs=1e-12)
    # disjoint supports after top-k: no drafted id has target mass
    lq = np.full(10, -5.0)
    lq[:3] = [4.0, 3.0, 2.0]
    lp = np.full(10, -5.0)
    lp[5:8] = [4.0, 3.0, 2.0]
    q, _, _ = oracle.filtered_distribution(lq, 1.0, 3)
    p, _, _ = oracle.filtered_distribution(lp, 1.0, 3)
    assert oracle.acceptance_probability(p, q) == 0.0


def test_ragged_batch_products_nan_and_empty_sequences():
    rng = np.random.default_rng(38)
    V = 40
    cu = np.array([0, 3, 3, 5])  # K_b = 3, 0, 2
    draft = rng.normal(0, 2, (5, V))
    target = rng.normal(0, 2, (5 + 3, V))
    draft[4, 7] = np.nan  # sequence 2, position 1 unusable
    r = oracle.acceptance_stats(draft, target, B=3, V=V, dtype="f64", temperature=0.9,
                                cu_draft=cu)
    b = r["beta"]
    for d, t in ((0, 0), (1, 1), (2, 2), (3, 5), (4, 6)):
        if d == 4:
            assert math.isnan(b[d])
            continue
        q, _, _ = oracle.filtered_distribution(draft[d], 0.9)
        p, _, _ = oracle.filtered_distribution(target[t], 0.9)
        assert b[d] == pytest.approx(np.minimum(p, q).sum(), abs=1e-12)
    e = r["expected_accepted"]
    assert e[0] == pytest.approx(b[0] + b[0] * b[1] + b[0] * b[1] * b[2], abs=1e-12)
    assert e[1] == 0.0
    assert math.isnan(e[2])


def test_rejects_greedy_temperature():
    with pytest.raises(ValueError):
        oracle.acceptance_stats(np.zeros((1, 4)), np.zeros((2, 4)), B=1, K=1, V=4,
                                dtype="f64", temperature=0.0)
