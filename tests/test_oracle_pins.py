"""Pins of the oracle against what the pages and mathematics fix.

- The two-token example and exercise printed on the aihero.vn page
  (tests/golden/two_token_examples.json): acceptance probabilities, residual
  location and the recovered marginal, as exact fractions.
- Exact path enumeration on tiny vocabularies: every emitted position is
  distributed as the target row, the per-position acceptance probability is
  sum_x min(p, q), the resample law is (p - q)+ / Z and sums to one.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from exact_paths import enumerate_sequence, marginals, step_measure

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "two_token_examples.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _logits(fracs):
    return np.log(np.array([float(Fraction(v)) for v in fracs]))


@pytest.mark.parametrize("case", _cases(), ids=["example", "exercise"])
def test_printed_two_token_values(case):
    q_l, p_l = _logits(case["q"]), _logits(case["p"])
    q, _, _ = oracle.filtered_distribution(q_l, 1.0)
    p, _, _ = oracle.filtered_distribution(p_l, 1.0)
    # acceptance of A and of B
    for tok, key in ((0, "accept_prob_A"), (1, "accept_prob_B")):
        want = float(Fraction(case[key]))
        assert min(1.0, oracle.accept_ratio(p, q, tok)) == pytest.approx(want, abs=1e-12)
    # residual lies entirely on B, with the printed mass
    rho = oracle.residual(p, q)
    want_rho = [float(Fraction(v)) for v in case["residual_unnormalised"]]
    assert rho == pytest.approx(want_rho, abs=1e-12)
    assert rho[0] == 0.0
    # resampling from the residual returns B for every uniform
    for u in (0.0, 1e-9, 0.25, 0.5, 0.999999):
        j, Z, _ = oracle.inverse_cdf(rho, u)
        assert j == 1
        assert Z == pytest.approx(float(sum(Fraction(v) for v in case["residual_unnormalised"])), abs=1e-12)


@pytest.mark.parametrize("case", _cases(), ids=["example", "exercise"])
def test_printed_two_token_marginal_by_path_sums(case):
    """Summing path probabilities (draft A or B, accept or resample) recovers p."""
    q_l, p_l = _logits(case["q"])[None, :], _logits(case["p"])
    # K = 1: the second target row (bonus row) is irrelevant to out_0; reuse p.
    p_rows = np.stack([p_l, p_l])
    q = softmax(q_l[0])
    total = np.zeros(2)
    for x in (0, 1):
        for prob, n, dist in enumerate_sequence(q_l, p_rows, [x], 1.0):
            if n == 0:
                total += q[x] * prob * dist
            else:
                total[x] += q[x] * prob
    want = [float(Fraction(v)) for v in case["output_marginal"]]
    assert total == pytest.approx(want, abs=1e-12)
    # and exactly as fractions: q_A * a_A + ... (closed form from the page)
    qa, pa = Fraction(case["q"][0]), Fraction(case["p"][0])
    acc_a = min(Fraction(1), pa / qa)
    assert qa * acc_a == Fraction(case["output_marginal"][0])
    assert 1 - qa * acc_a == Fraction(case["output_marginal"][1])


def _rand_rows(rng, K, V, sd=1.0, shift=0.7):
    base = rng.normal(0, sd, (K + 1, V))
    q_rows = base[:K]
    p_rows = base + rng.normal(0, shift, (K + 1, V))
    return q_rows, p_rows


@pytest.mark.parametrize("seed,K,V,T", [(0, 1, 5, 1.0), (1, 2, 4, 0.7), (2, 3, 3, 1.3), (3, 2, 4, 2.0)])
def test_exact_enumeration_output_marginals(seed, K, V, T):
    rng = np.random.default_rng(seed)
    q_rows, p_rows = _rand_rows(rng, K, V)
    q_probs = np.stack([softmax(q_rows[i] / T) for i in range(K)])
    p_probs = np.stack([softmax(p_rows[i] / T) for i in range(K + 1)])
    reach, emit = marginals(q_rows, p_rows, q_probs, T)
    assert reach[0] == pytest.approx(1.0, abs=1e-12)
    for j in range(K + 1):
        # the token emitted at position j, given position j is reached, ~ p_j
        assert emit[j] / reach[j] == pytest.approx(p_probs[j], abs=1e-10)
    for j in range(K):
        beta = np.minimum(p_probs[j], q_probs[j]).sum()
        assert reach[j + 1] / reach[j] == pytest.approx(beta, abs=1e-10)
    # expected number of accepted drafts: sum_{j<K} prod_{i<=j} beta_i
    betas = [np.minimum(p_probs[j], q_probs[j]).sum() for j in range(K)]
    e_n = sum(np.prod(betas[: j + 1]) for j in range(K))
    assert reach[1:].sum() == pytest.approx(e_n, abs=1e-10)


@pytest.mark.parametrize("seed,K,V,T,top_k,top_p", [
    (10, 1, 6, 1.0, 3, 1.0), (11, 2, 5, 0.8, 0, 0.8), (12, 2, 6, 1.0, 4, 0.85)])
def test_exact_enumeration_with_filters(seed, K, V, T, top_k, top_p):
    """With top-k/top-p applied to both rows, outputs follow the filtered target."""
    rng = np.random.default_rng(seed)
    q_rows, p_rows = _rand_rows(rng, K, V, sd=1.5, shift=1.0)
    q_probs = np.stack([oracle.filtered_distribution(q_rows[i], T, top_k, top_p)[0] for i in range(K)])
    p_probs = np.stack([oracle.filtered_distribution(p_rows[i], T, top_k, top_p)[0] for i in range(K + 1)])
    reach, emit = marginals(q_rows, p_rows, q_probs, T, top_k, top_p)
    for j in range(K + 1):
        assert emit[j] / reach[j] == pytest.approx(p_probs[j], abs=1e-10)


@pytest.mark.parametrize("seed", [20, 21, 22])
def test_resample_law_is_normalised_residual(seed):
    """Given a rejection at position 0, the emitted token ~ (p - q)+ / Z."""
    rng = np.random.default_rng(seed)
    V = 6
    q_rows, p_rows = _rand_rows(rng, 1, V, sd=1.2, shift=1.0)
    q, p = softmax(q_rows[0]), softmax(p_rows[0])
    want = np.maximum(p - q, 0)
    want /= want.sum()
    # choose a draft id the target under-weights so rejection is possible
    x = int(np.argmax(q - p))
    outs = enumerate_sequence(q_rows, p_rows, [x], 1.0)
    rej = [d for (pr, n, d) in outs if n == 0]
    assert len(rej) == 1
    assert rej[0].sum() == pytest.approx(1.0, abs=1e-12)
    assert rej[0] == pytest.approx(want, abs=1e-10)
    # acceptance probability of x is min(1, p/q)
    acc = [pr for (pr, n, d) in outs if n == 1]
    assert acc[0] == pytest.approx(min(1.0, p[x] / q[x]), abs=1e-12)


def test_resample_distance_to_total_variation():
    """Z of the residual equals 1 - sum min(p, q) = TV(p, q)."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        V = int(rng.integers(2, 50))
        p = softmax(rng.normal(0, 2, V))
        q = softmax(rng.normal(0, 2, V))
        _, Z, _ = oracle.inverse_cdf(oracle.residual(p, q), 0.5)
        assert Z == pytest.approx(1 - np.minimum(p, q).sum(), abs=1e-13)
        assert Z == pytest.approx(0.5 * np.abs(p - q).sum(), abs=1e-13)


def test_inverse_cdf_is_categorical_law():
    """The inverse CDF maps U[0,1) to the categorical law w / sum(w)."""
    rng = np.random.default_rng(7)
    for V in (1, 2, 7, 40):
        w = rng.random(V) * (rng.random(V) < 0.7)
        if w.sum() == 0:
            w[0] = 1.0
        meas = step_measure(lambda u: oracle.inverse_cdf(w, u)[0], V)
        assert meas == pytest.approx(w / w.sum(), abs=1e-12)
        # zero-weight ids are never drawn
        for u in np.linspace(0, 1, 257, endpoint=False):
            assert w[oracle.inverse_cdf(w, u)[0]] > 0


def test_inverse_cdf_uniform_weights_closed_form():
    """Equal weights over V ids: the draw is floor(u * V) away from boundaries."""
    V = 1000
    w = np.full(V, 0.25)
    for u in np.random.default_rng(3).random(500):
        if abs(u * V - round(u * V)) < 1e-6:
            continue
        assert oracle.inverse_cdf(w, u)[0] == math.floor(u * V)
