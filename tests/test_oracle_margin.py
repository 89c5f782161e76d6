"""Pins of the oracle's near-threshold margin (-m "not gpu").

The GPU parity tests skip the bit-exact comparison of a sequence whose oracle
margin is at most 1e-5. The margin is the smallest distance, in units of the
uniform, between a uniform the sequence used and the threshold of the decision
it took:
  - ratio test u_i < r_i: |u_i - r_i| (the test's own threshold is r_i; with
    u in [0, 1), r_i > 1 can only be misjudged if rounding carried r_i below
    u, which the same distance measures);
  - inverse CDF: the distance from u to the nearer end of the chosen interval
    [C_{j-1}/Z, C_j/Z);
  - top-p: |mass strictly above a level - top_p| at the level nearest the cut.
Each test below places a uniform (or top_p) at a known distance from a known
threshold and checks the margin equals that distance to 1e-12, so a margin in
the wrong units (u*Z instead of u), on the wrong interval end or of the wrong
decision fails.

Thresholds come from the pages' worked example (aihero.vn "Speculative
decoding", section "Chấp nhận bằng tỉ lệ, không chỉ bằng argmax": q = [0.4,
0.6], p = [0.3, 0.7], acceptance of A 0.75, residual on B; the exercise section
"Bài tập: chứng minh lại một phân bố hai token": q = [0.8, 0.2], acceptance of
A 0.375) and from closed forms (equal weights: C_j/Z = (j+1)/V; a row of
probabilities [0.5, 0.3, 0.15, 0.05]: masses above the levels 0, 0.5, 0.8,
0.95).
"""

import math

import numpy as np
import pytest

import oracle

A, B_ = 0, 1
EXAMPLE = dict(q=[0.4, 0.6], p=[0.3, 0.7])
EXERCISE = dict(q=[0.8, 0.2], p=[0.3, 0.7])


def _rows(case, bonus=(0.5, 0.5)):
    q = np.log(np.array([case["q"]]))
    p = np.log(np.array([case["p"], list(bonus)]))
    return q, p


@pytest.mark.parametrize("delta", [3e-6, 7.5e-6, 2e-4])
def test_accept_margin_below_threshold(delta):
    """u just below r_A = 3/4: accepted, margin = 3/4 - u; the bonus draw from
    [0.5, 0.5] at u = 0.25 lies 0.25 from both ends of its interval."""
    q, p = _rows(EXAMPLE)
    r = oracle.verify_sequence(q, p, [A], [0.75 - delta, 0.25], 1.0)
    assert r["n"] == 1 and r["tokens"] == [A, 0]
    assert abs(r["margin"] - delta) <= 1e-12


@pytest.mark.parametrize("delta", [4e-5, 1e-6])
def test_reject_margin_above_threshold(delta):
    """u just above r_A = 3/4: rejected; the residual [0, 0.1] puts all mass on
    B, whose interval is [0, 1), so the resample at u = 0.5 lies 0.5 (not
    0.05 = 0.5 * Z) from its ends, and the margin is the ratio test's."""
    q, p = _rows(EXAMPLE)
    r = oracle.verify_sequence(q, p, [A], [0.75 + delta, 0.5], 1.0)
    assert r["n"] == 0 and r["tokens"] == [B_, -1]
    assert r["resid_Z"] == pytest.approx(0.1, abs=1e-15)
    assert abs(r["margin"] - delta) <= 1e-12
    j, Z, m = oracle.inverse_cdf(oracle.residual(np.array(EXAMPLE["p"]), np.array(EXAMPLE["q"])),
                                 0.5)
    assert j == B_ and abs(m - 0.5) <= 1e-12


def test_accept_margin_exercise_threshold():
    """The exercise's acceptance of A, 3/8: u = 3/8 + 1e-7 rejects, margin 1e-7."""
    q, p = _rows(EXERCISE)
    r = oracle.verify_sequence(q, p, [A], [0.375 + 1e-7, 0.5], 1.0)
    assert r["n"] == 0
    assert abs(r["margin"] - 1e-7) <= 1e-12


def test_accept_margin_is_distance_to_the_ratio_above_one():
    """Drafting B in the example gives r_B = 0.7/0.6 = 7/6 > 1. The test u < r
    has its threshold at r itself, so at u = 0.99 the margin is 7/6 - 0.99
    (the bonus draw at u = 0.25 is farther)."""
    q, p = _rows(EXAMPLE)
    r = oracle.verify_sequence(q, p, [B_], [0.99, 0.25], 1.0)
    assert r["n"] == 1
    assert abs(r["margin"] - (7.0 / 6.0 - 0.99)) <= 1e-12


@pytest.mark.parametrize("j0,delta,side", [(437, 2.5e-6, -1), (437, 2.5e-6, +1), (0, 1e-7, -1),
                                           (998, 3e-9, +1)])
def test_inverse_cdf_margin_on_equal_weights(j0, delta, side):
    """Equal weights over V = 1000 ids: C_j/Z = (j+1)/V. A uniform delta below
    (j0+1)/V picks j0 and a uniform delta above picks j0+1; either way the
    margin is delta. Checked on the sampler alone and through a K = 0
    verification (plain sampling from p_0 by the bonus draw)."""
    V = 1000
    u = (j0 + 1) / V + side * delta
    want = j0 if side < 0 else j0 + 1
    j, Z, m = oracle.inverse_cdf(np.ones(V), u)
    assert j == want and Z == V
    assert abs(m - delta) <= 1e-12
    r = oracle.verify_sequence(None, np.zeros((1, V)), [], [u], 1.0)
    assert r["n"] == 0 and r["tokens"] == [want]
    assert abs(r["margin"] - delta) <= 1e-12


@pytest.mark.parametrize("top_p,kept", [(0.8 + 3e-6, 3), (0.8 - 3e-6, 2), (0.95 + 1e-8, 4),
                                        (0.5 - 2e-5, 1)])
def test_top_p_margin_at_level_boundary(top_p, kept):
    """Probabilities [0.5, 0.3, 0.15, 0.05]: the masses strictly above the four
    levels are 0, 0.5, 0.8 and 0.95. top_p a small distance from one of them
    keeps the levels whose mass above is below top_p, and the margin is that
    distance. Through verify_sequence the top-p margin of a used row enters the
    sequence's margin."""
    probs = np.array([0.5, 0.3, 0.15, 0.05])
    l = np.log(probs)
    dist = abs(top_p - min((0.0, 0.5, 0.8, 0.95), key=lambda a: abs(a - top_p)))
    prob, _, m = oracle.filtered_distribution(l, 1.0, 0, top_p)
    assert int((prob > 0).sum()) == kept
    assert abs(m - dist) <= 1e-12
    # K = 0: the bonus draw from p_0 at u = 0.5 * (kept mass) lies far from its
    # ends, so the top-p margin is the sequence's
    mass = probs[:kept].sum()
    u = (probs[0] / mass) * 0.5
    r = oracle.verify_sequence(None, l[None, :], [], [u], 1.0, top_p=top_p)
    assert r["tokens"] == [0]
    assert abs(r["margin"] - dist) <= 1e-12


def test_margin_is_infinite_without_decisions():
    """A greedy sequence takes no uniform-based decision: its margin stays at
    the oracle's 'cannot flip' value."""
    p = np.log(np.array([[0.2, 0.8], [0.6, 0.4]]))
    r = oracle.verify_sequence(None, p, [1], [0.5, 0.5], 0.0, greedy=True)
    assert r["n"] == 1 and r["tokens"] == [1, 0]
    assert math.isinf(r["margin"])
