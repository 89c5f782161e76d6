"""Special cases of the oracle that reduce to textbook results or library routines."""

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle


def test_decode_logits_matches_torch_widening():
    rng = np.random.default_rng(0)
    x = torch.from_numpy(rng.normal(0, 5, 4096).astype(np.float32))
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16), ("f32", torch.float32)):
        t = x.to(tdt)
        raw = t.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else t.numpy()
        want = t.to(torch.float64).numpy()
        np.testing.assert_array_equal(oracle.decode_logits(raw, dt), want)


def test_lse_matches_library_logsumexp():
    rng = np.random.default_rng(1)
    for T in (0.5, 0.7, 1.0, 3.0):
        l = rng.normal(0, 3, 5000)
        _, lse, _ = oracle.filtered_distribution(l, T)
        assert lse == pytest.approx(logsumexp(l / T), rel=1e-14, abs=1e-12)
        assert lse == pytest.approx(np.logaddexp.reduce(l / T), rel=1e-13, abs=1e-12)
        p, _, _ = oracle.filtered_distribution(l, T)
        np.testing.assert_allclose(p, softmax(l / T), rtol=1e-12, atol=1e-300)


def test_neg_inf_logits_get_zero_probability():
    l = np.array([0.0, -np.inf, 1.0, -np.inf])
    p, lse, _ = oracle.filtered_distribution(l, 1.0)
    assert p[1] == 0.0 and p[3] == 0.0
    assert p[[0, 2]] == pytest.approx(softmax(np.array([0.0, 1.0])))
    assert lse == pytest.approx(np.logaddexp(0.0, 1.0))


def test_identical_rows_accept_everything_and_bonus_is_categorical():
    """q = p: every ratio is 1, so all K drafts are accepted and the bonus is a
    plain draw from p_K."""
    rng = np.random.default_rng(2)
    K, V = 4, 64
    rows = rng.normal(0, 2, (K + 1, V))
    x = rng.integers(0, V, K)
    for u in rng.random((50, K + 1)):
        r = oracle.verify_sequence(rows[:K], rows, x, u, 1.0)
        assert r["n"] == K
        assert r["tokens"][:K] == list(x)
    p = softmax(rows[K])
    from exact_paths import step_measure
    meas = step_measure(lambda v: oracle.verify_sequence(rows[:K], rows, x, [0.0] * K + [v], 1.0)["tokens"][K], V)
    assert meas == pytest.approx(p, abs=1e-12)


def test_k0_is_plain_sampling():
    rng = np.random.default_rng(3)
    V = 300
    l = rng.normal(0, 2, V)
    from exact_paths import step_measure
    meas = step_measure(lambda v: oracle.verify_sequence(np.zeros((0, V)), l[None, :], [], [v], 1.0)["tokens"][0], V)
    assert meas == pytest.approx(softmax(l), abs=1e-12)


def test_greedy_matches_numpy_argmax_and_first_tie():
    rng = np.random.default_rng(4)
    K, V = 5, 200
    p_rows = np.round(rng.normal(0, 2, (K + 1, V)), 0)  # many ties
    am = [int(np.argmax(r)) for r in p_rows]
    # all drafts equal the argmax: all accepted, bonus = argmax of row K
    r = oracle.verify_sequence(None, p_rows, am[:K], [0.5] * (K + 1), 1.0, greedy=True)
    assert r["n"] == K and r["tokens"] == am
    # first mismatch at position 2
    x = list(am[:K])
    x[2] = (x[2] + 1) % V
    r = oracle.verify_sequence(None, p_rows, x, [0.5] * (K + 1), 1.0, greedy=True)
    assert r["n"] == 2 and r["tokens"][:3] == am[:3] and r["tokens"][3:] == [-1] * (K - 2)
    # lowest id on exact ties
    row = np.zeros(V)
    row[[7, 19, 150]] = 3.0
    assert oracle.greedy_token(row) == 7


def test_topk1_sampling_equals_greedy_on_tie_free_rows():
    rng = np.random.default_rng(5)
    V = 500
    for _ in range(20):
        l = rng.normal(0, 3, V)
        toks, _ = oracle.sample_rows(l[None, :], np.array([rng.random()], np.float32),
                                     V=V, dtype="f64", temperature=0.9, top_k=1)
        assert toks[0] == np.argmax(l)


def test_low_temperature_limit_is_greedy():
    rng = np.random.default_rng(6)
    V = 400
    for _ in range(20):
        l = rng.normal(0, 3, V)
        toks, _ = oracle.sample_rows(l[None, :], np.array([rng.random()], np.float32),
                                     V=V, dtype="f64", temperature=1e-3)
        assert toks[0] == np.argmax(l)


def test_top_k_keeps_ties():
    l = np.array([5.0, 1.0, 3.0, 3.0, 3.0, 0.0, 4.0])
    p, _, _ = oracle.filtered_distribution(l, 1.0, top_k=3)
    # top-3 values are 5, 4, 3; all three 3.0 entries are kept
    assert set(np.flatnonzero(p > 0)) == {0, 2, 3, 4, 6}
    want = softmax(l[[0, 2, 3, 4, 6]])
    assert p[[0, 2, 3, 4, 6]] == pytest.approx(want)


def test_top_k_matches_argsort_on_tie_free_rows():
    rng = np.random.default_rng(7)
    V = 1000
    for k in (1, 5, 50, 999):
        l = rng.normal(0, 3, V)
        p, _, _ = oracle.filtered_distribution(l, 0.8, top_k=k)
        top = np.argsort(-l)[:k]
        assert set(np.flatnonzero(p > 0)) == set(top)
        assert p[top] == pytest.approx(softmax(l[top] / 0.8), rel=1e-12)


def test_top_p_matches_sorted_cumsum_rule_on_tie_free_rows():
    rng = np.random.default_rng(8)
    V = 300
    for top_p in (0.1, 0.5, 0.9, 0.99):
        l = rng.normal(0, 2, V)
        p, _, margin = oracle.filtered_distribution(l, 1.0, top_p=top_p)
        pi = softmax(l)
        order = np.argsort(-pi)
        before = np.concatenate([[0.0], np.cumsum(pi[order])[:-1]])
        keep = order[before < top_p]
        if margin > 1e-9:
            assert set(np.flatnonzero(p > 0)) == set(keep)
            assert p[keep] == pytest.approx(pi[keep] / pi[keep].sum(), rel=1e-12)


def test_top_p_hand_example_and_ties():
    probs = np.array([0.5, 0.3, 0.15, 0.05])
    l = np.log(probs)
    p, _, _ = oracle.filtered_distribution(l, 1.0, top_p=0.7)
    assert set(np.flatnonzero(p > 0)) == {0, 1}
    assert p[[0, 1]] == pytest.approx([0.625, 0.375])
    # the most probable token alone already covers 0.5 >= 0.45
    p, _, _ = oracle.filtered_distribution(l, 1.0, top_p=0.45)
    assert set(np.flatnonzero(p > 0)) == {0}
    # equal logits share the same "mass strictly above": kept or dropped together
    l2 = np.log(np.array([0.4, 0.2, 0.2, 0.2]))
    p, _, _ = oracle.filtered_distribution(l2, 1.0, top_p=0.5)
    assert set(np.flatnonzero(p > 0)) == {0, 1, 2, 3}
    p, _, _ = oracle.filtered_distribution(l2, 1.0, top_p=0.39)
    assert set(np.flatnonzero(p > 0)) == {0}


def test_top_k_then_top_p_order():
    """top-p is computed on the renormalised top-k set (k first, then p)."""
    probs = np.array([0.3, 0.25, 0.2, 0.15, 0.1])
    l = np.log(probs)
    # top-2 renormalised: [0.545, 0.455]; top_p = 0.5 keeps only the first
    p, _, _ = oracle.filtered_distribution(l, 1.0, top_k=2, top_p=0.5)
    assert set(np.flatnonzero(p > 0)) == {0}
    # without top-k, mass above id 1 is 0.3 < 0.5 so ids 0 and 1 are kept
    p, _, _ = oracle.filtered_distribution(l, 1.0, top_p=0.5)
    assert set(np.flatnonzero(p > 0)) == {0, 1}


def test_zero_probability_draft_rules():
    p = np.array([0.5, 0.5, 0.0])
    q = np.array([0.0, 1.0, 0.0])
    assert oracle.accept_ratio(p, q, 0) == math.inf
    assert oracle.accept_ratio(p, q, 2) == 0.0
    assert oracle.accept_ratio(p, q, 1) == 0.5


def test_error_codes_and_precedence():
    V, K = 16, 3
    rng = np.random.default_rng(9)
    q_rows, p_rows = rng.normal(0, 1, (K, V)), rng.normal(0, 1, (K + 1, V))
    u = [0.3] * (K + 1)
    r = oracle.verify_sequence(q_rows, p_rows, [1, V, 2], u, 1.0)
    assert r["n"] == -1 and r["tokens"] == [-1] * (K + 1)
    # rows of position 0 are always read
    bad = p_rows.copy()
    bad[0, 5] = np.nan
    r = oracle.verify_sequence(q_rows, bad, [1, 2, 3], u, 1.0)
    assert r["n"] == -2 and r["tokens"] == [-1] * (K + 1)
    r = oracle.verify_sequence(q_rows, bad, [1, -1, 3], u, 1.0)
    assert r["n"] == -1  # an invalid id wins over an invalid row
    bad = q_rows.copy()
    bad[0, :] = -np.inf
    assert oracle.verify_sequence(bad, p_rows, [1, 2, 3], u, 1.0)["n"] == -2
    bad = p_rows.copy()
    bad[0, 0] = np.inf
    assert oracle.verify_sequence(q_rows, bad, [1, 2, 3], u, 1.0)["n"] == -2
    # greedy sequences never look at draft rows
    bad = q_rows.copy()
    bad[:] = np.nan
    r = oracle.verify_sequence(bad, p_rows, [1, 2, 3], u, 1.0, greedy=True)
    assert r["n"] >= 0


def test_rows_past_the_first_rejection_are_not_read():
    """R8 checks the rows the steps read: a NaN or +inf past the first
    rejection (or in the bonus row when a draft is rejected) changes nothing,
    while the same value in the bonus row of an all-accepted sequence fails it."""
    V, K = 16, 3
    rng = np.random.default_rng(11)
    q_rows, p_rows = rng.normal(0, 1, (K, V)), rng.normal(0, 1, (K + 1, V))
    x = [4, 2, 3]
    p_rows[0, 4] = -np.inf  # p_0(x_0) = 0: position 0 always rejects
    u = [0.5] * (K + 1)
    ref = oracle.verify_sequence(q_rows, p_rows, x, u, 1.0)
    assert ref["n"] == 0
    for row, col in ((1, 3), (2, 0), (3, 7)):
        bad = p_rows.copy()
        bad[row, col] = np.nan
        r = oracle.verify_sequence(q_rows, bad, x, u, 1.0)
        assert r["n"] == 0 and r["tokens"] == ref["tokens"]
        bad[row, col] = np.inf
        assert oracle.verify_sequence(q_rows, bad, x, u, 1.0)["tokens"] == ref["tokens"]
    badq = q_rows.copy()
    badq[2, :] = np.nan
    assert oracle.verify_sequence(badq, p_rows, x, u, 1.0)["tokens"] == ref["tokens"]
    # identical rows accept everything: the bonus row is read and must be valid
    same_q, same_p = p_rows[:K].copy(), p_rows.copy()
    same_q[0, 4] = same_p[0, 4] = 0.0
    ok = oracle.verify_sequence(same_q, same_p, x, u, 1.0)
    assert ok["n"] == K
    same_p[K, 1] = np.nan
    assert oracle.verify_sequence(same_q, same_p, x, u, 1.0)["n"] == -2
    # greedy: position 0 rejects (x_0 is not the argmax), later rows are unread
    g = p_rows.copy()
    g[0, :] = 0.0
    g[0, 9] = 5.0
    g[2, :] = np.nan
    r = oracle.verify_sequence(None, g, [1, 2, 3], u, 1.0, greedy=True)
    assert r["n"] == 0 and r["tokens"][0] == 9
    g[0, 3] = np.nan
    assert oracle.verify_sequence(None, g, [1, 2, 3], u, 1.0, greedy=True)["n"] == -2


def test_residual_zero_falls_back_to_target():
    """If the residual mass is exactly zero the resample draws from p."""
    p = np.array([0.25, 0.25, 0.5])
    j, Z, _ = oracle.inverse_cdf(oracle.residual(p, p), 0.6)
    assert j is None and Z == 0.0


def test_batch_driver_matches_per_sequence_calls_ragged():
    rng = np.random.default_rng(11)
    V, B = 64, 5
    Ks = np.array([2, 0, 3, 1, 4])
    cu = np.concatenate([[0], np.cumsum(Ks)])
    draft = rng.normal(0, 2, (cu[-1], V)).astype(np.float32)
    target = rng.normal(0, 2, (cu[-1] + B, V)).astype(np.float32)
    toks = rng.integers(0, V, cu[-1]).astype(np.int32)
    u = rng.random(cu[-1] + B).astype(np.float32)
    greedy = np.array([False, False, True, False, True])
    res = oracle.verify(draft, target, toks, u, B=B, V=V, dtype="f32", cu_draft=cu,
                        temperature=0.9, greedy=greedy)
    for b in range(B):
        d0, d1 = cu[b], cu[b + 1]
        t0, t1 = d0 + b, d1 + b + 1
        r = oracle.verify_sequence(draft[d0:d1].astype(np.float64), target[t0:t1].astype(np.float64),
                                   toks[d0:d1], u[t0:t1].astype(np.float64), 0.9, greedy=bool(greedy[b]))
        assert list(res["out_tokens"][t0:t1]) == r["tokens"]
        assert res["num_accepted"][b] == r["n"]
