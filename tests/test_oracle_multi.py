"""Pins of the several-chain verification oracle (oracle/multi.py).

- One chain is the single-draft verification (verify_sequence) with its
  uniforms laid out accordingly.
- The pages' two-token example (aihero.vn "Speculative decoding", section
  "Chấp nhận bằng tỉ lệ, không chỉ bằng argmax": q = [0.4, 0.6],
  p = [0.3, 0.7]) with two candidates from the same draft: by exact
  enumeration the output is still [0.3, 0.7], and a draft token is emitted
  with probability 1 - (0.4 * 1/4) * 0.4 = 24/25. One candidate gives 9/10:
  the second candidate is tested against the rejected mass, all on B.
- Exact enumeration on random small trees: the token emitted at position 0
  follows p_0, and the token at position 1, given that position 0 emitted t,
  follows the target row after the prefix t ([P1] s.6: the result follows
  the target). With top-k / top-p the same holds for the filtered target
  rows, candidates drawn from the filtered draft rows.
- With filters, and greedily (temperature 0), one chain is again the
  single-draft verification; a greedy hand example with several chains and a
  tied argmax (lowest id).
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from exact_multi import enumerate_multi


def test_one_chain_is_single_draft_verification():
    rng = np.random.default_rng(11)
    K, V, T = 4, 50, 0.9
    for trial in range(60):
        q = rng.normal(0, 2, (K, V))
        p = np.concatenate([q, rng.normal(0, 2, (1, V))]) + rng.normal(0, 1.0, (K + 1, V))
        x = rng.integers(0, V, K)
        u1 = rng.random(K + 1)
        single = oracle.verify_sequence(q, p, x, u1, T)
        um = np.stack([u1[:K + 1], np.full(K + 1, u1[K])], axis=1)  # [K+1, 2]
        multi = oracle.verify_multi_sequence(q[None], p[None], x[None], um, T)
        assert multi["n"] == single["n"] and multi["tokens"] == single["tokens"], trial
        assert multi["chain"] == 0


def _laws(outcomes, V):
    law0 = np.zeros(V)
    emitted = 0.0
    for prob, n, prefix, dist in outcomes:
        if n == 0:
            law0 += prob * dist
        else:
            law0[prefix[0]] += prob
            emitted += prob
    return law0, emitted


def test_printed_two_token_example_with_two_candidates():
    q = np.log(np.array([[0.4, 0.6]]))
    p = np.log(np.array([[0.3, 0.7], [0.5, 0.5]]))
    qrows = np.stack([q, q])               # [M=2, K=1, V=2]
    prows = np.stack([p, p])               # [M=2, K+1=2, V=2]
    qp = np.array([0.4, 0.6])
    law = np.zeros(2)
    passed = 0.0
    for x0, x1 in itertools.product(range(2), repeat=2):
        x = np.array([[x0], [x1]])
        w = qp[x0] * qp[x1]
        l0, e = _laws(enumerate_multi(qrows, prows, x, 1.0), 2)
        law += w * l0
        passed += w * e
    assert law == pytest.approx([0.3, 0.7], abs=1e-12)
    assert passed == pytest.approx(float(1 - Fraction(2, 5) * Fraction(1, 4) * Fraction(2, 5)),
                                   abs=1e-12)
    # one candidate: the page's own acceptance, 0.4 * 3/4 + 0.6 = 9/10
    single = sum(qp[x0] * _laws(enumerate_multi(q[None], p[None], np.array([[x0]]), 1.0), 2)[1]
                 for x0 in range(2))
    assert single == pytest.approx(0.9, abs=1e-12)


@pytest.mark.parametrize("M,K,V,seed", [(2, 1, 4, 0), (3, 1, 3, 1), (2, 2, 3, 2)])
def test_tree_outputs_follow_target_rows(M, K, V, seed):
    rng = np.random.default_rng([31, seed])
    T = 0.8
    qfun, pfun = {}, {}

    def qrow(m, prefix):  # drafter m's logits after its own prefix
        return qfun.setdefault((m, prefix), rng.normal(0, 1.5, V))

    def prow(prefix):     # the target's logits after a prefix (shared by chains)
        return pfun.setdefault(prefix, rng.normal(0, 1.5, V))

    law0 = np.zeros(V)
    law1 = {t: np.zeros(V) for t in range(V)}
    reach1 = np.zeros(V)
    for flat in itertools.product(range(V), repeat=M * K):
        x = np.array(flat).reshape(M, K)
        qrows = np.stack([[qrow(m, tuple(x[m, :j])) for j in range(K)] for m in range(M)])
        prows = np.stack([[prow(tuple(x[m, :j])) for j in range(K + 1)] for m in range(M)])
        w = 1.0
        for m in range(M):
            for j in range(K):
                w *= softmax(qrows[m, j] / T)[x[m, j]]
        for prob, n, prefix, dist in enumerate_multi(qrows, prows, x, T):
            pw = w * prob
            if n == 0:
                law0 += pw * dist
                continue
            t = prefix[0]
            law0[t] += pw
            reach1[t] += pw
            law1[t] += pw * (dist if n == 1 else np.eye(V)[prefix[1]])
    assert law0 == pytest.approx(softmax(prow(()) / T), abs=1e-9)
    for t in range(V):
        if reach1[t] > 1e-6:
            assert law1[t] / reach1[t] == pytest.approx(softmax(prow((t,)) / T), abs=1e-8), t


@pytest.mark.parametrize("top_k,top_p,T", [(5, 1.0, 0.9), (0, 0.7, 0.9), (8, 0.8, 1.3),
                                           (0, 1.0, 0.0), (5, 0.7, 0.0)])
def test_one_chain_is_single_draft_verification_filtered_and_greedy(top_k, top_p, T):
    rng = np.random.default_rng([12, top_k, int(top_p * 10), int(T * 10)])
    K, V = 4, 40
    for trial in range(40):
        q = rng.normal(0, 2, (K, V))
        p = np.concatenate([q, rng.normal(0, 2, (1, V))]) + rng.normal(0, 1.0, (K + 1, V))
        if T == 0.0:
            # greedy drafts: often the target's argmax too, so some prefixes pass
            x = np.array([int(np.argmax(p[i] if rng.random() < 0.6 else q[i])) for i in range(K)])
        else:
            x = rng.integers(0, V, K)
        u1 = rng.random(K + 1)
        single = oracle.verify_sequence(q, p, x, u1, T, top_k, top_p, greedy=T == 0.0)
        um = np.stack([u1[:K + 1], np.full(K + 1, u1[K])], axis=1)  # [K+1, 2]
        multi = oracle.verify_multi_sequence(q[None], p[None], x[None], um, T, top_k, top_p)
        assert multi["n"] == single["n"] and multi["tokens"] == single["tokens"], trial
        if T > 0.0:
            assert multi["margin"] == pytest.approx(single["margin"], abs=1e-12), trial


def test_greedy_several_chains_hand_example():
    V, K = 6, 2
    p = np.full((3, K + 1, V), -5.0)
    p[:, 0, 4] = 2.0           # position 0: argmax 4
    p[:, 1, 1] = 3.0           # position 1 after the prefix [4]: ids 1 and 3 tie, lowest id 1
    p[:, 1, 3] = 3.0
    p[:, 2, 5] = 1.0           # bonus: argmax 5
    q = np.zeros((3, K, V))
    u = np.full((K + 1, 4), 0.5)
    # chains 0 and 2 propose 4 then 1, chain 1 proposes 2: chain 0 accepted twice, then bonus 5
    res = oracle.verify_multi_sequence(q, p, np.array([[4, 1], [2, 2], [4, 1]]), u, 0.0)
    assert res["n"] == 2 and res["tokens"] == [4, 1, 5] and res["chosen"] == [0, 0, -1]
    assert res["chain"] == 0
    # only chain 1 proposes the argmax at position 0, then 3 (tied, not the lowest id)
    res = oracle.verify_multi_sequence(q, p, np.array([[0, 1], [4, 3], [2, 1]]), u, 0.0)
    assert res["n"] == 1 and res["tokens"] == [4, 1, -1] and res["chosen"] == [1, -1, -1]
    assert res["chain"] == 1
    # no chain proposes the argmax: the argmax is emitted at position 0
    res = oracle.verify_multi_sequence(q, p, np.array([[0, 1], [2, 3], [3, 1]]), u, 0.0)
    assert res["n"] == 0 and res["tokens"] == [4, -1, -1] and res["chain"] == 0
    # a NaN target row on the path is an invalid row; draft rows are not read
    p2 = p.copy()
    p2[0, 1, 2] = np.nan
    qn = np.full((3, K, V), np.nan)
    res = oracle.verify_multi_sequence(qn, p2, np.array([[4, 1], [2, 2], [4, 1]]), u, 0.0)
    assert res["n"] == -2


@pytest.mark.parametrize("M,K,V,top_k,top_p,seed", [(2, 1, 5, 3, 1.0, 0), (2, 1, 5, 0, 0.75, 1),
                                                   (2, 2, 4, 3, 0.8, 2)])
def test_tree_outputs_follow_filtered_target_rows(M, K, V, top_k, top_p, seed):
    rng = np.random.default_rng([32, seed])
    T = 0.9
    qfun, pfun = {}, {}

    def qrow(m, prefix):
        return qfun.setdefault((m, prefix), rng.normal(0, 1.5, V))

    def prow(prefix):
        return pfun.setdefault(prefix, rng.normal(0, 1.5, V))

    def filt(row):
        return oracle.filtered_distribution(row, T, top_k, top_p)[0]

    law0 = np.zeros(V)
    law1 = {t: np.zeros(V) for t in range(V)}
    reach1 = np.zeros(V)
    total = 0.0
    for flat in itertools.product(range(V), repeat=M * K):
        x = np.array(flat).reshape(M, K)
        qrows = np.stack([[qrow(m, tuple(x[m, :j])) for j in range(K)] for m in range(M)])
        prows = np.stack([[prow(tuple(x[m, :j])) for j in range(K + 1)] for m in range(M)])
        w = 1.0
        for m in range(M):
            for j in range(K):
                w *= filt(qrows[m, j])[x[m, j]]
        if w == 0.0:
            continue  # a draft outside its drafter's kept set is never proposed
        total += w
        for prob, n, prefix, dist in enumerate_multi(qrows, prows, x, T, top_k, top_p):
            pw = w * prob
            if n == 0:
                law0 += pw * dist
                continue
            t = prefix[0]
            law0[t] += pw
            reach1[t] += pw
            law1[t] += pw * (dist if n == 1 else np.eye(V)[prefix[1]])
    assert total == pytest.approx(1.0, abs=1e-12)
    assert law0 == pytest.approx(filt(prow(())), abs=1e-9)
    for t in range(V):
        if reach1[t] > 1e-6:
            assert law1[t] / reach1[t] == pytest.approx(filt(prow((t,))), abs=1e-8), t

