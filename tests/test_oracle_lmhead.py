"""Pins of the LM-head oracle (CPU): the logits it forms are h W^T, exactly,
in the orientation a model's last layer uses, and verification on them is the
already-pinned step on those rows."""

import numpy as np

import oracle
import workloads as W


def test_logits_are_explicit_dot_products():
    """l[r, v] = sum_d h[r, d] w[v, d], written out as Python loops."""
    rng = np.random.default_rng(5)
    h = rng.standard_normal((3, 7))
    w = rng.standard_normal((5, 7))
    got = oracle.lmhead_logits(h, w, scale=0.5)
    for r in range(3):
        for v in range(5):
            want = 0.5 * sum(float(h[r, d]) * float(w[v, d]) for d in range(7))
            assert abs(got[r, v] - want) <= 1e-14 * max(1.0, abs(want))


def test_integer_operands_are_exact():
    """Integer operands of the workload's ranges: the product equals the
    exact integer matmul at a hidden size near the largest the recipe allows
    without rounding in fp32."""
    rng = np.random.default_rng(6)
    d = 8192
    h = rng.integers(-8, 9, size=(4, d), dtype=np.int8)
    w = rng.integers(-64, 65, size=(9, d), dtype=np.int8)
    exact = h.astype(np.int64) @ w.astype(np.int64).T
    got = oracle.lmhead_logits(h, w, scale=W.LM_H_SCALE * W.LM_W_SCALE)
    assert np.array_equal(got, exact.astype(np.float64) / 4096.0)
    # the extreme: every term at its largest magnitude
    hmax = np.full((1, d), 8, dtype=np.int8)
    wmax = np.full((1, d), -64, dtype=np.int8)
    assert oracle.lmhead_logits(hmax, wmax)[0, 0] == -8 * 64 * d


def test_orientation_with_a_permutation_head():
    """W = permutation matrix (W[v, perm[v]] = 1): logit v is hidden entry
    perm[v]. A transposed product would give entry perm^-1[v] instead; the
    permutation is a 5-cycle, so the two differ everywhere but the fixed point."""
    perm = np.array([1, 2, 3, 4, 0, 5])
    w = np.zeros((6, 6), dtype=np.int8)
    w[np.arange(6), perm] = 1
    h = np.arange(12, dtype=np.int8).reshape(2, 6) - 3
    got = oracle.lmhead_logits(h, w)
    assert np.array_equal(got, h[:, perm].astype(np.float64))


def test_verify_lmhead_with_identity_head_is_verify_on_the_hidden_rows():
    """With W = I (V = D) the logits are the hidden rows themselves, so the
    LM-head verification must equal verification of those rows as logits."""
    rng = np.random.default_rng(7)
    B, K, V = 3, 4, 16
    hq = rng.integers(-8, 9, size=(B * K, V)).astype(np.int8)
    hp = rng.integers(-8, 9, size=(B * (K + 1), V)).astype(np.int8)
    eye = np.eye(V, dtype=np.int8)
    lq = hq.astype(np.float64) / 4.0
    lp = hp.astype(np.float64) / 4.0
    u_draft = rng.random(B * K, dtype=np.float32)
    uniforms = rng.random(B * (K + 1), dtype=np.float32)
    toks, _ = oracle.sample_rows(lq, u_draft, V=V, dtype="f64", temperature=0.9)
    a = oracle.verify_lmhead(hq, eye, hp, eye, toks, uniforms, B=B, K=K, V=V, temperature=0.9,
                             draft_scale=0.25, target_scale=0.25)
    b = oracle.verify(lq, lp, toks, uniforms, B=B, V=V, K=K, dtype="f64", temperature=0.9)
    assert np.array_equal(a["out_tokens"], b["out_tokens"])
    assert np.array_equal(a["num_accepted"], b["num_accepted"])


def test_greedy_verify_lmhead_by_hand():
    """Temperature 0 on an identity head: the target logits are the hidden
    rows, each position's check is draft token == the row's argmax (the lowest
    id on ties), and the emitted token at the first mismatch, or the bonus,
    is that argmax ([P3] section "Cùng phân bố không có nghĩa cùng chuỗi mỗi
    lần": greedy decoding checks the argmax). No draft hidden states are read."""
    rng = np.random.default_rng(11)
    B, K, V = 3, 4, 16
    hp = rng.integers(-8, 9, size=(B * (K + 1), V)).astype(np.int8)
    eye = np.eye(V, dtype=np.int8)
    am = np.argmax(hp.astype(np.int64), axis=1).reshape(B, K + 1)  # first maximum
    toks = am[:, :K].copy()
    toks[1, 1] = (toks[1, 1] + 1) % V  # sequence 1 stops at position 1
    toks[2, 0] = (toks[2, 0] + 3) % V  # sequence 2 stops at position 0
    res = oracle.verify_lmhead(None, None, hp, eye, toks.reshape(-1), np.zeros(B * (K + 1)),
                               B=B, K=K, V=V, temperature=0.0)
    want_n = [K, 1, 0]
    want = np.full((B, K + 1), -1)
    for b, n in enumerate(want_n):
        want[b, :n] = toks[b, :n]
        want[b, n] = am[b, n]
    assert res["num_accepted"].tolist() == want_n
    assert np.array_equal(res["out_tokens"].reshape(B, K + 1), want)


def test_workload_recipe_shares_the_draft_directions():
    """The generator's target logits at position i < K are the draft logits
    plus the term of the target's extra hidden entries (checked through the
    oracle's products); the bonus position is fresh."""
    w = W.make_lmhead(B=2, K=3, V=50, d_draft=16, d_target=40, seed=11)
    lq = oracle.lmhead_logits(w["hq"], w["wq"])
    lp = oracle.lmhead_logits(w["hp"], w["wp"])
    extra = oracle.lmhead_logits(w["hp"][:, 16:], w["wp"][:, 16:])
    for b in range(2):
        for i in range(3):
            assert np.array_equal(lp[b * 4 + i], lq[b * 3 + i] + extra[b * 4 + i])
    assert np.array_equal(w["wp"][:, :16], w["wq"])
