"""Float64 oracle of verification with several draft chains (CPU, numpy).

TEST INFRASTRUCTURE ONLY: imported by tests/; never by the library it checks.

[P2] part "1、第16講" notes that there can be several drafters but gives no
rule for checking their proposals. The rule here is the pages' own single
step applied again: [P1] s.6 shows that accepting a draft x ~ q with
probability min(1, p(x)/q(x)), and otherwise drawing from
max(0, p - q)/Z, is rejection sampling whose result follows p. Let r be the
law a step must reproduce. Test one candidate x ~ q against it: accept with
probability min(1, r(x)/q(x)); on a rejection the rest of the law is
max(0, r - q)/Z. That remainder is the law the next candidate is tested
against, drawn independently from its own drafter. By induction over the
candidates the result follows r. When every candidate is rejected, the token
is drawn from the last remainder.

Chains. M draft chains of K tokens share the prefix; chain m's rows at
position j are conditioned on that chain's own tokens 0..j-1. The step above
checks position j against the chains still alive: those whose tokens so far
equal the accepted ones, in chain order. All of them share the accepted
prefix, so the target row of position j is the one of the lowest live chain
(the caller's target rows of chains with equal prefixes must agree). After a
candidate is accepted, the chains whose token at j equals the accepted token
stay alive. Their next tokens are independent draws given that prefix, so
the next position is checked the same way. The bonus position K draws from
the lowest live chain's target row.

Filters and greedy verification as for one chain (aihero.vn "Speculative
decoding", section "Cùng phân bố không có nghĩa cùng chuỗi mỗi lần": the same
temperature, top-k and top-p on both models' rows, and a greedy check):
every row's law is its filtered distribution (R6), and the top-p margins of
the rows a walk uses join its margin. With temperature 0 the target law is a
point mass at the argmax (lowest id on ties), so the step above accepts a
candidate exactly when it equals that argmax, and a rejection leaves the law
unchanged: the first live chain whose token is the argmax is accepted, and
when none is, the argmax is emitted (the bonus position emits it too). Only
target rows are read then.

Layout (per sequence): q_rows [M, K, V], p_rows [M, K+1, V], x [M, K]; the
uniforms u [K+1, M+1]: u[j, m] tests chain m's candidate at position j,
u[j, M] is the draw at j (taken only at the position where the walk stops).
Readings R1-R8 of oracle/verify.py hold (accept iff u < r(x)/q(x); the
inverse CDF over ascending ids; a remainder whose mass rounds to zero keeps
the previous law; invalid ids -1, invalid used rows -2).
"""

import math

import numpy as np

from .verify import (ACCEPT_MARGIN_INF, accept_ratio, decode_logits, filtered_distribution,
                     greedy_token, inverse_cdf, residual, row_is_valid)


def verify_multi_sequence(q_rows, p_rows, x, u, temperature, top_k=0, top_p=1.0):
    """One sequence with M candidate chains (see the module docstring);
    temperature 0 verifies greedily.

    Returns dict(tokens (K+1, -1 padded), n, chosen [K+1] (the chain whose
    candidate was accepted at each position, -1 where the token was drawn or
    nothing was emitted), chain (the lowest chain holding the emitted prefix),
    margin (smallest distance of a used uniform from its threshold))."""
    q_rows = np.asarray(q_rows, np.float64)
    p_rows = np.asarray(p_rows, np.float64)
    x = np.asarray(x, np.int64)
    M, K = x.shape
    V = p_rows.shape[2]
    tokens = [-1] * (K + 1)
    chosen = [-1] * (K + 1)
    res = dict(tokens=tokens, n=0, chosen=chosen, chain=0, margin=ACCEPT_MARGIN_INF)
    if np.any((x < 0) | (x >= V)):
        res["n"] = -1
        return res
    margin = ACCEPT_MARGIN_INF
    live = list(range(M))
    greedy = temperature == 0.0
    for j in range(K + 1):
        lead = live[0]
        if not row_is_valid(p_rows[lead, j]):
            return dict(res, n=-2, tokens=[-1] * (K + 1), chosen=[-1] * (K + 1))
        if greedy:
            a = greedy_token(p_rows[lead, j])
            tokens[j] = a
            accepted = None if j == K else next((m for m in live if int(x[m, j]) == a), None)
            if accepted is None:
                res.update(n=j, chain=lead)
                return res
            chosen[j] = accepted
            live = [m for m in live if int(x[m, j]) == a]
            continue
        r, _, mp = filtered_distribution(p_rows[lead, j], temperature, top_k, top_p)
        margin = min(margin, mp)
        if j == K:
            t, _, m_ = inverse_cdf(r, float(u[K][M]))
            tokens[K] = t
            res.update(n=K, chain=lead, margin=min(margin, m_))
            return res
        accepted = None
        for m in live:
            if not row_is_valid(q_rows[m, j]):
                return dict(res, n=-2, tokens=[-1] * (K + 1), chosen=[-1] * (K + 1))
            q, _, mq = filtered_distribution(q_rows[m, j], temperature, top_k, top_p)
            ratio = accept_ratio(r, q, int(x[m, j]))
            margin = min(margin, mq, abs(float(u[j][m]) - ratio))
            if float(u[j][m]) < ratio:
                accepted = m
                break
            rho = residual(r, q)
            z = rho.sum()
            if z > 0.0:
                r = rho / z
        if accepted is None:
            t, _, m_ = inverse_cdf(r, float(u[j][M]))
            tokens[j] = t
            res.update(n=j, chain=lead, margin=min(margin, m_))
            return res
        t = int(x[accepted, j])
        tokens[j] = t
        chosen[j] = accepted
        live = [m for m in live if int(x[m, j]) == t]
    raise AssertionError("the bonus position always ends the walk")


def verify_multi(draft, target, draft_tokens, uniforms, *, B, M, K, V, dtype, temperature,
                 top_k=0, top_p=1.0):
    """Batch driver: draft [B, M, K, V], target [B, M, K+1, V] storage arrays,
    draft_tokens [B, M, K], uniforms [B, K+1, M+1] (float32 values);
    temperature 0 verifies greedily (the draft rows are not read, draft may be
    None). Returns dict(out_tokens [B*(K+1)] int32, num_accepted [B] int32,
    chain [B] int32, chosen [B*(K+1)] int32, margin [B] float64)."""
    if not (temperature >= 0.0) or math.isinf(temperature):
        raise ValueError("temperature must be finite and >= 0")
    if temperature == 0.0 and draft is None:
        d = np.zeros((B, M, K, V))
    else:
        d = decode_logits(np.asarray(draft), dtype).reshape(B, M, K, V)
    t = decode_logits(np.asarray(target), dtype).reshape(B, M, K + 1, V)
    x = np.asarray(draft_tokens).reshape(B, M, K)
    u = np.asarray(uniforms, np.float32).astype(np.float64).reshape(B, K + 1, M + 1)
    out = np.full(B * (K + 1), -1, np.int32)
    chosen = np.full(B * (K + 1), -1, np.int32)
    num = np.zeros(B, np.int32)
    chain = np.zeros(B, np.int32)
    margin = np.full(B, ACCEPT_MARGIN_INF)
    for b in range(B):
        r = verify_multi_sequence(d[b], t[b], x[b], u[b], temperature, top_k, top_p)
        out[b * (K + 1):(b + 1) * (K + 1)] = r["tokens"]
        chosen[b * (K + 1):(b + 1) * (K + 1)] = r["chosen"]
        num[b] = r["n"]
        chain[b] = r["chain"]
        margin[b] = r["margin"]
    return dict(out_tokens=out, num_accepted=num, chain=chain, chosen=chosen, margin=margin)
