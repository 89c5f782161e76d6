"""Plain float64 oracle of speculative-decoding verification (CPU, numpy).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py; never by the library it checks.

Pages followed (cited by title and section; the tags are used below):
  [P1] aivaro.ru, answer 289, "Как работает speculative decoding на уровне
       логитов, а не токенов?" -- numbered sections 1..12 (section 5 "Алгоритм
       ... (пошагово)", steps 1-4; section 6 "Математическая основа"; section 9
       "Реализация: псевдокод на Python").
  [P2] CSDN notes of Hung-yi Lee, "Introduction to Generative AI 2024",
       lecture 16 ("【Hung-yi Lee】《Introduction to Generative Artificial
       Intelligence》（11）") -- part "3、举个例子", item 3 (rejection sampling);
       part "4、推测解码验证流程图", items 1-4 (parallel scoring, token
       validation, truncation and correction, bonus token).
  [P3] aihero.vn, "Speculative decoding" -- sections "Chấp nhận bằng tỉ lệ,
       không chỉ bằng argmax" (accept by ratio), "Cùng phân bố không có nghĩa
       cùng chuỗi mỗi lần" (same distribution, not same sequence) and
       "Bài tập: chứng minh lại một phân bố hai token" (exercise).

Notation: q is the draft distribution and p the target distribution at the same
prefix ([P3] accept-by-ratio section). For one sequence with K drafts there are
K draft rows q_0..q_{K-1}, K+1 target rows p_0..p_K and K draft tokens
x_0..x_{K-1}; target row i is conditioned on the same prefix as draft row i, and
row K is the distribution after all K drafts ([P2] part 4, items 1 and 4).

Readings taken where the pages leave a step open (each is repeated where used):
  R1  accept iff u_i < r_i with r_i = p_i(x_i)/q_i(x_i), strict ([P1] s.9 draws
      a uniform and compares it with "<"); u == r rejects.
  R2  q(x) = 0 with p(x) > 0 gives r = +inf (always accepted); q(x) = p(x) = 0
      gives r = 0 (always rejected).
  R3  uniforms[K] is the single draw used either by the residual resample at the
      first rejected position or by the bonus sample; the two are exclusive.
  R4  categorical sampling (the pages' multinomial) is the inverse CDF over
      ascending token ids: the smallest j with C_j > u * Z, C_j = sum_{t<=j} w_t;
      if rounding leaves no such j, the largest j with w_j > 0.
  R5  if the residual mass Z rounds to <= 0 the resample uses p_n instead.
  R6  temperature, then top-k (value threshold, ties kept), then top-p (keep j
      iff the mass of kept tokens with a strictly larger logit is < top_p,
      computed on the softmax of the top-k set); each row filtered on its own
      logits with the same settings ([P3] same-distribution section).
  R7  greedy: argmax of the raw target logits, lowest id on ties; accept iff it
      equals the draft token; the correction or bonus is that argmax.
  R8  a sequence with a draft id outside [0, V) returns n = -1; otherwise one
      whose used rows hold NaN or +inf, or no finite value, returns n = -2. The
      used rows are those the steps read: draft and target rows of positions
      0..n (the ratio tests up to the first rejection and the resample at n),
      and the bonus row when every draft passes; rows past the first rejection
      are never read. Greedy sequences use no draft rows. All tokens are -1
      then.
"""

import math

import numpy as np

# Margin assigned to decisions that cannot flip under rounding.
ACCEPT_MARGIN_INF = math.inf


# --------------------------------------------------------------------------
# Input decoding: the same bytes the GPU reads, widened exactly to float64.
# --------------------------------------------------------------------------
def decode_logits(raw, dtype):
    """Widen stored logits to float64 exactly.

    ``raw`` is the storage array: float32 for 'f32', float16 (or its uint16
    bits) for 'f16', the uint16 bit patterns for 'bf16', float64 for 'f64'
    (test convenience). Every one of these converts to float64 without
    rounding.
    """
    a = np.asarray(raw)
    if dtype == "f64":
        return a.astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32, copy=False).astype(np.float64)
    if dtype == "f16":
        if a.dtype != np.float16:
            a = a.view(np.float16)
        return a.astype(np.float64)
    if dtype == "bf16":
        bits = a.view(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def row_is_valid(l):
    """R8: a usable row has no NaN, no +inf and at least one finite value."""
    if np.isnan(l).any() or np.isposinf(l).any():
        return False
    return bool(np.isfinite(l).any())


# --------------------------------------------------------------------------
# Step 0: temperature / top-k / top-p, then softmax ([P3] same-distribution
# section asks for these to be applied consistently to both models; [P1] s.1
# and s.9 define probabilities as the softmax of logits).
# --------------------------------------------------------------------------
def _softmax_over(z, keep):
    """Softmax of z restricted to the boolean mask ``keep`` (zeros elsewhere).

    Returns (probabilities, log of the partition sum sum_{keep} exp(z))."""
    m = z[keep].max()
    e = np.zeros_like(z)
    e[keep] = np.exp(z[keep] - m)
    s = e.sum()
    return e / s, m + math.log(s)


def _top_k_keep(z, top_k):
    """R6 top-k: keep every logit >= the k-th largest one (ties kept)."""
    V = z.shape[0]
    if top_k <= 0 or top_k >= V:
        return np.ones(V, dtype=bool)
    kth_largest = np.partition(z, V - top_k)[V - top_k]
    return z >= kth_largest


def _top_p_keep(z, keep, top_p):
    """R6 top-p on the softmax of the kept set.

    Token j stays iff the probability mass of kept tokens whose logit is
    strictly larger than z_j is below top_p. Returns (new mask, margin), where
    margin is the distance between top_p and the nearest "mass strictly above"
    value of any kept logit level (the decision that rounding could flip)."""
    if top_p >= 1.0:
        return keep, ACCEPT_MARGIN_INF
    pi, _ = _softmax_over(z, keep)
    levels, inv = np.unique(z[keep], return_inverse=True)  # ascending levels
    level_mass = np.zeros(levels.shape[0])
    np.add.at(level_mass, inv, pi[keep])
    # mass of all strictly larger levels, for each level (descending cumsum)
    above = np.concatenate([np.cumsum(level_mass[::-1])[::-1][1:], [0.0]])
    level_kept = above < top_p
    new_keep = keep.copy()
    new_keep[np.flatnonzero(keep)] = level_kept[inv]
    margin = float(np.min(np.abs(above - top_p)))
    return new_keep, margin


def filtered_distribution(l, temperature, top_k=0, top_p=1.0):
    """Probabilities of one row after temperature, top-k and top-p (R6).

    ``l`` is a float64 logit row. Returns (prob, lse, topp_margin): prob is zero
    outside the kept set, lse = log sum_{kept} exp(l / T)."""
    z = l / temperature
    keep = np.isfinite(z) if np.isneginf(z).any() else np.ones(z.shape[0], bool)
    keep &= _top_k_keep(z, top_k)
    keep, margin = _top_p_keep(z, keep, top_p)
    prob, lse = _softmax_over(z, keep)
    return prob, lse, margin


# --------------------------------------------------------------------------
# Step 1: ratio test ([P1] s.5 step 3 and s.6: accept(x) = min(1, p/q);
# [P2] part 3 item 3; [P3] accept-by-ratio section).
# --------------------------------------------------------------------------
def accept_ratio(p, q, x):
    """r = p(x) / q(x) with R2 for q(x) = 0. Acceptance probability is min(1, r)."""
    if q[x] > 0.0:
        return p[x] / q[x]
    return math.inf if p[x] > 0.0 else 0.0


# --------------------------------------------------------------------------
# Step 2: residual distribution after a rejection ([P1] s.5 step 3 and s.6:
# p_corrected proportional to max(0, p - q); [P3] accept-by-ratio section).
# --------------------------------------------------------------------------
def residual(p, q):
    """Unnormalised residual weights max(0, p - q) (normalised by the sampler)."""
    return np.maximum(p - q, 0.0)


# --------------------------------------------------------------------------
# Step 3: categorical draw by inverse CDF with a supplied uniform (R4); stands in
# for the pages' torch.multinomial ([P1] s.9).
# --------------------------------------------------------------------------
def inverse_cdf(w, u):
    """Smallest j with C_j > u * Z (C = sequential cumulative sum of w, Z = C[-1]).

    Returns (j, Z, margin) where margin is the distance from u to the nearer end
    of the chosen interval [C_{j-1}/Z, C_j/Z). Returns (None, Z, inf) if Z <= 0.
    """
    c = np.cumsum(w)
    total = c[-1]
    if not total > 0.0:
        return None, total, ACCEPT_MARGIN_INF
    t = u * total
    j = int(np.searchsorted(c, t, side="right"))
    if j >= c.shape[0]:
        j = int(np.flatnonzero(w > 0.0)[-1])
    lo = c[j - 1] / total if j > 0 else 0.0
    hi = c[j] / total
    margin = min(abs(u - lo), abs(hi - u))
    return j, total, margin


# --------------------------------------------------------------------------
# Greedy check ([P3] same-distribution section says greedy decoding verifies
# differently from sampling; R7 is the rule used).
# --------------------------------------------------------------------------
def greedy_token(l):
    """argmax of raw logits, lowest id on ties (numpy returns the first max)."""
    return int(np.argmax(l))


# --------------------------------------------------------------------------
# One sequence: the verification step in the pages' order.
# --------------------------------------------------------------------------
def verify_sequence(q_rows, p_rows, x, u, temperature, top_k=0, top_p=1.0,
                    greedy=False, want_diag=False):
    """Verify K draft tokens of one sequence.

    q_rows: float64 [K, V] draft logits (may be None when greedy).
    p_rows: float64 [K+1, V] target logits.
    x: K draft token ids; u: K+1 uniforms (R3).
    Returns dict(tokens (K+1 ints, -1 padded), n, margin, lse_q, lse_p,
    ratio, resid_Z). n is the number of accepted drafts or a negative code (R8).
    """
    K = len(x)
    V = p_rows.shape[1]
    tokens = [-1] * (K + 1)
    res = dict(tokens=tokens, n=0, margin=ACCEPT_MARGIN_INF,
               lse_q=[math.nan] * K, lse_p=[math.nan] * (K + 1),
               ratio=[math.nan] * K, resid_Z=math.nan)

    # R8: every draft id first; each row when the step that reads it comes.
    if any(not (0 <= int(t) < V) for t in x):
        res["n"] = -1
        return res

    def invalid(*rows):
        return not all(row_is_valid(r) for r in rows)

    def fail():
        res["n"] = -2
        res["tokens"] = [-1] * (K + 1)
        return res

    if greedy:
        # R7: compare the draft id with the target argmax, position by position.
        n = K
        for i in range(K):
            if invalid(p_rows[i]):
                return fail()
            if greedy_token(p_rows[i]) != int(x[i]):
                n = i
                break
        if n == K and invalid(p_rows[K]):
            return fail()
        for i in range(n):
            tokens[i] = int(x[i])
        tokens[n] = greedy_token(p_rows[n])
        res["n"] = n
        return res

    margin = ACCEPT_MARGIN_INF
    dists_p, dists_q = {}, {}

    def p_dist(i):
        if i not in dists_p:
            dists_p[i] = filtered_distribution(p_rows[i], temperature, top_k, top_p)
        return dists_p[i]

    def q_dist(i):
        if i not in dists_q:
            dists_q[i] = filtered_distribution(q_rows[i], temperature, top_k, top_p)
        return dists_q[i]

    # Ratio tests in order; stop at the first rejection ([P1] s.5 step 3 and
    # s.9; [P2] part 4 item 3; [P3] two-models section).
    n = K
    for i in range(K):
        if invalid(p_rows[i], q_rows[i]):
            return fail()
        p, _, mp = p_dist(i)
        q, _, mq = q_dist(i)
        r = accept_ratio(p, q, int(x[i]))
        margin = min(margin, mp, mq, abs(float(u[i]) - r))
        if float(u[i]) < r:  # R1
            tokens[i] = int(x[i])
            continue
        n = i
        break

    if n < K:
        # Resample the rejected position from the normalised residual (R4, R5).
        p, _, _ = p_dist(n)
        q, _, _ = q_dist(n)
        j, Z, m = inverse_cdf(residual(p, q), float(u[K]))
        if j is None:
            j, Z, m = inverse_cdf(p, float(u[K]))
    else:
        # Bonus token from the (K+1)-th target distribution ([P2] part 4 item 4).
        if invalid(p_rows[K]):
            return fail()
        p, _, mp = p_dist(K)
        margin = min(margin, mp)
        j, Z, m = inverse_cdf(p, float(u[K]))
    tokens[n] = j
    res["n"] = n
    res["margin"] = min(margin, m)
    res["resid_Z"] = Z

    if want_diag:
        # every valid row, used or not (an unused invalid row stays NaN)
        for i in range(K + 1):
            if row_is_valid(p_rows[i]):
                res["lse_p"][i] = p_dist(i)[1]
        for i in range(K):
            if row_is_valid(q_rows[i]):
                res["lse_q"][i] = q_dist(i)[1]
                if row_is_valid(p_rows[i]):
                    res["ratio"][i] = accept_ratio(p_dist(i)[0], q_dist(i)[0], int(x[i]))
    return res


# --------------------------------------------------------------------------
# Batch driver over packed rows (dense layout is the special case cu[b] = b*K).
# --------------------------------------------------------------------------
def verify(draft, target, draft_tokens, uniforms, *, B, V, dtype, K=None,
           cu_draft=None, temperature=1.0, top_k=0, top_p=1.0, greedy=None,
           want_diag=False):
    """Verify a batch.

    draft: storage array [sum K_b, V]; target: [sum (K_b+1), V]; draft_tokens:
    [sum K_b]; uniforms: [sum (K_b+1)] float32 values. Sequence b owns draft rows
    cu[b]..cu[b+1]-1 and target/uniform/output rows cu[b]+b..cu[b+1]+b.
    temperature == 0 makes every sequence greedy; otherwise ``greedy`` is an
    optional boolean mask [B].
    Returns dict(out_tokens [sum (K_b+1)] int32, num_accepted [B] int32,
    margin [B] float64, and when want_diag lse_draft, lse_target, ratio,
    resid_Z).
    """
    if not (temperature >= 0.0) or math.isinf(temperature):
        raise ValueError("temperature must be finite and >= 0")
    if not (0.0 < top_p <= 1.0):
        raise ValueError("top_p must lie in (0, 1]")
    if cu_draft is None:
        cu = np.arange(B + 1, dtype=np.int64) * int(K)
    else:
        cu = np.asarray(cu_draft, dtype=np.int64)
    draft = np.asarray(draft).reshape(-1, V) if draft is not None else None
    target = np.asarray(target).reshape(-1, V)
    x_all = np.asarray(draft_tokens).reshape(-1)
    u_all = np.asarray(uniforms, dtype=np.float32).reshape(-1).astype(np.float64)
    n_target = int(cu[B]) + B
    out = np.full(n_target, -1, dtype=np.int32)
    num = np.zeros(B, dtype=np.int32)
    margin = np.full(B, ACCEPT_MARGIN_INF)
    diag = dict(lse_draft=np.full(int(cu[B]), np.nan),
                lse_target=np.full(n_target, np.nan),
                ratio=np.full(int(cu[B]), np.nan),
                resid_Z=np.full(B, np.nan))
    for b in range(B):
        d0, d1 = int(cu[b]), int(cu[b + 1])
        t0, t1 = d0 + b, d1 + b + 1
        g = temperature == 0.0 or (greedy is not None and bool(greedy[b]))
        p_rows = decode_logits(target[t0:t1], dtype)
        q_rows = None if g else decode_logits(draft[d0:d1], dtype)
        r = verify_sequence(q_rows, p_rows, x_all[d0:d1], u_all[t0:t1],
                            temperature, top_k, top_p, greedy=g,
                            want_diag=want_diag)
        out[t0:t1] = r["tokens"]
        num[b] = r["n"]
        margin[b] = r["margin"]
        if want_diag:
            diag["lse_target"][t0:t1] = r["lse_p"]
            diag["lse_draft"][d0:d1] = r["lse_q"]
            diag["ratio"][d0:d1] = r["ratio"]
            diag["resid_Z"][b] = r["resid_Z"]
    res = dict(out_tokens=out, num_accepted=num, margin=margin)
    if want_diag:
        res.update(diag)
    return res


# --------------------------------------------------------------------------
# Acceptance statistics ([P1] s.6: a draft token x passes with probability
# min(1, p(x)/q(x)), and the acceptance rate measures how close the draft is
# to the target; [P3] section "Khi thời gian tiết kiệm bị chi phí ăn hết":
# measure the useful tokens per round and the acceptance rate; [P2]
# "工程里的关键优化点" item 3 adapts K to it). Not printed on the pages: the
# expectation below is the definition of "the probability that a draft drawn
# from q_i passes", and the expected count follows from the truncation rule
# ([P1] s.5 step 4) with the rows held fixed.
# --------------------------------------------------------------------------
def acceptance_probability(p, q):
    """beta = E_{x ~ q}[min(1, r(x))], r = p/q as in accept_ratio.

    Ids with q(x) = 0 are never drafted and carry no weight."""
    drafted = q > 0.0
    r = p[drafted] / q[drafted]
    return float(np.sum(q[drafted] * np.minimum(1.0, r)))


def acceptance_stats(draft, target, *, B, V, dtype, temperature, K=None,
                     cu_draft=None, top_k=0, top_p=1.0):
    """Acceptance probability of every draft position and the expected number
    of accepted drafts of every sequence, for sampling verification.

    Same storage layout as ``verify``; the bonus target row of each sequence is
    not used. For position i of sequence b, beta_i = acceptance_probability(p_i,
    q_i) on the filtered, tempered rows (R6), NaN if either row is unusable
    (R8). The walk stops at the first rejection, so draft j is accepted iff
    drafts 0..j all pass: with the rows fixed, E[n_b] = sum_{j<K_b}
    prod_{i<=j} beta_i (NaN if any beta of the sequence is NaN; 0 for K_b = 0).
    Returns dict(beta [sum K_b] float64, expected_accepted [B] float64,
    margin [sum K_b] float64: the nearer top-p margin of the pair's rows)."""
    if not (temperature > 0.0) or math.isinf(temperature):
        raise ValueError("acceptance statistics need a finite temperature > 0")
    if not (0.0 < top_p <= 1.0):
        raise ValueError("top_p must lie in (0, 1]")
    if cu_draft is None:
        cu = np.arange(B + 1, dtype=np.int64) * int(K)
    else:
        cu = np.asarray(cu_draft, dtype=np.int64)
    draft = np.asarray(draft).reshape(-1, V)
    target = np.asarray(target).reshape(-1, V)
    n_draft = int(cu[B])
    beta = np.full(n_draft, math.nan)
    margin = np.full(n_draft, ACCEPT_MARGIN_INF)
    expected = np.zeros(B)
    for b in range(B):
        d0, d1 = int(cu[b]), int(cu[b + 1])
        e, run = 0.0, 1.0
        for i in range(d1 - d0):
            lq = decode_logits(draft[d0 + i], dtype)
            lp = decode_logits(target[d0 + b + i], dtype)
            if row_is_valid(lq) and row_is_valid(lp):
                q, _, mq = filtered_distribution(lq, temperature, top_k, top_p)
                p, _, mp = filtered_distribution(lp, temperature, top_k, top_p)
                beta[d0 + i] = acceptance_probability(p, q)
                margin[d0 + i] = min(mq, mp)
            run *= beta[d0 + i]  # P(drafts 0..i all pass)
            e += run
        expected[b] = e
    return dict(beta=beta, expected_accepted=expected, margin=margin)


def sample_rows(rows, uniforms, *, V, dtype, temperature, top_k=0, top_p=1.0,
                greedy=None):
    """Draw one token per row by the inverse CDF of its filtered distribution.

    This is the draft model's own sampling step ([P1] s.5 step 1 and s.9, the
    multinomial draw), i.e. verification with K = 0. Used to make draft tokens
    for synthetic inputs. ``greedy`` is an optional boolean mask per row.
    Returns (tokens int32 [rows], margins float64 [rows])."""
    rows = np.asarray(rows).reshape(-1, V)
    u = np.asarray(uniforms, dtype=np.float32).reshape(-1).astype(np.float64)
    toks = np.empty(rows.shape[0], dtype=np.int32)
    margins = np.full(rows.shape[0], ACCEPT_MARGIN_INF)
    for r in range(rows.shape[0]):
        l = decode_logits(rows[r], dtype)
        if temperature == 0.0 or (greedy is not None and bool(greedy[r])):
            toks[r] = greedy_token(l)
            continue
        p, _, mp = filtered_distribution(l, temperature, top_k, top_p)
        j, _, m = inverse_cdf(p, float(u[r]))
        toks[r] = j
        margins[r] = min(mp, m)
    return toks, margins
