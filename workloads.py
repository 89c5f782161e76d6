"""Seeded synthetic workloads for speculative-decoding verification.

This module only draws random numbers and casts them: it holds none of the
verification arithmetic (no softmax, no ratio, no sampling). It is the single
piece shared by the oracle-side tests and the GPU side. Draft tokens, which the
draft model would sample from its own distribution, are made by a sampler the
caller passes in (the oracle's in tests, the library's K = 0 call in the bench),
from the uniform stream ``u_draft`` drawn here.

Shapes follow the workloads the pages discuss: LLM-sized vocabularies, K of 2 to
16 drafts per round (lecture-16 notes, "动态调整 K": 8/16 for a good drafter,
2/4 for a poor one), draft rows close to the target rows so that most drafts are
accepted, and a bonus row per sequence.

Recipe (numpy PCG64, fixed draw order; all arithmetic in float32):
  1. ragged workloads first draw K_b for every sequence from ``k_choices``;
  2. per sequence, base rows G ~ N(0, sd^2) of shape [K_b + 1, V];
  3. per row, ``peaks`` distinct ids (rng.choice without replacement) get +boost;
  4. noise E ~ N(0, 1) of the same shape; target = G + sd_t * E; draft = G[:K_b]
     (row K_b of G is a phantom draft row that only shapes the bonus target row);
  5. both are cast to the storage dtype with round-to-nearest-even (torch CPU);
  6. u_draft ~ U[0,1) float32 from stream [seed, 1], one per draft row;
     uniforms ~ U[0,1) float32 from stream [seed, 2], one per target row.
Steps 2-4 use stream [seed, 0]; the target-noise scale is applied after the draw,
so a sweep over sd_t at one seed shares its base rows and noise.
"""

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# The five workloads, named by what they are.
WORKLOADS = {
    "tiny_f32_B4_K4_V1024": dict(
        dtype="f32", B=4, K=4, V=1024, temperature=1.0, sd=2.0, peaks=0,
        boost=0.0, sd_t=0.5, top_k=0, top_p=1.0, seed=1000),
    "bf16_B32_K4_V32000": dict(
        dtype="bf16", B=32, K=4, V=32000, temperature=1.0, sd=3.0, peaks=20,
        boost=8.0, sd_t=1.0, top_k=0, top_p=1.0, seed=1001),
    "bf16_B64_K8_V128256": dict(
        dtype="bf16", B=64, K=8, V=128256, temperature=0.7, sd=3.0, peaks=20,
        boost=8.0, sd_t=1.0, top_k=0, top_p=1.0, seed=1002,
        sd_t_sweep=(0.25, 1.0, 4.0)),
    "f16_B256_K4_V151936_topk50_topp0.9": dict(
        dtype="f16", B=256, K=4, V=151936, temperature=0.8, sd=3.0, peaks=50,
        boost=6.0, sd_t=1.5, top_k=50, top_p=0.9, seed=1003),
    "bf16_B512_Kragged_V128256_halfgreedy": dict(
        dtype="bf16", B=512, K=None, k_choices=(2, 4, 8, 16), V=128256,
        temperature=1.0, sd=3.0, peaks=20, boost=8.0, sd_t=1.0, top_k=0,
        top_p=1.0, seed=1004, greedy="odd"),
}
HEADLINE = "bf16_B64_K8_V128256"
TINY = "tiny_f32_B4_K4_V1024"


def _cast(a32, dtype):
    return torch.from_numpy(a32).to(DTYPES[dtype])


def make(name=None, *, cfg=None, seed=None, sd_t=None, B=None, V=None, K=None,
         k_choices=None, ks=None, dtype=None, temperature=None):
    """Build a workload without draft tokens.

    Returns a dict with torch CPU tensors ``draft`` [sum K_b, V] and ``target``
    [sum (K_b + 1), V] in the storage dtype, int32 ``cu_draft`` [B + 1], bool
    ``greedy`` [B], float32 ``u_draft`` [sum K_b] and ``uniforms``
    [sum (K_b + 1)], plus the scalar settings. Overrides shrink a workload for
    quick tests while keeping its value distribution.
    """
    c = dict(WORKLOADS[name] if cfg is None else cfg)
    if seed is not None:
        c["seed"] = seed
    if sd_t is not None:
        c["sd_t"] = sd_t
    if B is not None:
        c["B"] = B
    if V is not None:
        c["V"] = V
    if K is not None:
        c["K"] = K
    if k_choices is not None:
        c["k_choices"] = tuple(k_choices)
        c["K"] = None
    if dtype is not None:
        c["dtype"] = dtype
    if temperature is not None:
        c["temperature"] = temperature
    if ks is not None:
        c["K"] = None
        c["B"] = len(ks)
    Bn, Vn = int(c["B"]), int(c["V"])
    rng = np.random.default_rng([c["seed"], 0])
    if ks is not None:
        Ks = np.asarray(ks, dtype=np.int64)
    elif c.get("K") is None:
        Ks = rng.choice(np.asarray(c["k_choices"], dtype=np.int64), Bn)
    else:
        Ks = np.full(Bn, int(c["K"]), dtype=np.int64)
    cu = np.zeros(Bn + 1, dtype=np.int64)
    cu[1:] = np.cumsum(Ks)
    n_draft, n_target = int(cu[-1]), int(cu[-1]) + Bn
    draft = torch.empty((n_draft, Vn), dtype=DTYPES[c["dtype"]])
    target = torch.empty((n_target, Vn), dtype=DTYPES[c["dtype"]])
    sd, sd_t = np.float32(c["sd"]), np.float32(c["sd_t"])
    boost = np.float32(c["boost"])
    for b in range(Bn):
        kb = int(Ks[b])
        g = rng.standard_normal((kb + 1, Vn), dtype=np.float32) * sd
        for r in range(kb + 1):
            if c["peaks"] > 0:
                ids = rng.choice(Vn, int(c["peaks"]), replace=False)
                g[r, ids] += boost
        e = rng.standard_normal((kb + 1, Vn), dtype=np.float32)
        t = g + sd_t * e
        d0 = int(cu[b])
        draft[d0:d0 + kb] = _cast(np.ascontiguousarray(g[:kb]), c["dtype"])
        target[d0 + b:d0 + b + kb + 1] = _cast(t, c["dtype"])
    greedy = np.zeros(Bn, dtype=bool)
    if c.get("greedy") == "odd":
        greedy[1::2] = True
    u_draft = np.random.default_rng([c["seed"], 1]).random(n_draft, dtype=np.float32)
    uniforms = np.random.default_rng([c["seed"], 2]).random(n_target, dtype=np.float32)
    return dict(
        name=name, dtype=c["dtype"], B=Bn, V=Vn,
        K=None if c.get("K") is None else int(c["K"]),
        ragged=c.get("K") is None,
        temperature=float(c["temperature"]), top_k=int(c["top_k"]),
        top_p=float(c["top_p"]), sd_t=float(c["sd_t"]), seed=int(c["seed"]),
        draft=draft, target=target, cu_draft=cu.astype(np.int32), Ks=Ks,
        greedy=greedy, u_draft=u_draft, uniforms=uniforms)


def draft_row_greedy_mask(w):
    """Per draft row: True where the owning sequence is greedy."""
    return np.repeat(w["greedy"], w["Ks"])


def raw_numpy(t):
    """Storage bits of a CPU tensor as numpy (bf16 -> uint16 bit patterns)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def compulsory_bytes(w):
    """Bytes a verification call must move at least once.

    Every logit of a sampling sequence's K_b draft rows and K_b + 1 target rows,
    only the target rows of a greedy sequence, plus draft ids, uniforms and the
    outputs."""
    esize = torch.tensor([], dtype=DTYPES[w["dtype"]]).element_size()
    Ks = np.asarray(w["Ks"])
    if w["temperature"] == 0.0:
        rows = int((Ks + 1).sum())
    else:
        g = np.asarray(w["greedy"], dtype=bool)
        rows = int(((Ks + 1) + np.where(g, 0, Ks)).sum())
    small = 4 * int(Ks.sum()) + 4 * int((Ks + 1).sum()) * 2 + 4 * w["B"]
    return rows * w["V"] * esize + small


# ---------------------------------------------------------------------------
# LM-head workloads: hidden states and LM-head weights instead of logit rows.
# A draft model with hidden size d_draft and a target with d_target share one
# vocabulary (a 1B-class drafter for an 8B-class target at V = 128256).
LMHEAD = dict(B=64, K=8, V=128256, d_draft=2048, d_target=4096, temperature=0.7, seed=2001)
LMHEAD_NAME = "lmhead_bf16_B64_K8_V128256_Dq2048_Dp4096"
LM_H_SCALE = 1.0 / 8.0    # hidden value = integer in [-8, 8] / 8
LM_W_SCALE = 1.0 / 512.0  # weight value = integer in [-64, 64] / 512


def make_lmhead(B=None, K=None, V=None, d_draft=None, d_target=None, temperature=None,
                seed=None):
    """Integer-valued LM-head inputs (numpy int8, times LM_H_SCALE or LM_W_SCALE).

    Hidden entries are uniform integers in [-8, 8], weight entries uniform in
    [-64, 64]: bf16 holds every value, and every product and partial sum of a
    logit (|sum| <= d * 8 * 64 < 2^24 for d < 32768) is exact in fp32, so the
    GPU's fp32 accumulation and the float64 oracle agree exactly. The target
    shares the draft's directions: for position i < K its first d_draft hidden
    entries repeat the draft's hidden state of that position and its weight's
    first d_draft columns are the draft weight; the remaining weight columns
    are drawn fresh, the remaining hidden entries fresh in [-2, 2], and the
    bonus position's hidden state fresh in [-8, 8]. Target logits are then the
    draft logits plus an independent term of about a quarter of their spread.
    Draw order (PCG64 stream [seed, 0]): draft hidden, draft weight, target
    weight tail, target hidden (fresh parts, row by row); u_draft from stream
    [seed, 1] and uniforms from [seed, 2] as in ``make``.
    """
    c = dict(LMHEAD)
    for k, v in dict(B=B, K=K, V=V, d_draft=d_draft, d_target=d_target,
                     temperature=temperature, seed=seed).items():
        if v is not None:
            c[k] = v
    Bn, Kn, Vn, dq, dp = c["B"], c["K"], c["V"], c["d_draft"], c["d_target"]
    if dp < dq:
        raise ValueError("the target's hidden size must be at least the draft's")
    rng = np.random.default_rng([c["seed"], 0])
    hq = rng.integers(-8, 9, size=(Bn * Kn, dq), dtype=np.int8)
    wq = rng.integers(-64, 65, size=(Vn, dq), dtype=np.int8)
    wp = np.empty((Vn, dp), dtype=np.int8)
    wp[:, :dq] = wq
    if dp > dq:
        wp[:, dq:] = rng.integers(-64, 65, size=(Vn, dp - dq), dtype=np.int8)
    hp = np.empty((Bn * (Kn + 1), dp), dtype=np.int8)
    for b in range(Bn):
        for i in range(Kn + 1):
            t = b * (Kn + 1) + i
            if i < Kn:
                hp[t, :dq] = hq[b * Kn + i]
                if dp > dq:
                    hp[t, dq:] = rng.integers(-2, 3, size=dp - dq, dtype=np.int8)
            else:
                hp[t] = rng.integers(-8, 9, size=dp, dtype=np.int8)
    u_draft = np.random.default_rng([c["seed"], 1]).random(Bn * Kn, dtype=np.float32)
    uniforms = np.random.default_rng([c["seed"], 2]).random(Bn * (Kn + 1), dtype=np.float32)
    return dict(B=Bn, K=Kn, V=Vn, d_draft=dq, d_target=dp, temperature=float(c["temperature"]),
                seed=int(c["seed"]), hq=hq, wq=wq, hp=hp, wp=wp, u_draft=u_draft,
                uniforms=uniforms)


def lmhead_to_device(a, scale, device="cuda"):
    """An int8 array as a bf16 device tensor of a * scale (exact: |a| <= 127,
    scale a power of two)."""
    t = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return t.to(torch.bfloat16) * scale


LMHEAD_REAL_NAME = "lmhead_real_bf16_B64_K8_V128256_Dq2048_Dp4096"


def make_lmhead_real(B=None, K=None, V=None, d_draft=None, d_target=None, temperature=None,
                     seed=None, sd=3.0, peaks=20, boost=8.0, sd_t=1.0):
    """General bf16 LM-head inputs (no integer grid): every value is a bf16
    number, returned as float32 arrays holding exactly those values.

    The logits follow the logit workloads' shape. The draft weight is W_q ~
    N(0, sd^2 / d_draft) per entry, and each draft hidden row is N(0, 1) plus,
    for `peaks` distinct ids k of that row, (boost / |W_q[k]|^2) W_q[k]. So
    logits have spread about sd, and those ids sit about `boost` higher. The
    target shares the draft's directions: its weight is [W_q | W_e] with
    W_e ~ N(0, sd_t^2 / (d_target - d_draft)), and its hidden row at position
    i < K is [the draft's row i | e] with e ~ N(0, 1), so its logits are the
    draft's plus about N(0, sd_t^2). Its bonus row is a fresh draft-like row
    followed by e. Hidden rows and weights are then cast to bf16
    (round-to-nearest-even, torch CPU).
    Draw order (PCG64 stream [seed, 0]): W_q, W_e, then per sequence and
    position the hidden row, its peak ids and e; u_draft from [seed, 1] and
    uniforms from [seed, 2] as in ``make``.
    """
    c = dict(LMHEAD)
    for k, v in dict(B=B, K=K, V=V, d_draft=d_draft, d_target=d_target,
                     temperature=temperature, seed=seed).items():
        if v is not None:
            c[k] = v
    Bn, Kn, Vn, dq, dp = c["B"], c["K"], c["V"], c["d_draft"], c["d_target"]
    if dp < dq:
        raise ValueError("the target's hidden size must be at least the draft's")
    rng = np.random.default_rng([c["seed"], 1000])
    wq = (rng.standard_normal((Vn, dq), dtype=np.float32) * np.float32(sd / np.sqrt(dq)))
    de = dp - dq
    we = (rng.standard_normal((Vn, de), dtype=np.float32) * np.float32(sd_t / np.sqrt(de))
          if de > 0 else np.zeros((Vn, 0), np.float32))
    wq = _bf16(wq)
    we = _bf16(we)
    norm2 = np.einsum("vd,vd->v", wq.astype(np.float64), wq.astype(np.float64))

    def draft_like():
        h = rng.standard_normal(dq, dtype=np.float32).astype(np.float64)
        if peaks > 0:
            ids = rng.choice(Vn, int(peaks), replace=False)
            h += (boost / norm2[ids]) @ wq[ids].astype(np.float64)
        return h.astype(np.float32)

    hq = np.empty((Bn * Kn, dq), dtype=np.float32)
    hp = np.empty((Bn * (Kn + 1), dp), dtype=np.float32)
    for b in range(Bn):
        for i in range(Kn + 1):
            h = draft_like()
            e = rng.standard_normal(de, dtype=np.float32)
            if i < Kn:
                hq[b * Kn + i] = h
            hp[b * (Kn + 1) + i, :dq] = h
            hp[b * (Kn + 1) + i, dq:] = e
    # rounding is elementwise, so the target's copy of each draft row rounds alike
    hq, hp = _bf16(hq), _bf16(hp)
    wp = np.concatenate([wq, we], axis=1)
    u_draft = np.random.default_rng([c["seed"], 1]).random(Bn * Kn, dtype=np.float32)
    uniforms = np.random.default_rng([c["seed"], 2]).random(Bn * (Kn + 1), dtype=np.float32)
    return dict(B=Bn, K=Kn, V=Vn, d_draft=dq, d_target=dp, temperature=float(c["temperature"]),
                seed=int(c["seed"]), hq=hq, wq=wq, hp=hp, wp=wp, u_draft=u_draft,
                uniforms=uniforms)


def _bf16(a):
    """float32 array rounded to bf16 (round-to-nearest-even), as float32."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(
        torch.bfloat16).to(torch.float32).numpy()


# ---------------------------------------------------------------------------
# Several draft chains per sequence (M drafters, each proposing K tokens).
def make_multi(B=16, M=3, K=4, V=32000, dtype="bf16", temperature=1.0, seed=3001, sd=3.0,
               peaks=20, boost=8.0, sd_t=1.0):
    """Rows of M draft chains per sequence, without draft tokens.

    Target rows follow the logit workloads' recipe, N(0, sd^2) with `peaks`
    ids raised by `boost`, one fresh row per (sequence, chain, position); the
    rows of position 0 are the chain-0 row for every chain (one shared
    prefix). A chain's draft row is its target row plus N(0, sd_t^2) noise of
    its own (a different drafter per chain). Draft tokens come from a sampler
    the caller passes in, position by position. share_target_prefixes then
    makes the target rows of chains with equal prefixes agree. Draw order
    (PCG64 stream [seed, 0]) per sequence, chain, position: the target row,
    its peak ids, the draft noise. u_draft [B, M, K] comes from [seed, 1],
    uniforms [B, K+1, M+1] from [seed, 2]. Rows are cast to `dtype`
    (round-to-nearest-even, torch CPU)."""
    rng = np.random.default_rng([seed, 0])
    tgt = np.empty((B, M, K + 1, V), np.float32)
    dft = np.empty((B, M, K, V), np.float32)
    for b in range(B):
        for m in range(M):
            for j in range(K + 1):
                g = rng.standard_normal(V, dtype=np.float32) * np.float32(sd)
                if peaks > 0:
                    g[rng.choice(V, int(peaks), replace=False)] += np.float32(boost)
                tgt[b, m, j] = g if (j > 0 or m == 0) else tgt[b, 0, 0]
                if j < K:
                    dft[b, m, j] = tgt[b, m, j] + (rng.standard_normal(V, dtype=np.float32)
                                                   * np.float32(sd_t))
    u_draft = np.random.default_rng([seed, 1]).random((B, M, K), dtype=np.float32)
    uniforms = np.random.default_rng([seed, 2]).random((B, K + 1, M + 1), dtype=np.float32)
    return dict(B=B, M=M, K=K, V=V, dtype=dtype, temperature=float(temperature),
                draft=_cast(dft.reshape(B * M * K, V), dtype).reshape(B, M, K, V),
                target=_cast(tgt.reshape(B * M * (K + 1), V), dtype).reshape(B, M, K + 1, V),
                u_draft=u_draft, uniforms=uniforms)


def share_target_prefixes(target, tokens):
    """Copy, for every position j >= 1, the target row of the lowest chain
    with a given prefix (tokens 0..j-1) to the other chains with that prefix
    (target [B, M, K+1, V] torch tensor, tokens [B, M, K] ints; in place)."""
    B, M, K1 = target.shape[:3]
    tok = np.asarray(tokens).reshape(B, M, K1 - 1)
    for b in range(B):
        for j in range(1, K1):
            first = {}
            for m in range(M):
                key = tuple(int(t) for t in tok[b, m, :j])
                if key in first:
                    target[b, m, j] = target[b, first[key], j]
                else:
                    first[key] = m
    return target
