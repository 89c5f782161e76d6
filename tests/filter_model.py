"""A CPU model of the top-k filter's usual path, restated in numpy.

This is not the oracle: it models what the library computes per filtered row,
so that the design itself can be checked on the CPU against the oracle's
top-k / top-p rule on full-size rows:
- the statistics pass's chunk records: a chunk of 2048 16-byte vectors is held
  by 256 threads, thread t holding vectors t + 256*u (u < 8); its bound is the
  largest group maximum that at least k group maxima reach (groups of 4, 2 or
  1 threads, the largest size leaving at least k groups), and its record holds
  every logit at or above the bound;
- the filter's row bound, the largest chunk bound: the row's k-th largest
  logit is never below it, so the candidates at or above it decide the row;
- the histogram of those candidates over 2048 bins of one level each, from the
  bound's level up (a widened bf16 / fp16 logit's low 16 / 13 key bits are
  constant, so a bin is one value and its count that value's multiplicity);
- tau's bin, where the count from the top reaches k, and the walk down the
  bins with masses count * 2^(l*c - R), keeping a level while the mass of the
  strictly larger levels over the top-k mass is below top_p.

Rows that the model cannot take (a chunk with more candidates than its record
holds, candidates beyond 2048 levels, at most k finite logits) go to the
library's general path; the model reports them as None.

Page: aihero.vn "Speculative decoding", section "Cùng phân bố không có nghĩa
cùng chuỗi mỗi lần" (the same temperature, top-k and top-p on both rows).
"""

import numpy as np

BINS = 2048
THREADS = 256
VECS_PER_THREAD = 8
PER_VEC = 8  # 16-bit values per 16-byte vector
CHUNK = THREADS * VECS_PER_THREAD * PER_VEC
LOW_BITS = {"bf16": 16, "f16": 13}


def kcap_for(k):
    """Entries a chunk record holds for top-k = k."""
    return (k + 256 + 63) // 64 * 64


def key_of(f):
    """Order-preserving uint32 keys of float32 values (-0 and +0 share one)."""
    f = np.where(np.asarray(f, np.float32) == 0, np.float32(0), f).astype(np.float32)
    u = np.atleast_1d(f).view(np.uint32)
    return np.where(u & np.uint32(0x80000000), ~u, u | np.uint32(0x80000000)).astype(np.uint32)


def float_of_key(k):
    k = np.atleast_1d(np.asarray(k, np.uint32))
    bits = np.where(k & np.uint32(0x80000000), k & np.uint32(0x7FFFFFFF), ~k).astype(np.uint32)
    return bits.view(np.float32)


def chunk_bound(vals, k):
    """Lower bound of a chunk's k-th largest value from group maxima (-inf if none)."""
    v = np.full(CHUNK, -np.inf, np.float32)
    v[:vals.shape[0]] = vals
    # vector u of thread t covers ids (t + 256*u)*8 .. +7
    per_thread = v.reshape(VECS_PER_THREAD, THREADS, PER_VEC).max(axis=(0, 2))
    g = 4 if k <= THREADS // 4 else (2 if k <= THREADS // 2 else 1)
    gm = per_thread.reshape(THREADS // g, g).max(axis=1)
    cands = [m for m in gm if np.isfinite(m) and (gm >= m).sum() >= k]
    return np.float32(max(cands)) if cands else np.float32(-np.inf)


def filter_row(l, temperature, top_k, top_p, dtype, strict_above=True):
    """(theta, kept-set sum) of one finite row as the usual path finds them, or
    None for a row that takes the general path. ``strict_above`` False plants
    a mistake: a level is kept while the mass up to and including it is below
    top_p."""
    l = np.asarray(l, np.float32)
    low = LOW_BITS[dtype]
    kcap = kcap_for(top_k)
    bounds, cands = [], []
    for c0 in range(0, l.shape[0], CHUNK):
        ch = l[c0:c0 + CHUNK]
        b = chunk_bound(ch, top_k)
        if b == -np.inf:
            return None  # no bound: the record would need the exact path
        rec = ch[ch >= b]
        if rec.shape[0] > kcap:
            return None  # more candidates than the record holds: exact path
        bounds.append(b)
        cands.append(rec)
    if np.isfinite(l).sum() <= top_k:
        return None
    bnd = max(bounds)
    x = np.concatenate(cands)
    x = x[x >= bnd]
    kb = int(key_of(bnd)[0]) & ~((1 << low) - 1)
    bins = (key_of(x).astype(np.int64) - kb) >> low
    if bins.max() >= BINS:
        return None  # candidates beyond 2048 levels
    hist = np.bincount(bins, minlength=BINS)

    def level(b):
        key = kb + (b << low)
        if not key & 0x80000000:
            key |= (1 << low) - 1
        return float(float_of_key(np.uint32(key))[0])

    desc = np.arange(BINS - 1, -1, -1)
    btau = desc[np.searchsorted(np.cumsum(hist[desc]), top_k)]
    c = np.float32(1.4426950408889634 / temperature)
    m = np.float32(level(int(np.flatnonzero(hist)[-1])))
    R = np.float32(m * c)
    live = [int(b) for b in desc if b >= btau and hist[b]]
    e = [np.float32(hist[b]) * np.exp2(np.float32(np.float64(level(b)) * c - R), dtype=np.float32)
         for b in live]
    S_k = float(np.sum(np.float64(e)))
    above, kept, theta = 0.0, 0.0, None
    for b, eb in zip(live, e):
        test = above if strict_above else above + float(eb)
        if top_p >= 1.0 or test / S_k < top_p:
            theta, kept = level(b), above + float(eb)
        above += float(eb)
    return theta, kept
