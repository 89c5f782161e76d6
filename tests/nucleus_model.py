"""A CPU model of the top-p-alone threshold search the library runs per row
(the radix descent on order-preserving logit keys, with fixed-point masses).

This is not the oracle: it restates the kernel's search in numpy, so that the
search itself (the window pass, the pass below the window, the bin splits and
the range each pass covers) can be checked on the CPU against the oracle's
top-p rule on full-size rows. Rows are float32 arrays of widened logits; every
rounding step the kernel takes in fp32 is taken in fp32 here.

The rule it must reproduce (aihero.vn "Speculative decoding", section "Cùng phân
bố không có nghĩa cùng chuỗi mỗi lần": the same top-p on both rows; the reading
taken: keep id j iff the mass of strictly larger logits is below top_p) leaves
one threshold theta per row: the ids kept are those with l >= theta.
"""

import numpy as np

BINS = 2048
SCALE = np.float32(2.0 ** 40)  # fixed-point unit of a mass 2^(l*c - R)
TOP_WINDOW = 16.0  # the first pass bins the masses from 2^-16 of the maximum's up
CUTOFF = -40.0  # masses below 2^-40 are zero in the fixed point
LOW_BITS = {"bf16": 16, "f16": 13, "f32": 0}  # key bits every level shares


def key_of(f):
    """Order-preserving uint32 keys of float32 values (-0 and +0 share one)."""
    f = np.where(np.asarray(f, np.float32) == 0, np.float32(0), f).astype(np.float32)
    u = f.view(np.uint32)
    return np.where(u & np.uint32(0x80000000), ~u, u | np.uint32(0x80000000)).astype(np.uint32)


def float_of_key(k):
    k = np.asarray(k, np.uint32)
    bits = np.where(k & np.uint32(0x80000000), k & np.uint32(0x7FFFFFFF), ~k).astype(np.uint32)
    return bits.view(np.float32)


def fma32(a, b, c):
    """fp32 a*b + c with one rounding (the float32 product is exact in float64)."""
    return (np.asarray(a, np.float32).astype(np.float64) * np.float64(np.float32(b))
            + np.float64(np.float32(c))).astype(np.float32)


def _smallest_key_passing(m, c, R, cut):
    """Smallest key whose value passes fma(l, c, -R) >= cut (monotone in the key)."""
    lo = int(key_of(np.float32(-np.inf)))
    hi = int(key_of(np.float32(m)))
    while hi - lo > 1:
        mid = lo + (hi - lo) // 2
        if fma32(float_of_key(np.uint32(mid)), c, -R) >= np.float32(cut):
            hi = mid
        else:
            lo = mid
    return hi


def nucleus_threshold(l, temperature, top_p, dtype, clamp_top=True, info=None):
    """theta and the kept-set sum of one finite row, as the library's search
    finds them (theta = -inf: every id kept). ``clamp_top`` keeps each split
    bin within the key range of its pass (the search as it must be); False
    lets a split bin run past it. ``info`` (a dict) receives the passes taken
    and whether the search went below the top window."""
    l = np.asarray(l, np.float32)
    c = np.float32(1.4426950408889634 / temperature)
    m = np.float32(l.max())
    R = np.float32(m * c)
    low = LOW_BITS[dtype]
    low_mask = (1 << low) - 1
    kb_all = _smallest_key_passing(m, c, R, CUTOFF) & ~low_mask
    kb_top = _smallest_key_passing(m, c, R, -TOP_WINDOW) & ~low_mask
    x = fma32(l, c, -R)
    live = x >= np.float32(CUTOFF)
    q = (np.exp2(x[live]).astype(np.float32) * SCALE).astype(np.uint64)
    keys = key_of(l[live]).astype(np.int64)
    # the row total is the statistics pass's fp32 sum of the masses, not the
    # fixed-point one (a logit below the window only adds to that total)
    total = float(np.exp2(x).astype(np.float32).sum(dtype=np.float32))
    bound = float(np.float32(top_p)) * total * float(SCALE)
    kbase, kmax = kb_top, int(key_of(m))
    span = kmax - kbase
    above, kept, found = 0, 0, False
    lv = 0
    while True:
        s = low
        while (span >> s) >= BINS:
            s += 1
        d = keys - kbase
        inr = (d >= 0) & (d <= span)
        hist = np.zeros(BINS, dtype=np.uint64)
        np.add.at(hist, (d[inr] >> s).astype(np.int64), q[inr])
        # bins from the largest key down: the strictly-larger mass is below the
        # bound and the running mass reaches it within the bin
        h = hist[::-1].astype(object)
        acc = above
        sel = -1
        for i, hb in enumerate(h):
            if float(acc) < bound and float(acc + hb) >= bound:
                sel, sbase = BINS - 1 - i, acc
                break
            acc += hb
        if sel < 0:
            if lv == 0 and kb_top > kb_all:
                if info is not None:
                    info["below_window"] = True
                above += int(hist.sum())
                kbase, kmax = kb_all, kb_top - 1
                span = kmax - kbase
                lv += 1
                continue
            break
        found = True
        kbase += sel << s
        above = sbase
        kept = sbase + int(hist[sel])
        if s == low:
            break
        span = (1 << s) - 1
        if clamp_top:
            span = min(span, kmax - kbase)
        lv += 1
    if info is not None:
        info["passes"] = lv + 1
        info.setdefault("below_window", False)
    if not found:
        return -np.inf, None
    key = kbase | (0 if kbase & 0x80000000 else low_mask)
    return float(float_of_key(np.uint32(key))), kept / float(SCALE)
