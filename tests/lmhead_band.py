"""Near-threshold band of the LM-head path on general bf16 operands.

The library forms each logit l = sum_k h_k w_k on the matrix cores. The
products of bf16 values are exact in fp32. Each matrix-core step adds a
16-term block into an fp32 accumulator: D/16 accumulator roundings, plus at
most 15 inside a block. Each rounding is at most 2^-24 of a partial sum whose
magnitude is at most S = sum_k |h_k w_k|. Counting each as 2 units to allow
any rounding mode, the blocked-summation bound is

    |l_gpu - l| <= eps = 2 * 2^-24 * (D/16 + 16) * S.

For a row, E is the largest eps over its ids. The decisions move by at most:
  - the ratio test: r = p(x)/q(x) = e^{(l_p(x) - l_q(x))/T} S_q/S_p, and each
    normaliser moves by at most e^{E/T}, so r moves by a factor within
    e^{+-2(E_p + E_q)/T}. A test can flip only if |u - r| <= r (e^{2(E_p + E_q)/T} - 1);
  - the inverse CDF: each probability moves by a factor within e^{+-2E/T}
    (rho = e^{2E/T} - 1 relative). The residual weights max(0, p - q) then move
    by at most rho_p p + rho_q q, so every cumulative sum and the mass Z move by at
    most delta = rho_p + rho_q, and C_j/Z by at most 2 delta / (Z - delta). The
    bonus draw from p moves by at most 2 rho_p.
A sequence is compared bit for bit when the oracle's margin (the distance of
every used uniform from its threshold) exceeds 1e-5 (the logit path's band
for the fp32 verification arithmetic) plus the largest of these bounds over
its decisions.
"""

import math

import numpy as np

UNIT = 2.0 ** -24
BAND = 1e-5


def row_error_bounds(hidden, weight):
    """eps bound of every logit of every row, reduced to its largest per row.
    Computed in float32; the small excess of that sum is covered by 1.001."""
    d = hidden.shape[1]
    a = np.abs(np.asarray(hidden, np.float32)) @ np.abs(np.asarray(weight, np.float32)).T
    return 1.001 * 2.0 * UNIT * (d / 16.0 + 16.0) * a.max(axis=1).astype(np.float64)


def logit_error_bounds(hidden, weight):
    """eps bound of every logit (rows x ids), float64."""
    d = hidden.shape[1]
    a = np.abs(np.asarray(hidden, np.float64)) @ np.abs(np.asarray(weight, np.float64)).T
    return 2.0 * UNIT * (d / 16.0 + 16.0) * a


def sequence_bands(ora, E_draft, E_target, B, K, T):
    """Band of every sequence from the oracle's diagnostics (its ratios and
    final-draw mass Z, ``verify(..., want_diag=True)``) and the per-row bounds."""
    bands = np.full(B, BAND)
    for b in range(B):
        n = int(ora["num_accepted"][b])
        if n < 0:
            continue  # an error code: no sampled decision
        errs = []
        for i in range(min(n + 1, K)):
            r = float(ora["ratio"][b * K + i])
            if not math.isfinite(r):
                continue  # q(x) = 0 accepts whatever the rounding
            e = E_target[b * (K + 1) + i] + E_draft[b * K + i]
            errs.append(r * math.expm1(2.0 * e / T))
        rho_p = math.expm1(2.0 * E_target[b * (K + 1) + n] / T)
        if n < K:
            delta = rho_p + math.expm1(2.0 * E_draft[b * K + n] / T)
            z = float(ora["resid_Z"][b])
            errs.append(2.0 * delta / (z - delta) if z > delta else math.inf)
        else:
            errs.append(2.0 * rho_p)
        bands[b] = BAND + max(errs)
    return bands
