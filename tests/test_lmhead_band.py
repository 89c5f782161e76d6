"""Pins of the LM-head near-threshold band (tests/lmhead_band.py), no GPU.

1. The logit bound: fp32 accumulation of bf16 products in 16-term blocks, with
   one rounding per block and with a rounding after every add inside a block,
   stays within eps = 2 * 2^-24 * (D/16 + 16) * sum|h w| on general bf16
   operands at the hidden sizes of the LM-head workload.
2. The propagation to decisions: the oracle's verification on logits moved by
   up to eps (adversarial signs: the draft ids and the rest moved apart)
   never changes a sequence whose margin exceeds its band; with the band
   built from a tenth of eps, some sequence outside that smaller band does
   change, so the check has power.
"""

import numpy as np
import pytest

import oracle
import workloads as W
from lmhead_band import BAND, logit_error_bounds, sequence_bands


def _blocked_fp32(h, w, block_rounding):
    """fp32 dot products in 16-term blocks: block sums exact (rounded once) or
    rounded after every add, then added into an fp32 accumulator."""
    d = h.shape[1]
    acc = np.zeros((h.shape[0], w.shape[0]), np.float32)
    for k0 in range(0, d, 16):
        hb = h[:, k0:k0 + 16].astype(np.float64)
        wb = w[:, k0:k0 + 16].astype(np.float64)
        if block_rounding == "once":
            blk = (hb @ wb.T).astype(np.float32)
        else:
            blk = np.zeros_like(acc)
            for k in range(hb.shape[1]):
                # a bf16 x bf16 product is exact in fp32
                blk = (blk + np.outer(hb[:, k], wb[:, k]).astype(np.float32)).astype(np.float32)
        acc = (acc + blk).astype(np.float32)
    return acc


@pytest.mark.parametrize("d", [64, 2048, 4096])
@pytest.mark.parametrize("mode", ["once", "every-add"])
def test_blocked_fp32_accumulation_within_bound(d, mode):
    w = W.make_lmhead_real(B=4, K=2, V=96, d_draft=min(d, 2048), d_target=d, seed=60 + d)
    h, wt = w["hp"], w["wp"]
    exact = h.astype(np.float64) @ wt.astype(np.float64).T
    got = _blocked_fp32(h, wt, mode).astype(np.float64)
    bound = logit_error_bounds(h, wt)
    err = np.abs(got - exact)
    assert np.all(err <= bound), (err.max(), bound.min())
    print(f"d={d} {mode}: max error {err.max():.2e}, max error/bound {np.max(err / bound):.3f}")


def _perturbed(lq, lp, toks, K, eps, sign):
    """Logits moved by +-eps: the draft rows' logit at each draft id one way and
    every other logit the other way (the target rows the opposite way)."""
    dq = np.full_like(lq, -sign * eps)
    dp = np.full_like(lp, sign * eps)
    B = lp.shape[0] // (K + 1)
    for b in range(B):
        for i in range(K):
            x = int(toks[b * K + i])
            dq[b * K + i, x] = sign * eps
            dp[b * (K + 1) + i, x] = -sign * eps
    return lq + dq, lp + dp


@pytest.mark.parametrize("seed", [0, 1])
def test_band_covers_moved_logits(seed):
    B, K, V, T, eps = 128, 4, 600, 0.7, 3e-3
    w = W.make_lmhead_real(B=B, K=K, V=V, d_draft=64, d_target=128, temperature=T,
                           seed=300 + seed)
    lq = w["hq"].astype(np.float64) @ w["wq"].astype(np.float64).T
    lp = w["hp"].astype(np.float64) @ w["wp"].astype(np.float64).T
    toks, _ = oracle.sample_rows(lq, w["u_draft"], V=V, dtype="f64", temperature=T)
    ora = oracle.verify(lq, lp, toks, w["uniforms"], B=B, V=V, K=K, dtype="f64", temperature=T,
                        want_diag=True)
    E_d, E_t = np.full(B * K, eps), np.full(B * (K + 1), eps)
    bands = sequence_bands(ora, E_d, E_t, B, K, T)
    small = sequence_bands(ora, E_d / 10, E_t / 10, B, K, T)
    changed_outside_small = 0
    for sign in (1.0, -1.0):
        mq, mp = _perturbed(lq, lp, toks, K, eps, sign)
        got = oracle.verify(mq, mp, toks, w["uniforms"], B=B, V=V, K=K, dtype="f64",
                            temperature=T)
        for b in range(B):
            sl = slice(b * (K + 1), (b + 1) * (K + 1))
            same = (got["num_accepted"][b] == ora["num_accepted"][b]
                    and np.array_equal(got["out_tokens"][sl], ora["out_tokens"][sl]))
            if ora["margin"][b] > bands[b]:
                assert same, (b, ora["margin"][b], bands[b])
            elif ora["margin"][b] > small[b] and not same:
                changed_outside_small += 1
    near = int((ora["margin"] <= bands).sum())
    print(f"seed {seed}: {near} of {B} sequences inside the band, "
          f"{changed_outside_small} changed outside the tenth-size band")
    assert changed_outside_small > 0
    assert near < B  # the band leaves most sequences to the bit-exact check


def test_band_is_the_logit_band_without_rounding():
    """With no logit error the band is the logit path's 1e-5."""
    B, K = 3, 2
    ora = dict(num_accepted=np.array([0, 2, 1]), ratio=np.array([0.5, 1.2, 2.0, 0.9, 0.8, 0.3]),
               resid_Z=np.array([0.2, np.nan, 0.4]))
    bands = sequence_bands(ora, np.zeros(B * K), np.zeros(B * (K + 1)), B, K, 0.7)
    assert np.allclose(bands, BAND)
