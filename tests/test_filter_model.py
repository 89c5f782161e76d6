"""The top-k filter's usual path, modelled on the CPU (tests/filter_model.py),
against the oracle's top-k / top-p rule on full-size rows (-m "not gpu").

Rows follow the filtered workload's recipe (fp16, V = 151936, N(0, 3^2) logits
with 50 peaks at +6) and the sampling workloads' bf16 recipe at V = 128256.
Every row must take the usual path (the chunk records, the row bound and the
one-level histogram cover it), and the kept set l >= theta must equal the
oracle's, with the kept-set sum to 1e-5. Rows whose top-p decision lies within
1e-6 of top_p are excluded and counted. A planted mistake in the top-p walk
(the mass up to and including a level instead of the strictly larger one) must
change some row's kept set.

Page: aihero.vn "Speculative decoding", section "Cùng phân bố không có nghĩa
cùng chuỗi mỗi lần" (the same temperature, top-k and top-p on both models'
rows).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from filter_model import filter_row


def _rows(name, dtype, shift=0.0):
    """Full-size rows of a workload; ``shift`` moves every logit (rounded back
    to the storage type), so that the candidates can be negative values."""
    w = W.make(name, B=2)
    rows = np.concatenate([oracle.decode_logits(W.raw_numpy(w["draft"]), dtype),
                           oracle.decode_logits(W.raw_numpy(w["target"]), dtype)])
    if shift:
        t = torch.from_numpy(rows.astype(np.float32) + np.float32(shift))
        rows = t.to(torch.bfloat16 if dtype == "bf16" else torch.float16).to(torch.float64).numpy()
    return rows, w["temperature"]


CASES = [("f16_B256_K4_V151936_topk50_topp0.9", "f16", 50, 0.9, 0.0),
         ("f16_B256_K4_V151936_topk50_topp0.9", "f16", 5, 1.0, 0.0),
         ("f16_B256_K4_V151936_topk50_topp0.9", "f16", 200, 0.95, 0.0),
         ("f16_B256_K4_V151936_topk50_topp0.9", "f16", 50, 0.9, -60.0),
         (W.HEADLINE, "bf16", 50, 0.9, 0.0),
         (W.HEADLINE, "bf16", 1, 1.0, 0.0),
         (W.HEADLINE, "bf16", 50, 0.9, -60.0)]


@pytest.mark.parametrize("name,dtype,top_k,top_p,shift", CASES)
def test_usual_path_matches_oracle(name, dtype, top_k, top_p, shift):
    """shift -60 makes every candidate negative: a negative level's key has its
    low bits set, which the bins and the level values must respect."""
    rows, T = _rows(name, dtype, shift)
    checked = near = 0
    for r in rows:
        prob, lse, margin = oracle.filtered_distribution(r, T, top_k, top_p)
        res = filter_row(r.astype(np.float32), T, top_k, top_p, dtype)
        assert res is not None, "the row left the usual path"
        if margin <= 1e-6:
            near += 1
            continue
        theta, kept = res
        np.testing.assert_array_equal(r >= theta, prob > 0.0)
        # kept sum in units of 2^R: sum of 2^(l*c - R) over the kept set
        c = np.float32(1.4426950408889634 / T)
        R = np.float32(np.float32(r.max()) * c)
        np.testing.assert_allclose(kept * 2.0 ** float(R), np.exp(lse), rtol=1e-5)
        checked += 1
    print(f"{dtype} k={top_k} p={top_p} shift={shift}: checked={checked} near={near}")
    assert checked >= len(rows) - 2


def test_inclusive_mass_walk_would_keep_too_few():
    rows, T = _rows("f16_B256_K4_V151936_topk50_topp0.9", "f16")
    wrong = 0
    for r in rows:
        prob, _, margin = oracle.filtered_distribution(r, T, 50, 0.9)
        if margin <= 1e-6:
            continue
        theta, _ = filter_row(r.astype(np.float32), T, 50, 0.9, "f16", strict_above=False)
        wrong += not np.array_equal(r >= theta, prob > 0.0)
    assert wrong > 0
