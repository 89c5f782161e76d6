"""The top-p-alone threshold search, modelled on the CPU (tests/nucleus_model.py),
against the oracle's top-p rule on full-size rows (-m "not gpu").

Rows follow the sampling workloads' recipe (N(0, 3^2) logits with 20 peaks at
+8, V = 128256) in each storage type. At top_p 0.99 and 0.995 the last kept
level of many rows lies below the first pass's top window (masses from 2^-16 of
the maximum's), where the search bins the keys below the window and then splits
a bin; the test requires such rows to be present, so the range each pass covers
is exercised. Rows whose top-p decision lies within 1e-6 of top_p (the
fixed-point masses carry up to ~1e-7 of relative error) are excluded and
counted.

Page: aihero.vn "Speculative decoding", section "Cùng phân bố không có nghĩa
cùng chuỗi mỗi lần" (the same top-p on both models' rows).
"""

import numpy as np
import pytest

import oracle
import workloads as W
from nucleus_model import nucleus_threshold


def _oracle_keep(l, temperature, top_p):
    prob, _, margin = oracle.filtered_distribution(l, temperature, 0, top_p)
    return prob > 0.0, margin


CASES = [(dt, 1.0, 0.99) for dt in ("bf16", "f16")] + \
        [(dt, 0.7, 0.995) for dt in ("bf16", "f16")] + \
        [(dt, 0.7, 0.9) for dt in ("bf16", "f16", "f32")] + [("f32", 1.0, 0.95)]


@pytest.mark.parametrize("dtype,temperature,top_p", CASES)
def test_search_matches_oracle_top_p(dtype, temperature, top_p):
    """fp32 rows take their own settings: every fp32 value is its own level, so
    near top_p 0.99 most rows have a level within 1e-6 of the cut."""
    w = W.make("bf16_B32_K4_V32000", B=3, V=128256, dtype=dtype)
    rows = np.concatenate([oracle.decode_logits(W.raw_numpy(w["draft"]), dtype),
                           oracle.decode_logits(W.raw_numpy(w["target"]), dtype)])
    checked = below = split = near = 0
    for r in rows:
        keep, margin = _oracle_keep(r, temperature, top_p)
        if margin <= 1e-6:
            near += 1
            continue
        info = {}
        theta, kept_sum = nucleus_threshold(r.astype(np.float32), temperature, top_p, dtype,
                                            info=info)
        np.testing.assert_array_equal(r >= theta, keep)
        checked += 1
        below += info["below_window"]
        split += info["passes"] > (2 if info["below_window"] else 1)
    print(f"{dtype} T={temperature} p={top_p}: checked={checked} near={near} "
          f"below-window={below} split-passes={split}")
    assert checked >= len(rows) // 2
    if top_p >= 0.99 and dtype != "f32":
        assert below > 0 and split > 0  # the passes below the window ran


def test_unclamped_split_would_count_the_window_twice():
    """The same search with a split bin allowed to run past its pass's key
    range (back into the window, whose mass is already counted) keeps too few
    ids on some of these rows: the test above would catch that mistake."""
    w = W.make("bf16_B32_K4_V32000", B=3, V=128256)
    rows = oracle.decode_logits(W.raw_numpy(w["target"]), "bf16")
    wrong = 0
    for r in rows:
        keep, margin = _oracle_keep(r, 1.0, 0.99)
        if margin <= 1e-6:
            continue
        theta, _ = nucleus_threshold(r.astype(np.float32), 1.0, 0.99, "bf16", clamp_top=False)
        wrong += not np.array_equal(r >= theta, keep)
    assert wrong > 0
