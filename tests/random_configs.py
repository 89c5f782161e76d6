"""Seeded random small configurations for the GPU parity sweep (test helper).

Each configuration draws a dtype, a batch with dense or ragged K (zero
included), a vocabulary size (vector and scalar paths, tiny ones included),
temperature, top-k and top-p settings, a greedy mask and the generator's
value distribution. Draft tokens still come from the oracle's sampler."""

import numpy as np

import workloads as W

VOCABS = (1, 7, 64, 1000, 4099, 16384, 40000)


def make_config(i):
    rng = np.random.default_rng([4242, i])
    dtype = ["f32", "f16", "bf16"][int(rng.integers(3))]
    V = int(rng.choice(VOCABS, p=[0.05, 0.1, 0.15, 0.2, 0.2, 0.15, 0.15]))
    B = int(rng.integers(1, 9))
    ragged = bool(rng.integers(2))
    T = float(rng.choice([0.0, 0.5, 1.0, 1.7], p=[0.15, 0.3, 0.35, 0.2]))
    top_k = int(rng.choice([0, 0, 1, 5, 50, V]))
    top_p = float(rng.choice([1.0, 1.0, 0.9, 0.5]))
    peaks = int(min(V, rng.choice([0, 5])))
    cfg = dict(dtype=dtype, B=B, V=V, temperature=T, sd=float(rng.choice([1.0, 3.0])),
               peaks=peaks, boost=float(rng.choice([4.0, 8.0])),
               sd_t=float(rng.choice([0.25, 1.0, 3.0])), top_k=top_k, top_p=top_p,
               seed=10000 + i)
    if ragged:
        cfg["K"] = None
        ks = [int(k) for k in rng.integers(0, 13, B)]
        w = W.make(cfg=cfg, ks=ks)
    else:
        cfg["K"] = int(rng.integers(0, 11))
        w = W.make(cfg=cfg)
    w["name"] = f"random{i}"
    if T > 0.0 and rng.integers(3) == 0:
        w["greedy"] = rng.integers(2, size=B).astype(bool)
    return w
