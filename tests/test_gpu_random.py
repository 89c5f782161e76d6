"""GPU parity on a seeded sweep of random small configurations (see
random_configs.py): verification through the dense, ragged or diag entry point
against the oracle, to the bar of test_gpu_parity.py, and the acceptance
statistics to the bar of test_gpu_accept.py."""

import sys

import numpy as np
import pytest
import torch

from parity import compare, draft_tokens_from_oracle, run_gpu, run_oracle
from random_configs import make_config  # noqa: E402
from test_gpu_accept import _compare as compare_accept, _gpu as gpu_accept, _oracle as oracle_accept

pytestmark = pytest.mark.gpu

N_CONFIGS = 40


@pytest.mark.parametrize("i", range(N_CONFIGS))
def test_random_config(i):
    w = make_config(i)
    dense = not w["ragged"] and not w["greedy"].any()
    diag = i % 2 == 1
    api = "dense" if (dense and not diag) else "ragged"
    print(f"[gpu] random {i}: {w['dtype']} B={w['B']} V={w['V']} K={w['K']} Ks={list(w['Ks'])} "
          f"T={w['temperature']} k={w['top_k']} p={w['top_p']} greedy={int(w['greedy'].sum())} "
          f"api={api} diag={diag}", flush=True)
    sys.stdout.flush()
    toks = draft_tokens_from_oracle(w)
    ora = run_oracle(w, toks, want_diag=diag)
    gpu = run_gpu(w, toks, api=api, diag=diag)
    rep = compare(w, toks, gpu, ora, check_diag=diag)
    assert not rep["mismatches"], rep["mismatches"][:3]
    if w["temperature"] > 0.0:
        beta, exp = gpu_accept(w, "dense" if not w["ragged"] else "ragged")
        compare_accept(w, beta, exp, oracle_accept(w))
