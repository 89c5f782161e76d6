"""Float64 oracle of verification from LM-head hidden states (CPU, numpy).

TEST INFRASTRUCTURE ONLY: imported by tests/ and bench.py's cpu_baseline leg;
never by the library it checks.

A model's last layer maps its hidden state h (one per position) to one logit
per vocabulary id, l = h W^T with the LM-head weight W [V, D] ([P2] part 4,
item 1: the target model scores every drafted position in one forward pass,
and its output at each position is that position's logit row). [P1] section 8
names the memory the draft and target logit rows take up, which is why the
library forms them inside its GEMM and never stores them; the verification
step on those logits is the one ``verify`` defines, unchanged.
"""

import numpy as np

from .verify import verify

# Largest |sum| an fp32 accumulation holds exactly (2^24): integer-valued
# operands below it give the exact product in any precision and order.
_EXACT_INT_LIMIT = float(1 << 24)


def lmhead_logits(hidden, weight, scale=1.0):
    """Logits l[r, v] = scale * sum_d hidden[r, d] * weight[v, d], in float64.

    hidden [R, D] and weight [V, D] hold values (any float dtype) or integers.
    With integer operands whose every partial sum is below 2^24 in magnitude
    (checked here from the operands' largest entries), the product is formed
    in float32, where it is exact, then widened; otherwise in float64.
    """
    h = np.asarray(hidden)
    w = np.asarray(weight)
    if h.ndim != 2 or w.ndim != 2 or h.shape[1] != w.shape[1]:
        raise ValueError("hidden [R, D] and weight [V, D] must share D")
    if np.issubdtype(h.dtype, np.integer) and np.issubdtype(w.dtype, np.integer):
        bound = (float(np.abs(h.astype(np.int64)).max(initial=0))
                 * float(np.abs(w.astype(np.int64)).max(initial=0)) * h.shape[1])
        if bound < _EXACT_INT_LIMIT:
            prod = h.astype(np.float32) @ w.astype(np.float32).T
            return prod.astype(np.float64) * float(scale)
    return (h.astype(np.float64) @ w.astype(np.float64).T) * float(scale)


def verify_lmhead(hidden_draft, weight_draft, hidden_target, weight_target, draft_tokens,
                  uniforms, *, B, K, V, temperature, draft_scale=1.0, target_scale=1.0,
                  want_diag=False):
    """The verification step on the LM-head logits of both models.

    hidden_draft [B*K, Dq], weight_draft [V, Dq], hidden_target [B*(K+1), Dp],
    weight_target [V, Dp]; the logits are ``lmhead_logits`` of each pair (times
    its scale), then ``verify`` runs on them as float64 rows (dense layout,
    sampling at ``temperature``; temperature 0 verifies greedily, reading no
    draft rows (R7), so the draft pair may be None).
    """
    if temperature == 0.0:
        lq = None
    else:
        lq = (lmhead_logits(hidden_draft, weight_draft, draft_scale) if K > 0
              else np.zeros((0, V), dtype=np.float64))
    lp = lmhead_logits(hidden_target, weight_target, target_scale)
    return verify(lq, lp, draft_tokens, uniforms, B=B, V=V, K=K, dtype="f64",
                  temperature=temperature, want_diag=want_diag)
