"""The binding's argument checks (-m "not gpu"): a tensor of the wrong dtype or
element count raises ValueError naming it before any pointer reaches the C
ABI, which trusts the sizes it is given. CPU tensors suffice: the checks run
before the device is touched."""

import pytest
import torch

import speculative_decoding_verification_13_amd as sv

B, K, V = 3, 4, 64


def _dense(**ov):
    a = dict(draft_logits=torch.zeros(B, K, V, dtype=torch.bfloat16),
             target_logits=torch.zeros(B, K + 1, V, dtype=torch.bfloat16),
             draft_tokens=torch.zeros(B, K, dtype=torch.int32),
             uniforms=torch.zeros(B, K + 1, dtype=torch.float32))
    a.update(ov)
    return a


@pytest.mark.parametrize("name,bad", [
    ("draft_logits", torch.zeros(B, K, V, dtype=torch.float16)),       # other storage type
    ("draft_logits", torch.zeros(B, K, V - 1, dtype=torch.bfloat16)),  # short rows
    ("target_logits", torch.zeros(B, K, V, dtype=torch.bfloat16)),     # no bonus rows
    ("draft_tokens", torch.zeros(B, K, dtype=torch.int64)),
    ("draft_tokens", torch.zeros(B, K - 1, dtype=torch.int32)),
    ("uniforms", torch.zeros(B, K + 1, dtype=torch.float64)),
    ("uniforms", torch.zeros(B, K, dtype=torch.float32)),
])
def test_dense_rejects_mismatched_tensors(name, bad):
    a = _dense(**{name: bad})
    with pytest.raises(ValueError, match=name):
        sv.spec_verify(a["draft_logits"], a["target_logits"], a["draft_tokens"], a["uniforms"],
                       B, K, V, 1.0)


def test_dense_rejects_mismatched_outputs():
    a = _dense()
    with pytest.raises(ValueError, match="out_tokens"):
        sv.spec_verify(*a.values(), B, K, V, 1.0, out_tokens=torch.zeros(B, K, dtype=torch.int32))
    with pytest.raises(ValueError, match="num_accepted"):
        sv.spec_verify(*a.values(), B, K, V, 1.0,
                       out_tokens=torch.zeros(B, K + 1, dtype=torch.int32),
                       num_accepted=torch.zeros(B, dtype=torch.int64))


def test_dense_optional_tensors():
    """Greedy calls need no uniforms and K = 0 calls no drafts; the checks then
    pass and the call stops only at the host-tensor check."""
    a = _dense()
    with pytest.raises(ValueError, match="device tensors"):
        sv.spec_verify(a["draft_logits"], a["target_logits"], a["draft_tokens"], None, B, K, V,
                       0.0, out_tokens=torch.zeros(B, K + 1, dtype=torch.int32),
                       num_accepted=torch.zeros(B, dtype=torch.int32),
                       workspace=torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="uniforms"):
        sv.spec_verify(a["draft_logits"], a["target_logits"], a["draft_tokens"], None, B, K, V,
                       1.0)


def test_ragged_and_accept_stats_checks():
    n_draft = 5
    draft = torch.zeros(n_draft, V, dtype=torch.float32)
    target = torch.zeros(n_draft + B, V, dtype=torch.float32)
    toks = torch.zeros(n_draft, dtype=torch.int32)
    u = torch.zeros(n_draft + B, dtype=torch.float32)
    cu = torch.tensor([0, 2, 2, 5], dtype=torch.int32)
    with pytest.raises(ValueError, match="cu_draft"):
        sv.spec_verify_ragged(draft, target, toks, u, cu.long(), None, B, V, 1.0)
    with pytest.raises(ValueError, match="greedy"):
        sv.spec_verify_ragged(draft, target, toks, u, cu, torch.zeros(B, dtype=torch.bool), B, V,
                              1.0)
    with pytest.raises(ValueError, match="target_logits"):
        sv.spec_verify_ragged(draft, target[:-1], toks, u, cu, None, B, V, 1.0)
    with pytest.raises(ValueError, match="ratio"):
        sv.spec_verify_ragged(draft, target, toks, u, cu, None, B, V, 1.0,
                              diag=dict(ratio=torch.zeros(n_draft + 1)))
    with pytest.raises(ValueError, match="draft_logits"):
        sv.spec_verify_accept_stats(draft.half(), target, cu, B, V, 1.0, total_draft_rows=n_draft)
    with pytest.raises(ValueError, match="beta"):
        sv.spec_verify_accept_stats(draft, target, cu, B, V, 1.0,
                                    beta=torch.zeros(n_draft, dtype=torch.float64))


def test_lmhead_checks():
    dq, dp, Vl = 16, 32, 40
    hq = torch.zeros(B * K, dq, dtype=torch.bfloat16)
    wq = torch.zeros(Vl, dq, dtype=torch.bfloat16)
    hp = torch.zeros(B * (K + 1), dp, dtype=torch.bfloat16)
    wp = torch.zeros(Vl, dp, dtype=torch.bfloat16)
    toks = torch.zeros(B * K, dtype=torch.int32)
    u = torch.zeros(B * (K + 1), dtype=torch.float32)
    with pytest.raises(ValueError, match="weight_target"):
        sv.spec_verify_lmhead(hq, wq, hp, wp[:-1], toks, u, B, K, Vl, 1.0)
    with pytest.raises(ValueError, match="hidden_draft"):
        sv.spec_verify_lmhead(hq.float(), wq, hp, wp, toks, u, B, K, Vl, 1.0)
    with pytest.raises(ValueError, match="uniforms"):
        sv.spec_verify_lmhead(hq, wq, hp, wp, toks, u[:-1], B, K, Vl, 1.0)
    # sampling needs the draft pair and the uniforms; only greedy (T = 0) may omit them
    with pytest.raises(ValueError, match="uniforms"):
        sv.spec_verify_lmhead(hq, wq, hp, wp, toks, None, B, K, Vl, 1.0)
    with pytest.raises(ValueError, match="hidden_draft"):
        sv.spec_verify_lmhead(None, wq, hp, wp, toks, u, B, K, Vl, 1.0)


def test_lmhead_logits_arrays_must_not_overlap():
    """A sampling call writes the diag logits arrays and its draw reads them
    back, so the binding refuses arrays that share bytes with each other or
    with the workspace."""
    dq, dp, Vl = 16, 32, 40
    hq = torch.zeros(B * K, dq, dtype=torch.bfloat16)
    wq = torch.zeros(Vl, dq, dtype=torch.bfloat16)
    hp = torch.zeros(B * (K + 1), dp, dtype=torch.bfloat16)
    wp = torch.zeros(Vl, dp, dtype=torch.bfloat16)
    toks = torch.zeros(B * K, dtype=torch.int32)
    u = torch.zeros(B * (K + 1), dtype=torch.float32)
    both = torch.zeros(B * (K + 1) * Vl + B * K * Vl, dtype=torch.float32)
    lt = both[:B * (K + 1) * Vl]
    ld = both[B * (K + 1) * Vl - 1:B * (K + 1) * Vl - 1 + B * K * Vl]  # one float shared
    ws = torch.zeros(int(sv.lib().spec_verify_lmhead_workspace_bytes(B, K, Vl)) + 4 * B * K * Vl,
                     dtype=torch.uint8)
    with pytest.raises(ValueError, match="overlap"):
        sv.spec_verify_lmhead(hq, wq, hp, wp, toks, u, B, K, Vl, 1.0, workspace=ws,
                              logits_draft=ld, logits_target=lt)
    inside = ws[-4 * B * K * Vl:].view(torch.float32)
    with pytest.raises(ValueError, match="overlap"):
        sv.spec_verify_lmhead(hq, wq, hp, wp, toks, u, B, K, Vl, 1.0, workspace=ws,
                              logits_draft=inside)
