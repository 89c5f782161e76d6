"""MI355X-native batched speculative-decoding verification.

The work runs in hand-written HIP kernels for gfx950 behind the C ABI of
``include/spec_verify.h`` (``libspecverify.so``, built in-tree by
``python -m speculative_decoding_verification_13_amd.build``). This package is
the thin Python binding: it marshals torch device tensors and the current
stream into those calls.
"""

from ._lib import (  # noqa: F401
    SV_MAX_K,
    SV_SEQ_BAD_OFFSETS,
    SV_SEQ_BAD_ROW,
    SV_SEQ_BAD_TOKEN,
    SV_SEQ_SYNC_TIMEOUT,
    SequenceError,
    SpecVerifyError,
    lib,
    make_lmhead_workspace,
    make_stage_events,
    make_workspace,
    num_stages,
    spec_verify,
    spec_verify_accept_stats,
    spec_verify_lmhead,
    spec_verify_multi,
    spec_verify_noalloc,
    spec_verify_ragged,
    strerror,
    workspace_bytes,
)
