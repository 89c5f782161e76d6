"""Float64 CPU oracle of batched speculative-decoding verification.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this package. The product (the HIP
kernels, the C ABI and the Python binding under
``speculative_decoding_verification_13_amd/``) shares no code with it and never
imports, links or calls it.

Every function here is pinned by tests under ``tests/test_oracle_*.py`` against
values the pages print, closed forms, exact path enumeration and library
routines; see the docstrings for the passage each step follows.
"""

from .verify import (  # noqa: F401
    ACCEPT_MARGIN_INF,
    decode_logits,
    row_is_valid,
    filtered_distribution,
    accept_ratio,
    residual,
    inverse_cdf,
    greedy_token,
    verify_sequence,
    verify,
    sample_rows,
    acceptance_probability,
    acceptance_stats,
)
from .lmhead import lmhead_logits, verify_lmhead  # noqa: F401,E402
from .multi import verify_multi, verify_multi_sequence  # noqa: F401,E402
