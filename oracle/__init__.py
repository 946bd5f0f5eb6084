"""fp64 CPU oracle for cascade beam-decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this package: only the tests, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` do. It shares no code with the HIP path.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (brute force at 50 digits, library attention,
closed forms, invariants and printed values); none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attend,
    beam_attention_one,
    beam_decode_attention,
    beam_partial_attention,
    bucket_rows,
    cached_prefix_attention,
    cached_prefix_partial,
    merge_states,
    prefill_attention,
    prefill_attention_one,
    sequence_slots,
    write_kv,
)
from .plan import prefix_page_table, tail_slots  # noqa: F401
