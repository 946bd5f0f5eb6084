"""fp64 CPU oracle for cascade beam-decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this package: only the tests, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` do. It shares no code with the HIP path.

Pins (CPU tests in ``tests/test_oracle_pins.py``), function by function:

* ``attend``: closed forms (identical keys, single key, empty set), 50-digit
  brute force through every function below;
* ``merge_states``: merge = unsplit at every split point, n-way association
  orders, empty parts;
* ``sequence_slots``, ``tail_slots``, ``prefix_page_table``, ``write_kv``,
  ``bucket_rows``: hand-derived index values under ``tests/golden/`` and the
  generator's logical placement of every row;
* ``beam_decode_attention``: 50-digit brute force over sequences rebuilt from
  the logical draws, torch SDPA (fp64) for beam 1 without a tail, zero-query
  and relabelling invariants;
* ``beam_attention_one``: bit-equal to the slice of ``beam_decode_attention``
  and 50-digit brute force;
* ``beam_partial_attention``: 50-digit brute force of each part over the
  logical prompt rows and the logical tail rows separately (a boundary off by
  one at the prompt end fails), and a tail-only change leaves the prefix part
  unchanged;
* ``cached_prefix_attention``: 50-digit brute force, SDPA with the explicit
  ``[Sq, bound + Sq]`` mask, bound-row invariance with the Phi-4 PR's printed
  cases, garbage and NaN past the valid rows;
* ``cached_prefix_partial``: 50-digit brute force over explicit key ranges
  (inside, across and past the valid length) and the new-row segment, and the
  merge of chunked partials with the new-row segment = the whole call;
* ``prefill_attention(_one)``: torch causal SDPA, SDPA with an explicit mask
  over cached rows, 50-digit brute force, two chunks = one chunk.

None is "parity unpinned".
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
