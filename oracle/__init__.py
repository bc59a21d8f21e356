"""CPU oracles for paged decode attention and paged prefix (prefill) attention (fp64, NumPy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``, and by nothing else.  The GPU
library never imports, links or calls it, and it imports nothing from the GPU
library.  Every function is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle.py`` and ``tests/test_oracle_prefill.py`` (brute force,
closed forms, invariants, the log-sum-exp merge identity, the pages' two-phase
prefill form, float64 library special cases and hand-worked fixtures).  The
two helpers that serve sampled checks at full size, ``attend_logical`` and
``prefill_rows``, are pinned row for row against pure-Python brute force and
against ``decode_attention`` / ``prefill_attention``; there is no "parity
unpinned" function.
"""

from .attention import (  # noqa: F401
    attend,
    attend_logical,
    decode_attention,
    decode_attention_split,
    gather_sequence,
    kv_head_for,
    merge_partitions,
    partition_stats,
    widen,
)
from .prefill import (  # noqa: F401
    chunk_bounds,
    prefill_attention,
    prefill_rows,
    prefix_attention_two_phase,
    write_chunk,
)
