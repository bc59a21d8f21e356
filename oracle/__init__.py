"""CPU oracle for paged single-token decode attention (fp64, NumPy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``, and by nothing else.  The GPU
library never imports, links or calls it, and it imports nothing from the GPU
library.  Every function is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle.py`` (brute force, closed forms, invariants, the
log-sum-exp merge identity, a float64 library special case and hand-worked
fixtures); there is no "parity unpinned" function.
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
