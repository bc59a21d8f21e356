"""MI355X (gfx950) paged single-token decode attention, and paged prefix (chunked
prefill) attention.

The compute lives in ``libpad.so`` (hand-written HIP kernels behind a C ABI,
``include/paged_attention_decode.h`` and ``include/paged_attention_prefill.h``).  This package exposes the same entry
points for torch tensors (:mod:`._binding`) and the seeded synthetic input
generator (:mod:`.inputs`).  Importing the binding raises if the library has
not been built: there is no fallback path.
"""

from ._binding import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    PAD_DTYPE_BF16,
    PAD_DTYPE_F32,
    PadDims,
    PadError,
    PadPrefillDims,
    alloc_prefill_split_workspace,
    alloc_workspace,
    check_build,
    make_dims,
    make_prefill_dims,
    paged_attention_decode,
    paged_attention_decode_build_id,
    paged_attention_decode_choose_partition,
    paged_attention_decode_choose_partition_for_batch,
    paged_attention_decode_entry_ranges,
    paged_attention_decode_no_alloc,
    paged_attention_decode_phase1,
    paged_attention_decode_phase2,
    paged_attention_decode_strerror,
    paged_attention_decode_workspace_init,
    paged_attention_decode_workspace_layout,
    paged_attention_decode_workspace_size,
    paged_attention_prefill,
    paged_attention_prefill_choose_split,
    paged_attention_prefill_split,
    paged_attention_prefill_split_ranges,
    paged_attention_prefill_split_workspace_size,
    paged_attention_prefill_write_kv,
)
