"""Paged attention for AMD Instinct MI355X (gfx950).

A thin Python face of ``libpa.so``: the functions here carry the names of the
library's C entry points and only marshal torch device tensors into them.
"""
from ._binding import (  # noqa: F401
    CHECK_LIB_PATH,
    LIB_PATH,
    BlockManager,
    PA_BF16,
    PA_F16,
    PAError,
    checked_indices,
    decode_workspace,
    load_library,
    pa_cache_flush,
    pa_stream_read,
    pa_copy_blocks,
    pa_decode,
    pa_decode_int8,
    pa_decode_merge,
    pa_decode_order,
    pa_decode_partial,
    pa_decode_partition_hint,
    pa_decode_partitions,
    pa_decode_step,
    pa_decode_step_int8,
    pa_decode_step_rope,
    pa_decode_step_scratch,
    pa_decode_workspace_size,
    pa_merge_partials,
    pa_prefill_chunk,
    pa_reshape_and_cache,
    pa_reshape_and_cache_int8,
    pa_set_kernel_events,
    pa_rope_reshape_and_cache,
    pa_take_index_errors,
    pa_version,
)
