"""paged_kv_cache_269_amd: PagedAttention decode for AMD Instinct MI355X (gfx950).

Thin Python binding over ``libpagedattn.so`` (C ABI in ``include/pagedattn.h``).
It only marshals torch tensors (device memory) and streams into the library's
entry points; every step of the computation runs in the library's HIP
kernels.  Importing the package never loads the library; the first call does,
and raises if the library is missing -- there is no fallback path.
"""
from ._binding import (  # noqa: F401
    BlockManager,
    KVCacheExhausted,
    PagedAttnError,
    cascade_workspace,
    cascade_workspace_bytes,
    copy_blocks,
    decode_workspace,
    decode_workspace_bytes,
    lib_path,
    load_library,
    multi_query_partition_size,
    multi_query_workspace,
    multi_query_workspace_bytes,
    paged_attention_decode,
    paged_attention_decode_cascade,
    paged_attention_multi_query,
    paged_attention_reduce,
    reshape_and_cache,
    reshape_and_decode,
    reshape_and_decode_cascade,
    reshape_and_decode_static,
    STATIC_SCRATCH_BYTES,
    status_string,
    swap_blocks,
    swap_blocks_mapped,
    validate_copy_host,
    validate_query_start_host,
    validate_slots_host,
    validate_step_host,
    validate_tables_host,
    version,
    EXPORTS,
)

__all__ = [
    "BlockManager", "KVCacheExhausted", "PagedAttnError", "cascade_workspace",
    "cascade_workspace_bytes", "copy_blocks", "decode_workspace", "decode_workspace_bytes",
    "lib_path", "load_library", "multi_query_partition_size", "multi_query_workspace", "multi_query_workspace_bytes",
    "paged_attention_decode", "paged_attention_decode_cascade", "paged_attention_multi_query",
    "paged_attention_reduce", "reshape_and_cache", "reshape_and_decode", "reshape_and_decode_cascade",
    "reshape_and_decode_static", "STATIC_SCRATCH_BYTES", "status_string",
    "swap_blocks",
    "swap_blocks_mapped",
    "validate_copy_host", "validate_query_start_host", "validate_slots_host", "validate_step_host",
    "validate_tables_host", "version", "EXPORTS",
]
