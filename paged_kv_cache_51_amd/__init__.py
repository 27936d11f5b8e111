"""paged_kv_cache_51_amd — paged KV cache + PagedAttention decode for MI355X.

A thin ctypes binding over libpagedkv.so (include/pagedkv.h): every step of
the decode path runs in the library's HIP kernels; this module only turns
torch tensors into pointers, sizes and the current HIP stream.  There is no
fallback: if the library is missing or fails to load, importing the binding
raises.
"""
from ._binding import (  # noqa: F401
    BF16, FP16, FP8_E4M3, IMPL_AUTO, IMPL_MFMA, IMPL_VECTOR, IMPL_MFMA_PERSISTENT, STAGE_PARTITIONS, STAGE_REDUCE,
    PagedKVError, KVPool, lib, lib_path, version, last_error, bytes_per_token, tile_bytes,
    layer_pool_bytes, workspace_bytes, default_partition_tokens, plan_bytes, build_plan,
    decode_slot_mapping, reshape_and_cache,
    paged_attention_decode, paged_attention_decode_append, check_block_tables, torch_dtype, dtype_code, EXPORTS,
    BlockManager, copy_blocks, paged_attention_prefill, paged_attention_decode_tokens, token_runs_bytes, token_runs,
    paged_attention_decode_runs, RUNS_MIN_KEYS,
    move_tokens,
    repack_blocks,
    read_probe,
)
