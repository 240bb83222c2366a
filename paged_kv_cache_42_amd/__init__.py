"""MI355X-native attention over a paged KV cache (libpkv, HIP for gfx950).

The compute lives in libpkv.so (C++ host code + HIP kernels, C ABI in include/pkv.h);
this package is its thin Python binding. Build with
`python -m paged_kv_cache_42_amd.build`.
"""
from ._lib import (  # noqa: F401
    BF16, F32, FP8, OutOfBlocks, PkvError, Pool, build_decode_work, decode_set_profile_event, decode_workspace_bytes, header_functions, kv_cache_write, lib,
    paged_attention_decode, build_varlen_work, paged_attention_prefill_varlen, SplitPlan, build_decode_split,
    decode_split_slots, decode_split_workspace_bytes, paged_attention_decode_split, Scheduler, StepPlan,
    MixedPlan, build_mixed_step, paged_attention_prefill_chunks, ChunkPlan, build_chunk_work, chunk_slots,
    chunk_workspace_bytes, swap_workspace_bytes, swap_out, swap_in, decode_split_noalloc_max_bytes,
    decode_split_workspace, split_plan_len,
    paged_attention_decode_split_noalloc, mixed_decode_slots, paged_attention_mixed,
)
