"""paged_kv_cache_11_amd — PagedAttention for AMD Instinct MI355X (gfx950).

The compute lives in ``libpa.so`` (hand-written HIP, C ABI in include/pa.h);
``binding`` is a thin ctypes layer with the same function names.
``workloads`` holds the seeded synthetic input generators.
"""
from .binding import (  # noqa: F401
    PA_BF16, PA_F32, PA_FP8_E4M3, PA_PARTITION_BALANCED, BlockManager, PagedAttentionError, load,
    pa_cache_write, pa_copy_blocks,
    pa_decode, pa_decode_workspace_size, pa_pool_bytes, pa_prefill_chunk, pa_version,
)
