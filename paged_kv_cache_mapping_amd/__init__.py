"""Paged KV-cache hot path for AMD Instinct MI355X (gfx950).

Slot mapping, KV-cache writes and paged attention (decode and chunked, with
grouped-query heads, sliding windows and FP8 E4M3 or INT4 caches) run in the
hand-written HIP kernels of ``libpagedkv.so``; this package marshals torch
tensors into its C ABI (``include/pagedkv.h``) and holds the host-side block
pool and layout helpers.  Importing it does not load the library; the first
call does, and fails loudly if it has not been built.
"""

from .api import (CacheView, cache_write, chunked_workspace_size, copy_blocks, decode_plan,  # noqa: F401
                  fp8_dequantize, fp8_quantize, int4_dequantize, int4_quantize, kv_bytes_per_token,
                  paged_attention_chunked,
                  paged_attention_decode, paged_attention_decode_combine, paged_attention_decode_step,
                  paged_attention_decode_partials, slot_mapping, slot_mapping_cache_write, status_string,
                  new_workspace, tune_plan)
from ._lib import PkvError, load  # noqa: F401
from . import kv_cache, workloads  # noqa: F401
