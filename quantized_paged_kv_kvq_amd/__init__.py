"""MI355X-native quantized paged KV cache: quantize-on-write into packed pages, and decode /
verify / extend attention that dequantises K and V inside the attention loop.

The hot path is libkvq.so (hand-written HIP for gfx950, C ABI in include/kvq.h); the module
``kvq`` is its ctypes binding.  Importing this package does not load the library; the first
call does, and raises if it has not been built.
"""
from .kvq import (FMT, PAGE_SIZE, KVQError, PagedKVCache, Pages, cell_bytes, kvq_append,  # noqa: F401
                  kvq_decode_attn, kvq_decode_attn_append, kvq_decode_attn_noalloc, kvq_decode_workspace_bytes, kvq_dequant_gather,
                  kvq_extend_attn, kvq_extend_workspace_bytes, lib)
