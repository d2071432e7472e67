"""MI355X (gfx950) paged-KV decode library: Python face of libpagedattn.so.

The work runs in hand-written HIP kernels behind a C ABI (include/pagedattn.h);
this package only marshals torch tensors to it.
"""
from .binding import (LIB_PATH, PreparedCall, chunk_elems, copy_blocks, decode_step,
                      default_partition_size, prepare_copy_blocks,
                      gather_kv, k_cache_shape, load_library, paged_attention, paged_prefill,
                      prepare_decode_step, prepare_paged_attention, prepare_reshape_and_cache,
                      reshape_and_cache, v_cache_shape, workspace_size)

__all__ = ["LIB_PATH", "PreparedCall", "copy_blocks", "prepare_copy_blocks", "decode_step",
           "prepare_decode_step",
           "prepare_paged_attention", "prepare_reshape_and_cache",
           "chunk_elems", "default_partition_size", "gather_kv", "k_cache_shape",
           "load_library", "paged_attention", "paged_prefill", "reshape_and_cache", "v_cache_shape",
           "workspace_size"]
