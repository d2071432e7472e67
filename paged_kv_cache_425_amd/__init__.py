"""MI355X (gfx950) paged-KV decode library: Python face of libpagedattn.so.

The work runs in hand-written HIP kernels behind a C ABI (include/pagedattn.h);
this package only marshals torch tensors to it.
"""
from .binding import (LIB_PATH, PreparedCall, chunk_elems, copy_blocks, decode_math,
                      decode_step, get_decode_math, set_decode_math,
                      decode_step_noalloc, decode_step_shared_prefix, read_probe, coexec_probe,
                      plan_pairs, prepare_decode_step_shared_prefix,
                      decode_step_fp8, default_partition_size, gather_kv, k_cache_shape,
                      load_library, prepare_decode_step_fp8, paged_attention,
                      prepare_swap_blocks, swap_blocks, paged_attention_fp8, paged_prefill, prepare_copy_blocks,
                      prepare_decode_step, prepare_paged_attention, prepare_paged_attention_fp8,
                      prepare_reshape_and_cache, prepare_reshape_and_cache_fp8, reshape_and_cache,
                      reshape_and_cache_fp8, v_cache_shape, v_group, workspace_size)

__all__ = ["LIB_PATH", "PreparedCall", "chunk_elems", "copy_blocks", "decode_math",
           "decode_step", "get_decode_math", "set_decode_math",
           "decode_step_noalloc", "decode_step_shared_prefix", "read_probe", "coexec_probe",
           "plan_pairs", "prepare_decode_step_shared_prefix",
           "decode_step_fp8", "prepare_decode_step_fp8", "prepare_swap_blocks", "swap_blocks",
           "default_partition_size", "gather_kv", "k_cache_shape", "load_library",
           "paged_attention", "paged_attention_fp8", "paged_prefill", "prepare_copy_blocks",
           "prepare_decode_step", "prepare_paged_attention", "prepare_paged_attention_fp8",
           "prepare_reshape_and_cache", "prepare_reshape_and_cache_fp8", "reshape_and_cache",
           "reshape_and_cache_fp8", "v_cache_shape", "v_group", "workspace_size"]
