"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library shares no code with it and never calls
it.  Every function is pinned by a check in the test suite; none is marked
"parity unpinned".
"""
from .paged_attention import (ELEMENT_BYTES, attention_one, chunk_elems, combine_partitions,
                              copy_blocks, decode, empty_pools, gather_kv, gather_sequence,
                              k_cache_shape, paged_attention, paged_prefill, partition_stats,
                              reshape_and_cache, swap_blocks, v_cache_shape)

from .fp8_kv import (FP8_MAX, e4m3_decode, e4m3_encode, e4m3_values, empty_fp8_pools,
                     paged_attention_fp8, quantize, quantize_bf16, reshape_and_cache_fp8)

__all__ = ["FP8_MAX", "e4m3_decode", "e4m3_encode", "e4m3_values", "empty_fp8_pools",
           "paged_attention_fp8", "quantize", "quantize_bf16", "reshape_and_cache_fp8",
           "ELEMENT_BYTES", "attention_one", "chunk_elems", "combine_partitions", "copy_blocks",
           "decode",
           "empty_pools", "gather_kv", "gather_sequence", "k_cache_shape",
           "paged_attention", "paged_prefill", "partition_stats", "reshape_and_cache", "swap_blocks",
           "v_cache_shape"]
