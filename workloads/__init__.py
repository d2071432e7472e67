"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's
checks.  Holds no attention arithmetic: only random draws and integer tables."""
from .block_pool import BlockPool, PoolExhausted, SequenceBlocks, SlotWrite, append_token
from .configs import (BF16_NAN_BITS, CONFIG_NAMES, PREFILL_NAMES, PrefillBatch, Workload,
                      element_size, f32_to_bf16_bits, make_config, make_prefill,
                      make_prefill_config, make_workload)

__all__ = ["BlockPool", "PoolExhausted", "SequenceBlocks", "SlotWrite", "append_token",
           "BF16_NAN_BITS", "CONFIG_NAMES", "PREFILL_NAMES", "PrefillBatch", "Workload",
           "element_size", "f32_to_bf16_bits", "make_config", "make_prefill",
           "make_prefill_config", "make_workload"]
