"""Shared test plumbing: pools built on the CPU from a workload's records."""
from __future__ import annotations

import numpy as np

import oracle
from workloads import Workload


def build_pools(w: Workload, include_new: bool = True, fill: str = "nan"):
    """Pools as the oracle's scatter writes them from the workload's records.

    Slots no record owns keep ``fill`` (NaN by default, so any read of them
    by a kernel shows up in its output).
    """
    kc, vc = oracle.empty_pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size,
                                w.dtype, fill=fill)
    recs = np.arange(len(w.rec_slot)) if include_new else w.history_records
    oracle.reshape_and_cache(w.rec_key[recs], w.rec_value[recs], w.rec_slot[recs], kc, vc,
                             inplace=True)
    return kc, vc


def oracle_out(w: Workload, kc, vc, seqs=None) -> np.ndarray:
    return oracle.paged_attention(w.query, w.block_table, w.context_lens, kc, vc, w.scale,
                                  w.dtype, seqs=seqs)
