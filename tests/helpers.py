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


def per_sequence(fn, seqs, threads: int = 16):
    """[fn(s) for s in seqs], run on a thread pool with BLAS held to one thread per call.

    The oracle's large array operations release the GIL, so whole-batch references of
    the full-size workloads finish in seconds instead of minutes.  The result does not
    depend on the thread count: every call is one sequence, computed alone.
    """
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    seqs = list(seqs)
    workers = max(1, min(threads, len(os.sched_getaffinity(0)), len(seqs)))
    with threadpool_limits(1):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, seqs))


def fp8_reference_pools(w, recs, k_scale: float, v_scale: float, fill: int = 0x7F):
    """FP8 pools holding records ``recs`` of a bf16 workload, quantised by the oracle
    (through its table of every bf16 pattern) and scattered by the oracle."""
    kc, vc = oracle.empty_fp8_pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size,
                                    fill=fill)
    kq = oracle.quantize_bf16(w.rec_key[recs], k_scale)
    vq = oracle.quantize_bf16(w.rec_value[recs], v_scale)
    oracle.reshape_and_cache(kq, vq, w.rec_slot[recs], kc, vc, inplace=True)
    return kc, vc


def fp8_reference_out(w, kc, vc, k_scale: float, v_scale: float) -> np.ndarray:
    """Oracle FP8 attention of every sequence (one sequence per call, threaded)."""
    def one(s):
        return oracle.paged_attention_fp8(w.query[s:s + 1], w.block_table[s:s + 1],
                                          w.context_lens[s:s + 1], kc, vc, w.scale, k_scale,
                                          v_scale, w.dtype)[0]
    return np.stack(per_sequence(one, range(w.num_seqs)))


def prefill_reference(w, pb, kc, vc) -> np.ndarray:
    """Oracle prefill of every row of a batch (one sequence per call, threaded)."""
    qsl = pb.query_start_loc

    def one(s):
        r0, r1 = int(qsl[s]), int(qsl[s + 1])
        return oracle.paged_prefill(pb.query[r0:r1], np.array([0, r1 - r0], dtype=np.int32),
                                    w.block_table[s:s + 1], w.context_lens[s:s + 1], kc, vc,
                                    w.scale, w.dtype)
    return np.concatenate(per_sequence(one, range(w.num_seqs)))
