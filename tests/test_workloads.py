"""Host logic: block pool, copy-on-write, and the five named workloads' shapes."""
from __future__ import annotations

import numpy as np
import pytest

from workloads import (BlockPool, PoolExhausted, SequenceBlocks, append_token, make_config,
                       make_workload)


def test_pool_hands_out_each_block_once_then_raises():
    pool = BlockPool(5, np.random.default_rng(0))
    got = [pool.allocate() for _ in range(5)]
    assert sorted(got) == list(range(5))
    with pytest.raises(PoolExhausted):
        pool.allocate()
    pool.release(got[2])
    assert pool.allocate() == got[2]


def test_append_allocates_on_demand_one_block_per_block_size_tokens():
    pool = BlockPool(10, np.random.default_rng(1))
    seq = SequenceBlocks()
    slots = [append_token(seq, pool, 4).slot for _ in range(9)]
    assert len(seq.blocks) == 3 and pool.num_free == 7
    for t, slot in enumerate(slots):
        assert slot == seq.blocks[t // 4] * 4 + t % 4


def test_fork_shares_and_copy_on_write_splits_the_partial_block():
    pool = BlockPool(20, np.random.default_rng(2))
    prompt = SequenceBlocks()
    for _ in range(6):                     # 1 full block + 2 tokens in the second
        append_token(prompt, pool, 4)
    samples = [prompt.fork(pool) for _ in range(3)]
    assert pool.refcount[prompt.blocks[1]] == 4
    writes = []
    for i, s in enumerate(samples):
        writes.append(append_token(s, pool, 4))
        # each writer finds the partial block shared, copies it, drops its reference
        assert writes[-1].copy_from == prompt.blocks[1] and writes[-1].copy_to >= 0
        assert pool.refcount[prompt.blocks[1]] == 3 - i
    # with the template's reference gone the last holder writes in place
    pool.release(prompt.blocks[1])
    solo = SequenceBlocks(blocks=[prompt.blocks[0], pool.allocate()], num_tokens=6)
    assert append_token(solo, pool, 4).copy_from == -1
    assert len({w.slot for w in writes}) == 3
    assert all(s.blocks[0] == prompt.blocks[0] for s in samples)   # full block stays shared


def test_parallel_sampling_workload_layout():
    w = make_config(3, variant="parallel-sampling")
    assert w.num_seqs == 128
    BS = w.block_size
    for p in range(32):
        group = range(4 * p, 4 * p + 4)
        Lp = int(w.context_lens[4 * p]) - 1
        full = Lp // BS
        tables = w.block_table[list(group)]
        assert (tables[:, :full] == tables[0, :full]).all()       # full prompt blocks shared
        if Lp % BS:
            last = tables[:, full]
            assert len(set(last.tolist())) == 4                   # every sample owns its copy
        # the copies hold the same prompt tokens as the original
        for s in group:
            recs = w.seq_records[s]
            assert np.array_equal(w.rec_key[recs[:Lp]], w.rec_key[w.seq_records[4 * p][:Lp]])


def test_prefix_workload_stores_prefix_once():
    w = make_config(3)
    assert (w.block_table[:, :64] == w.block_table[0, :64]).all()
    assert (w.context_lens >= 1024 + 32).all() and (w.context_lens <= 1024 + 512).all()
    assert w.kv_bytes_unique < w.kv_bytes_logical


@pytest.mark.parametrize("index", [0, 1, 3])
def test_named_workload_tables_and_slots(index):
    w = make_config(index)
    BS = w.block_size
    assert w.block_table.dtype == np.int32 and w.context_lens.dtype == np.int32
    assert ((w.block_table >= 0) & (w.block_table < w.num_blocks)).all()
    # every record's slot is where its sequence's table says it is
    for s in range(w.num_seqs):
        t = np.arange(int(w.context_lens[s]))
        expect = w.block_table[s, t // BS].astype(np.int64) * BS + t % BS
        assert np.array_equal(w.rec_slot[w.seq_records[s]], expect)
    # slots written are distinct (history and new together)
    assert len(np.unique(w.rec_slot)) == len(w.rec_slot)
    # the step's new tokens are the last positions
    assert len(w.new_records) == w.num_seqs
    for s in range(w.num_seqs):
        assert w.seq_records[s][-1] == w.new_records[s]


def test_config_shapes():
    w0 = make_config(0)
    assert list(w0.context_lens) == [5, 17, 33, 64]
    assert (w0.num_heads, w0.num_kv_heads, w0.head_dim, w0.block_size, w0.num_blocks) == \
        (4, 4, 64, 16, 64)
    assert w0.dtype == "f32" and w0.scale == 1 / 8
    w1 = make_config(1)
    assert (w1.num_seqs, w1.num_heads, w1.num_kv_heads, w1.head_dim, w1.block_size) == \
        (64, 32, 8, 128, 16)
    assert w1.context_lens.min() >= 128 and w1.context_lens.max() <= 2048
    need = sum(-(-int(L) // 16) for L in w1.context_lens)
    assert w1.num_blocks == int(np.ceil(1.2 * need))


@pytest.mark.slow
def test_large_configs_shapes():
    w2 = make_config(2, block_size=8)
    assert w2.num_seqs == 256 and w2.block_size == 8
    assert (w2.context_lens >= 2000).sum() == 26
    w4 = make_config(4)
    assert (w4.num_heads, w4.num_kv_heads, w4.block_size) == (64, 8, 32)
    assert w4.context_lens.min() >= 16384 and w4.context_lens.max() <= 32768


def test_seed_reproducibility():
    a = make_workload(name="a", context_lens=[10, 70], num_heads=4, num_kv_heads=2,
                      head_dim=16, block_size=8, dtype="bf16", seed=7)
    b = make_workload(name="b", context_lens=[10, 70], num_heads=4, num_kv_heads=2,
                      head_dim=16, block_size=8, dtype="bf16", seed=7)
    assert np.array_equal(a.block_table, b.block_table)
    assert np.array_equal(a.rec_key, b.rec_key) and np.array_equal(a.query, b.query)
