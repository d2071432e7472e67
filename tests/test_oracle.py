"""Pins for the CPU oracle: each check ties it to something other than itself.

* values printed in a hand-worked fixture (tests/golden/hand_worked_fp32.json);
* dense brute-force attention over the never-paged sequence, written with
  explicit loops, math.exp and math.fsum, and bf16 decoded by torch;
* the invariances the pages state: physical blocks may sit anywhere, may be
  shared, and the block size is a tunable that does not change the result;
* closed forms of softmax attention (single token, zero scale, constant V,
  needle, two tokens = logistic function, scipy's softmax);
* the log-sum-exp combination of partitions against the direct result.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from tests.helpers import build_pools, oracle_out
from workloads import f32_to_bf16_bits, make_config, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_fp32.json")


def torch_decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values decoded by torch (independent of the oracle's decode)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
        return t.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def dense_bruteforce(w, s: int, h: int) -> list:
    """Softmax attention of query (s, h) over the never-paged K/V, plain loops."""
    g = w.num_heads // w.num_kv_heads
    kvh = h // g
    recs = w.seq_records[s]
    K = torch_decode(w.rec_key[recs][:, kvh], w.dtype)
    V = torch_decode(w.rec_value[recs][:, kvh], w.dtype)
    q = torch_decode(w.query[s, h], w.dtype)
    L, D = K.shape
    if L == 0:
        return [0.0] * D
    z = [w.scale * math.fsum(float(q[d]) * float(K[t, d]) for d in range(D)) for t in range(L)]
    m = max(z)
    e = [math.exp(zt - m) for zt in z]
    den = math.fsum(e)
    return [math.fsum(e[t] * float(V[t, d]) for t in range(L)) / den for d in range(D)]


def tiny(dtype="bf16", lens=(1, 7, 21, 40), Hq=4, Hkv=2, D=16, BS=8, seed=5, **kw):
    return make_workload(name="tiny", context_lens=list(lens), num_heads=Hq, num_kv_heads=Hkv,
                         head_dim=D, block_size=BS, dtype=dtype, seed=seed, **kw)


# ---------------------------------------------------------------------------
# element decoding
# ---------------------------------------------------------------------------
def test_bf16_decode_matches_torch_on_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode(bits, "bf16")
    ref = torch_decode(bits, "bf16")
    assert np.array_equal(ours, ref, equal_nan=True)


def test_generator_rounding_matches_torch_including_ties():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100_000).astype(np.float32)
    # exact ties: low 16 bits 0x8000, with both parities of the kept bit
    ties = (rng.integers(0, 1 << 16, 1000).astype(np.uint32) << 16) | np.uint32(0x8000)
    ties = ties[np.isfinite(ties.view(np.float32))].view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


# ---------------------------------------------------------------------------
# hand-worked fixture
# ---------------------------------------------------------------------------
def _golden():
    with open(GOLDEN) as f:
        g = json.load(f)

    def arr(x):
        return np.array(x, dtype=object).astype(float).astype(np.float32)

    nanify = lambda x: np.where(np.array(x, dtype=object) == None, np.nan, x).astype(np.float32)  # noqa: E711,E731
    # The fixture lists V as [block][kv_head][d][offset].  With 2-token blocks of f32 a block
    # is a single V group, so the pool's [block][kv_head][group][d][offset in group] holds the
    # same numbers with a unit group axis.
    return g, nanify(g["k_cache"]), nanify(g["v_cache"])[:, :, None, :, :], arr


def test_golden_layout_shapes():
    g, kc, vc, _ = _golden()
    assert kc.shape == oracle.k_cache_shape(g["num_blocks"], g["num_kv_heads"], g["head_dim"],
                                            g["block_size"], "f32")
    assert vc.shape == oracle.v_cache_shape(g["num_blocks"], g["num_kv_heads"], g["head_dim"],
                                            g["block_size"], "f32")


def test_golden_gather():
    g, kc, vc, arr = _golden()
    table = np.array(g["block_table"], dtype=np.int32)
    for s, L in enumerate(g["context_lens"]):
        k, v = oracle.gather_sequence(table[s], L, kc, vc)
        assert np.array_equal(k, arr(g["expected_gather"]["k"][s]))
        assert np.array_equal(v, arr(g["expected_gather"]["v"][s]))


def test_golden_attention():
    g, kc, vc, arr = _golden()
    out = oracle.paged_attention(arr(g["query"]), np.array(g["block_table"]),
                                 np.array(g["context_lens"]), kc, vc, g["scale"], "f32")
    np.testing.assert_allclose(out, np.array(g["expected_out"], dtype=float), rtol=0, atol=1e-13)


def test_golden_append_then_attention():
    g, kc, vc, arr = _golden()
    a = g["append"]
    kc2, vc2 = oracle.reshape_and_cache(arr(a["key"]), arr(a["value"]), np.array(a["slot_mapping"]),
                                        kc, vc)
    changed_k = ~((kc2 == kc) | (np.isnan(kc2) & np.isnan(kc)))
    changed_v = ~((vc2 == vc) | (np.isnan(vc2) & np.isnan(vc)))
    # slot 1 = physical block 0, offset 1: only those elements changed
    assert changed_k.sum() == 8 and changed_k[0, :, 1, :].all()
    assert changed_v.sum() == 8 and changed_v[0, :, 0, :, 1].all()   # group 0, offset 1
    out = oracle.paged_attention(arr(g["query"]), np.array(g["block_table"]),
                                 np.array(a["context_lens_after"]), kc2, vc2, g["scale"], "f32")
    np.testing.assert_allclose(out[0], np.array(a["expected_out_seq0"], dtype=float),
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[1], np.array(g["expected_out"][1], dtype=float),
                               rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# gather and scatter against independent formulations
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,BS,D", [("f32", 16, 64), ("bf16", 8, 16), ("bf16", 32, 32),
                                        ("f32", 8, 8)])
def test_gather_matches_flat_index_loop_and_never_paged_records(dtype, BS, D):
    w = tiny(dtype=dtype, BS=BS, D=D, lens=(1, 9, 33))
    kc, vc = build_pools(w)
    kflat, vflat = kc.reshape(-1), vc.reshape(-1)
    Hkv = w.num_kv_heads
    for s in range(w.num_seqs):
        k, v = oracle.gather_sequence(w.block_table[s], w.context_lens[s], kc, vc)
        # the never-paged sequence the pool was filled from
        assert np.array_equal(k, w.rec_key[w.seq_records[s]])
        assert np.array_equal(v, w.rec_value[w.seq_records[s]])
        # one element at a time, flat offsets written out by hand (V: groups of X tokens,
        # X = min(16 bytes / element, BS), each group channel-major)
        X = min(16 // (4 if dtype == "f32" else 2), BS)
        for t in range(int(w.context_lens[s])):
            b = int(w.block_table[s, t // BS])
            o = t % BS
            for h in range(Hkv):
                for d in range(D):
                    ko = ((b * Hkv + h) * BS + o) * D + d
                    vo = (((b * Hkv + h) * (BS // X) + o // X) * D + d) * X + o % X
                    assert k[t, h, d] == kflat[ko]
                    assert v[t, h, d] == vflat[vo]


def test_scatter_touches_only_its_slots_and_skips_negative():
    w = tiny(dtype="bf16", BS=16, D=32, lens=(5, 20))
    kc, vc = build_pools(w, include_new=False)
    new = w.new_records
    slots = w.rec_slot[new].copy()
    slots[0] = -1                                  # padding entry: no write
    kc2, vc2 = oracle.reshape_and_cache(w.rec_key[new], w.rec_value[new], slots, kc, vc)
    BS = w.block_size
    for i, slot in enumerate(slots):
        blk, off = divmod(int(w.rec_slot[new][i]), BS)
        if slot < 0:
            assert np.array_equal(kc2[blk, :, off, :], kc[blk, :, off, :])
            continue
        X = vc.shape[4]
        kc2[blk, :, off, :] = kc[blk, :, off, :]
        vc2[blk, :, off // X, :, off % X] = vc[blk, :, off // X, :, off % X]
    assert np.array_equal(kc2, kc) and np.array_equal(vc2, vc)  # nothing else changed


def test_scatter_rejects_duplicate_slots():
    w = tiny(dtype="f32", lens=(3,))
    kc, vc = build_pools(w)
    with pytest.raises(AssertionError):
        oracle.reshape_and_cache(w.rec_key[:2], w.rec_value[:2], np.array([4, 4]), kc, vc)


# ---------------------------------------------------------------------------
# attention against brute force and closed forms
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,BS,Hq,Hkv", [("bf16", 8, 4, 2), ("f32", 16, 4, 1),
                                             ("bf16", 32, 8, 2), ("f32", 8, 2, 2)])
def test_attention_matches_dense_bruteforce(dtype, BS, Hq, Hkv):
    w = tiny(dtype=dtype, BS=BS, Hq=Hq, Hkv=Hkv, lens=(1, 7, 21, 40), scale=0.3)
    kc, vc = build_pools(w)
    out = oracle_out(w, kc, vc)
    for s in range(w.num_seqs):
        for h in range(w.num_heads):
            np.testing.assert_allclose(out[s, h], dense_bruteforce(w, s, h), rtol=1e-12,
                                       atol=1e-13)


def test_attention_matches_scipy_softmax():
    w = make_config(0)
    kc, vc = build_pools(w)
    out = oracle_out(w, kc, vc)
    for s in range(w.num_seqs):
        K = w.rec_key[w.seq_records[s]].astype(np.float64)
        V = w.rec_value[w.seq_records[s]].astype(np.float64)
        for h in range(w.num_heads):
            p = scipy.special.softmax(w.scale * K[:, h] @ w.query[s, h].astype(np.float64))
            np.testing.assert_allclose(out[s, h], p @ V[:, h], rtol=1e-12, atol=1e-14)


def test_single_token_returns_its_value_exactly():
    w = tiny(dtype="bf16", lens=(1, 1, 1))
    kc, vc = build_pools(w)
    out = oracle_out(w, kc, vc)
    g = w.num_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        for h in range(w.num_heads):
            v = torch_decode(w.rec_value[w.seq_records[s][0], h // g], "bf16")
            assert np.array_equal(out[s, h], v)


def test_zero_scale_gives_mean_of_values():
    w = tiny(dtype="f32", lens=(3, 17, 50), scale=0.0)
    kc, vc = build_pools(w)
    out = oracle_out(w, kc, vc)
    g = w.num_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        V = w.rec_value[w.seq_records[s]].astype(np.float64)
        for h in range(w.num_heads):
            np.testing.assert_allclose(out[s, h], V[:, h // g].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_constant_values_and_group_mapping():
    """V constant over tokens with a distinct constant per KV head: query head h
    must return the constant of KV head h // g (a wrong grouping shows)."""
    w = tiny(dtype="f32", lens=(9, 30), Hq=8, Hkv=2, D=8)
    for kvh in range(w.num_kv_heads):
        w.rec_value[:, kvh, :] = np.float32(kvh + 1) * np.arange(1, 9, dtype=np.float32)
    kc, vc = build_pools(w)
    out = oracle_out(w, kc, vc)
    for h in range(w.num_heads):
        expect = (h // 4 + 1) * np.arange(1, 9, dtype=np.float64)
        np.testing.assert_allclose(out[:, h], np.broadcast_to(expect, out[:, h].shape),
                                   rtol=1e-14, atol=0)


@pytest.mark.parametrize("BS", [8, 16, 32])
def test_needle_sweep_every_position(BS):
    """One key aligned with the query (logit 60 above the rest) at every position,
    including the last partial block: the output is that position's V row."""
    L = 2 * BS + 5
    w = tiny(dtype="f32", lens=(L,), Hq=1, Hkv=1, D=8, BS=BS, scale=1.0)
    q = np.zeros(8, dtype=np.float32)
    q[0] = 1.0
    w.query[0, 0] = q
    for pos in range(L):
        w.rec_key[:] = 0.0
        w.rec_key[w.seq_records[0][pos], 0, 0] = 60.0
        kc, vc = build_pools(w)
        out = oracle_out(w, kc, vc)
        v = w.rec_value[w.seq_records[0][pos], 0].astype(np.float64)
        np.testing.assert_allclose(out[0, 0], v, rtol=1e-20, atol=1e-20)


def test_two_tokens_is_logistic_interpolation():
    w = tiny(dtype="f32", lens=(2, 2, 2), Hq=2, Hkv=2, D=8, scale=0.7)
    kc, vc = build_pools(w)
    out = oracle_out(w, kc, vc)
    for s in range(w.num_seqs):
        r = w.seq_records[s]
        for h in range(w.num_heads):
            q = w.query[s, h].astype(np.float64)
            z0 = 0.7 * (w.rec_key[r[0], h].astype(np.float64) @ q)
            z1 = 0.7 * (w.rec_key[r[1], h].astype(np.float64) @ q)
            v0 = w.rec_value[r[0], h].astype(np.float64)
            v1 = w.rec_value[r[1], h].astype(np.float64)
            np.testing.assert_allclose(out[s, h], v1 + scipy.special.expit(z0 - z1) * (v0 - v1),
                                       rtol=1e-12, atol=1e-14)


def test_empty_sequence_gives_zeros():
    w = tiny(dtype="f32", lens=(4,))
    kc, vc = build_pools(w)
    lens = np.array([0], dtype=np.int32)
    out = oracle.paged_attention(w.query, w.block_table, lens, kc, vc, w.scale, "f32")
    assert np.array_equal(out, np.zeros_like(out))


# ---------------------------------------------------------------------------
# invariances the pages state
# ---------------------------------------------------------------------------
def test_physical_block_permutation_is_bit_invariant():
    """Blocks may sit anywhere in the pool: relabel every physical block."""
    w = tiny(dtype="bf16", BS=8, lens=(3, 19, 40))
    kc, vc = build_pools(w)
    ref = oracle_out(w, kc, vc)
    perm = np.random.default_rng(9).permutation(w.num_blocks)     # old id -> new id
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    table2 = perm[w.block_table].astype(np.int32)
    out = oracle.paged_attention(w.query, table2, w.context_lens, kc2, vc2, w.scale, w.dtype)
    assert np.array_equal(out, ref)


def test_shared_prefix_equals_private_copies_bitwise():
    w = make_workload(name="share", context_lens=[40, 57, 33], num_heads=4, num_kv_heads=2,
                      head_dim=16, block_size=8, dtype="bf16", seed=3, shared_prefix_len=32)
    kc, vc = build_pools(w)
    shared = w.block_table[:, :4]
    assert (shared == shared[0]).all()                 # the prefix is stored once
    ref = oracle_out(w, kc, vc)
    # give every sequence private copies of the prefix blocks
    n_extra = 4 * w.num_seqs
    kc2 = np.concatenate([kc, np.empty((n_extra,) + kc.shape[1:], kc.dtype)])
    vc2 = np.concatenate([vc, np.empty((n_extra,) + vc.shape[1:], vc.dtype)])
    table2 = w.block_table.copy()
    nxt = w.num_blocks
    for s in range(w.num_seqs):
        for j in range(4):
            kc2[nxt], vc2[nxt] = kc[w.block_table[s, j]], vc[w.block_table[s, j]]
            table2[s, j] = nxt
            nxt += 1
    out = oracle.paged_attention(w.query, table2, w.context_lens, kc2, vc2, w.scale, w.dtype)
    assert np.array_equal(out, ref)


def test_block_size_does_not_change_the_result_bitwise():
    base = tiny(dtype="bf16", BS=8, lens=(5, 31, 64))
    outs = []
    for BS in (8, 16, 32):
        w = make_workload(name="bs", context_lens=list(base.context_lens), num_heads=4,
                          num_kv_heads=2, head_dim=16, block_size=BS, dtype="bf16", seed=11)
        # same logical contents as ``base`` in a differently blocked pool
        w.query[:] = base.query
        for s in range(w.num_seqs):
            w.rec_key[w.seq_records[s]] = base.rec_key[base.seq_records[s]]
            w.rec_value[w.seq_records[s]] = base.rec_value[base.seq_records[s]]
        kc, vc = build_pools(w)
        outs.append(oracle_out(w, kc, vc))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_nan_poison_outside_the_sequences_never_leaks():
    w = tiny(dtype="bf16", BS=16, lens=(1, 17, 31))
    kc, vc = build_pools(w)           # every unowned slot holds NaN
    assert np.isnan(oracle.decode(kc, "bf16")).any()
    assert np.isfinite(oracle_out(w, kc, vc)).all()


# ---------------------------------------------------------------------------
# partitions and their log-sum-exp combination
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("P", [1, 7, 32, 512])
def test_partition_combination_equals_direct(P):
    rng = np.random.default_rng(P)
    q = rng.standard_normal((4, 32))
    k = rng.standard_normal((300, 32)) * 3
    v = rng.standard_normal((300, 32))
    direct = oracle.attention_one(q, k, v, 0.25)
    m, l, acc = oracle.partition_stats(q, k, v, 0.25, P)
    assert m.shape[0] == -(-300 // P)
    np.testing.assert_allclose(oracle.combine_partitions(m, l, acc), direct, rtol=1e-13, atol=1e-14)


def test_single_token_partitions_are_logit_one_value():
    rng = np.random.default_rng(2)
    q, k, v = rng.standard_normal((2, 8)), rng.standard_normal((5, 8)), rng.standard_normal((5, 8))
    m, l, acc = oracle.partition_stats(q, k, v, 0.5, 1)
    np.testing.assert_allclose(m, 0.5 * (k @ q.T), rtol=1e-15)
    assert np.array_equal(l, np.ones_like(l))
    assert np.array_equal(acc, np.broadcast_to(v[:, None, :], acc.shape))


def test_one_partition_covering_everything_is_softmax_numerator_and_denominator():
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((3, 16)), rng.standard_normal((40, 16)), rng.standard_normal((40, 16))
    m, l, acc = oracle.partition_stats(q, k, v, 0.2, 64)
    z = 0.2 * (k @ q.T)
    np.testing.assert_allclose(m[0], z.max(axis=0), rtol=1e-15)
    np.testing.assert_allclose(acc[0] / l[0][:, None], scipy.special.softmax(z, axis=0).T @ v,
                               rtol=1e-12)


# ---------------------------------------------------------------------------
# copy-on-write block copies
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,BS,D", [("f32", 8, 16), ("bf16", 16, 64), ("bf16", 32, 128)])
def test_copy_blocks_matches_element_loop(dtype, BS, D):
    rng = np.random.default_rng(40)
    NB, Hkv = 12, 2
    kc, vc = oracle.empty_pools(NB, Hkv, D, BS, dtype, fill="zero")
    if dtype == "bf16":
        kc[:] = rng.integers(0, 1 << 16, size=kc.shape, dtype=np.uint16)
        vc[:] = rng.integers(0, 1 << 16, size=vc.shape, dtype=np.uint16)
    else:
        kc[:] = rng.standard_normal(kc.shape, dtype=np.float32)
        vc[:] = rng.standard_normal(vc.shape, dtype=np.float32)
    pairs = np.array([[3, 7], [3, 9], [0, 11], [5, 2]], dtype=np.int64)
    k2, v2 = oracle.copy_blocks(kc, vc, pairs)
    kf, vf = kc.reshape(NB, -1), vc.reshape(NB, -1)
    k2f, v2f = k2.reshape(NB, -1), v2.reshape(NB, -1)
    dsts = {int(d): int(s) for s, d in pairs}
    for b in range(NB):
        sb = dsts.get(b, b)
        for i in range(kf.shape[1]):
            assert kf[sb, i].tobytes() == k2f[b, i].tobytes()
            assert vf[sb, i].tobytes() == v2f[b, i].tobytes()


def test_copy_blocks_rejects_overlapping_pairs():
    kc, vc = oracle.empty_pools(8, 1, 16, 8, "f32")
    with pytest.raises(AssertionError):
        oracle.copy_blocks(kc, vc, np.array([[1, 2], [3, 2]]))
    with pytest.raises(AssertionError):
        oracle.copy_blocks(kc, vc, np.array([[1, 2], [2, 4]]))


def test_copy_blocks_reproduces_the_copy_on_write_records():
    """Parallel sampling: the pools before the copies plus copy_blocks equal the pools
    that hold the workload's per-token duplicate records (NaN where nothing is stored)."""
    w = make_config(3, variant="parallel-sampling")
    assert len(w.cow_pairs) > 0
    keep_after = np.setdiff1d(np.arange(len(w.rec_slot)), w.new_records)
    keep_before = np.setdiff1d(keep_after, w.cow_records)
    kb, vb = oracle.empty_pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, w.dtype)
    oracle.reshape_and_cache(w.rec_key[keep_before], w.rec_value[keep_before],
                             w.rec_slot[keep_before], kb, vb, inplace=True)
    ka, va = oracle.empty_pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, w.dtype)
    oracle.reshape_and_cache(w.rec_key[keep_after], w.rec_value[keep_after],
                             w.rec_slot[keep_after], ka, va, inplace=True)
    kc, vc = oracle.copy_blocks(kb, vb, w.cow_pairs)
    assert np.array_equal(kc, ka) and np.array_equal(vc, va)


# ---------------------------------------------------------------------------
# swapping blocks between the HBM pool and a host pool
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_swap_blocks_matches_element_loop(dtype):
    rng = np.random.default_rng(90)
    Hkv, D, BS = 2, 32, 8
    shape_k = lambda nb: (nb, Hkv, BS, D)
    np_t = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dtype]

    def pool(nb):
        k = rng.integers(0, 255, size=shape_k(nb)).astype(np_t)
        X = min(16 // np.dtype(np_t).itemsize, BS)
        v = rng.integers(0, 255, size=(nb, Hkv, BS // X, D, X)).astype(np_t)
        return k, v

    sk, sv = pool(10)
    dk, dv = pool(6)                       # a smaller destination pool
    sk0, sv0, dk0, dv0 = sk.copy(), sv.copy(), dk.copy(), dv.copy()
    pairs = np.array([[9, 0], [2, 5], [2, 3], [7, 1]], dtype=np.int64)
    k2, v2 = oracle.swap_blocks(sk, sv, dk, dv, pairs)
    assert np.array_equal(sk, sk0) and np.array_equal(sv, sv0)          # inputs untouched
    assert np.array_equal(dk, dk0) and np.array_equal(dv, dv0)
    dsts = {int(d): int(s_) for s_, d in pairs}
    for b in range(6):
        for pool_new, pool_old, src in ((k2, dk, sk), (v2, dv, sv)):
            flat_new, flat_old = pool_new.reshape(6, -1), pool_old.reshape(6, -1)
            flat_src = src.reshape(10, -1)
            for i in range(flat_new.shape[1]):
                want = flat_src[dsts[b], i] if b in dsts else flat_old[b, i]
                assert flat_new[b, i].tobytes() == want.tobytes()


def test_swap_blocks_rejects_bad_pairs():
    k, v = oracle.empty_pools(8, 1, 16, 8, "f32")
    hk, hv = oracle.empty_pools(4, 1, 16, 8, "f32")
    with pytest.raises(AssertionError):
        oracle.swap_blocks(k, v, hk, hv, np.array([[1, 2], [3, 2]]))      # same destination
    with pytest.raises(AssertionError):
        oracle.swap_blocks(k, v, hk, hv, np.array([[1, 4]]))              # past the host pool
    with pytest.raises(AssertionError):
        oracle.swap_blocks(k, v, hk, hv, np.array([[8, 0]]))              # past the HBM pool


def test_swap_out_and_back_in_keeps_every_result():
    """Preempt a quarter of the sequences: their blocks go to a compact host pool, the HBM
    blocks are reused (NaN-filled here), and on resumption the blocks come back into other
    free HBM blocks with the tables rewritten.  Every sequence's attention is unchanged, bit
    for bit, and nothing but the chosen blocks moved."""
    w = tiny("bf16", lens=(5, 40, 17, 64, 33, 90, 8, 71), Hq=8, Hkv=2, D=32, BS=8, seed=91,
             pool_factor=2.0)
    kc, vc = build_pools(w)
    before = oracle_out(w, kc, vc)
    victims = [1, 3]
    nblk = {s: -(-int(w.context_lens[s]) // w.block_size) for s in victims}
    out_pairs, host = [], 0
    for s in victims:
        for i in range(nblk[s]):
            out_pairs.append([int(w.block_table[s, i]), host])
            host += 1
    out_pairs = np.array(out_pairs, dtype=np.int64)
    hk, hv = oracle.empty_pools(host, w.num_kv_heads, w.head_dim, w.block_size, w.dtype)
    hk, hv = oracle.swap_blocks(kc, vc, hk, hv, out_pairs)
    kc2, vc2 = kc.copy(), vc.copy()
    nan = np.uint16(0x7FC0)
    kc2[out_pairs[:, 0]] = nan                        # the freed blocks get reused
    vc2[out_pairs[:, 0]] = nan
    used = {int(b) for s in range(w.num_seqs) for b in
            w.block_table[s, :-(-int(w.context_lens[s]) // w.block_size)]}
    free = [b for b in range(w.num_blocks) if b not in used]
    assert len(free) >= host
    in_pairs = np.stack([np.arange(host), np.array(free[:host])], axis=1).astype(np.int64)
    kc2, vc2 = oracle.swap_blocks(hk, hv, kc2, vc2, in_pairs)
    table = w.block_table.copy()
    h = 0
    for s in victims:
        for i in range(nblk[s]):
            table[s, i] = free[h]
            h += 1
    w2 = w.__class__(**{**w.__dict__, "block_table": table})
    after = oracle_out(w2, kc2, vc2)
    assert np.array_equal(before, after)
    # only the chosen blocks changed
    changed = {int(b) for b in range(w.num_blocks)
               if not (np.array_equal(kc2[b], kc[b]) and np.array_equal(vc2[b], vc[b]))}
    assert changed == set(out_pairs[:, 0].tolist()) | set(free[:host])


# ---------------------------------------------------------------------------
# paged prefill (causal chunks over the paged context)
# ---------------------------------------------------------------------------
from workloads import make_prefill  # noqa: E402


def test_prefill_of_one_token_is_the_decode():
    w = tiny("bf16", lens=(1, 9, 30, 64), Hq=8, Hkv=2, D=32, BS=8, seed=60)
    pb = make_prefill(w, [1, 1, 1, 1], 60)
    kc, vc = build_pools(w)
    a = oracle.paged_prefill(pb.query, pb.query_start_loc, w.block_table, w.context_lens, kc, vc,
                             w.scale, w.dtype)
    b = oracle.paged_attention(pb.query, w.block_table, w.context_lens, kc, vc, w.scale, w.dtype)
    # the two take their products in other orders (a masked matrix product against one
    # query row at a time), so they agree to float64 rounding, not bit for bit
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_matches_causal_bruteforce(dtype):
    w = tiny(dtype, lens=(3, 17, 26), Hq=4, Hkv=2, D=16, BS=8, seed=61)
    pb = make_prefill(w, [3, 5, 9], 61)
    kc, vc = build_pools(w)
    got = oracle.paged_prefill(pb.query, pb.query_start_loc, w.block_table, w.context_lens, kc, vc,
                               w.scale, dtype)
    g = w.num_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        r0, r1 = pb.query_start_loc[s], pb.query_start_loc[s + 1]
        L = int(w.context_lens[s])
        for i in range(r1 - r0):
            p = L - (r1 - r0) + i
            recs = w.seq_records[s][:p + 1]
            for h in range(w.num_heads):
                K = torch_decode(w.rec_key[recs][:, h // g], dtype)
                V = torch_decode(w.rec_value[recs][:, h // g], dtype)
                q = torch_decode(pb.query[r0 + i, h], dtype)
                z = [w.scale * math.fsum(float(q[d]) * float(K[t, d]) for d in range(K.shape[1]))
                     for t in range(p + 1)]
                m = max(z)
                e = [math.exp(zt - m) for zt in z]
                den = math.fsum(e)
                ref = [math.fsum(e[t] * float(V[t, d]) for t in range(p + 1)) / den
                       for d in range(K.shape[1])]
                np.testing.assert_allclose(got[r0 + i, h], ref, rtol=1e-12, atol=1e-13)


def test_prefill_chunk_split_in_two_calls_agrees():
    """A chunk of n tokens equals its first half (context shortened to end there) followed
    by its second half: each token only sees positions up to its own."""
    w = tiny("bf16", lens=(40, 64, 25), Hq=8, Hkv=2, D=32, BS=16, seed=62)
    n = np.array([12, 20, 8])
    pb = make_prefill(w, n, 62)
    kc, vc = build_pools(w)
    whole = oracle.paged_prefill(pb.query, pb.query_start_loc, w.block_table, w.context_lens,
                                 kc, vc, w.scale, w.dtype)
    half = n // 2
    rows_a = np.concatenate([np.arange(pb.query_start_loc[s], pb.query_start_loc[s] + half[s])
                             for s in range(3)])
    rows_b = np.concatenate([np.arange(pb.query_start_loc[s] + half[s], pb.query_start_loc[s + 1])
                             for s in range(3)])
    qa = np.concatenate([[0], np.cumsum(half)]).astype(np.int32)
    qb = np.concatenate([[0], np.cumsum(n - half)]).astype(np.int32)
    part_a = oracle.paged_prefill(pb.query[rows_a], qa, w.block_table, w.context_lens - (n - half),
                                  kc, vc, w.scale, w.dtype)
    part_b = oracle.paged_prefill(pb.query[rows_b], qb, w.block_table, w.context_lens, kc, vc,
                                  w.scale, w.dtype)
    # the calls sum over key ranges of other lengths, so they agree to float64 rounding
    np.testing.assert_allclose(whole[rows_a], part_a, rtol=0, atol=1e-13)
    np.testing.assert_allclose(whole[rows_b], part_b, rtol=0, atol=1e-13)


def test_prefill_is_block_permutation_invariant():
    w = tiny("bf16", lens=(33, 50), Hq=4, Hkv=4, D=16, BS=8, seed=63)
    pb = make_prefill(w, [10, 30], 63)
    kc, vc = build_pools(w)
    a = oracle.paged_prefill(pb.query, pb.query_start_loc, w.block_table, w.context_lens, kc, vc,
                             w.scale, w.dtype)
    perm = np.random.default_rng(3).permutation(w.num_blocks)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    b = oracle.paged_prefill(pb.query, pb.query_start_loc, perm[w.block_table], w.context_lens,
                             kc2, vc2, w.scale, w.dtype)
    assert np.array_equal(a, b)


def test_prefill_chunks_are_the_last_positions():
    w = tiny("bf16", lens=(5, 9, 1), Hq=4, Hkv=2, D=16, BS=8, seed=64)
    pb = make_prefill(w, [2, 9, 3], 64)
    assert list(pb.query_start_loc) == [0, 2, 11, 12]        # the last chunk is clipped to L
    assert list(pb.chunk_records[:2]) == list(w.seq_records[0][3:5])
    assert list(pb.chunk_records[2:11]) == list(w.seq_records[1])
