"""GPU parity: the HIP library (called through its C ABI) against the CPU oracle.

* reshape_and_cache and the block gather: bit-exact;
* paged attention: f32 max |err| <= 1e-5; bf16 max |err| <= 1e-2 where |ref| < 4
  (from 4 up half a bf16 ulp of the output exceeds 1e-2) and relative error <= 2e-2
  where |ref| >= 1e-2;
* the invariances the pages state hold bit for bit on the GPU (physical block
  permutation, shared blocks vs private copies, block size), and the result
  is deterministic.
Pools are NaN everywhere no token was written, and block-table entries past a
sequence's end hold ids of other sequences' blocks, so any stray read shows.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_425_amd as pk
from tests.gpu_util import bits, check_close, to_dev, to_f64, upload_inputs
from tests.helpers import build_pools, oracle_out, prefill_reference
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def run_gpu(w, kc_np, vc_np, partition_size=0, out_dtype_check=True):
    inp = upload_inputs(w, DEV)
    kc, vc = to_dev(kc_np, w.dtype, DEV), to_dev(vc_np, w.dtype, DEV)
    out = pk.paged_attention(inp["query"], inp["block_table"], inp["context_lens"], kc, vc,
                             w.scale, max_context_len=w.max_context_len,
                             partition_size=partition_size)
    torch.cuda.synchronize()
    return out


def tiny(dtype, lens, Hq, Hkv, D, BS, seed=0, **kw):
    return make_workload(name="tiny", context_lens=list(lens), num_heads=Hq, num_kv_heads=Hkv,
                         head_dim=D, block_size=BS, dtype=dtype, seed=seed, **kw)


# ---------------------------------------------------------------------------
# write path and gather: bit-exact
# ---------------------------------------------------------------------------
CACHE_CASES = [("cfg0", lambda: make_config(0)),
               ("bf16-bs8", lambda: tiny("bf16", (1, 9, 40, 64), 8, 2, 128, 8)),
               ("bf16-bs32-d64", lambda: tiny("bf16", (3, 33, 95), 4, 4, 64, 32)),
               ("f32-bs16-d128", lambda: tiny("f32", (17, 2, 50), 8, 4, 128, 16)),
               ("cfg2-bs16", lambda: make_config(2, block_size=16))]


@pytest.mark.parametrize("name,make", CACHE_CASES, ids=[c[0] for c in CACHE_CASES])
def test_reshape_and_cache_bit_exact(name, make):
    w = make()
    say(f"reshape_and_cache {name} T={len(w.new_records)}")
    kc_np, vc_np = build_pools(w, include_new=False)
    new = w.new_records
    slots = w.rec_slot[new].copy()
    slots[0] = -1                                   # padding entry: no write
    ref_k, ref_v = oracle.reshape_and_cache(w.rec_key[new], w.rec_value[new], slots, kc_np, vc_np)
    kc, vc = to_dev(kc_np, w.dtype, DEV), to_dev(vc_np, w.dtype, DEV)
    pk.reshape_and_cache(to_dev(w.rec_key[new], w.dtype, DEV), to_dev(w.rec_value[new], w.dtype, DEV),
                         torch.from_numpy(slots).to(DEV), kc, vc)
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc), ref_k.view(bits(kc).dtype))
    assert np.array_equal(bits(vc), ref_v.view(bits(vc).dtype))


@pytest.mark.parametrize("name,make", CACHE_CASES[:4] + [("cfg1", lambda: make_config(1))],
                         ids=[c[0] for c in CACHE_CASES[:4]] + ["cfg1"])
def test_gather_kv_bit_exact(name, make):
    w = make()
    say(f"gather_kv {name}")
    kc_np, vc_np = build_pools(w)
    ref_k, ref_v = oracle.gather_kv(w.block_table, w.context_lens, kc_np, vc_np)
    offs = np.concatenate([[0], np.cumsum(w.context_lens.astype(np.int64))[:-1]])
    inp = upload_inputs(w, DEV)
    k, v = pk.gather_kv(inp["block_table"], inp["context_lens"], to_dev(kc_np, w.dtype, DEV),
                        to_dev(vc_np, w.dtype, DEV), seq_offsets=torch.from_numpy(offs).to(DEV),
                        total_tokens=int(w.context_lens.sum()), max_context_len=w.max_context_len)
    torch.cuda.synchronize()
    assert np.array_equal(bits(k), ref_k.view(bits(k).dtype))
    assert np.array_equal(bits(v), ref_v.view(bits(v).dtype))


# ---------------------------------------------------------------------------
# attention on the named workloads: the full step (scatter the new tokens, decode)
# ---------------------------------------------------------------------------
STEP_CASES = [("cfg0", lambda: make_config(0)),
              ("cfg1", lambda: make_config(1)),
              ("cfg2-bs8", lambda: make_config(2, block_size=8)),
              ("cfg2-bs16", lambda: make_config(2, block_size=16)),
              ("cfg2-bs32", lambda: make_config(2, block_size=32)),
              ("cfg3-prefix", lambda: make_config(3)),
              ("cfg3-parallel-sampling", lambda: make_config(3, variant="parallel-sampling")),
              ("cfg4", lambda: make_config(4))]


@pytest.mark.parametrize("name,make", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_decode_step_matches_oracle(name, make):
    w = make()
    part = w.partition_size or 0
    say(f"decode step {name} S={w.num_seqs} maxlen={w.max_context_len} BS={w.block_size} P={part}")
    hist_k, hist_v = build_pools(w, include_new=False)
    ref_k, ref_v = oracle.reshape_and_cache(w.rec_key[w.new_records], w.rec_value[w.new_records],
                                            w.rec_slot[w.new_records], hist_k, hist_v)
    inp = upload_inputs(w, DEV)
    kc, vc = to_dev(hist_k, w.dtype, DEV), to_dev(hist_v, w.dtype, DEV)
    new = w.new_records
    pk.reshape_and_cache(to_dev(w.rec_key[new], w.dtype, DEV), to_dev(w.rec_value[new], w.dtype, DEV),
                         torch.from_numpy(w.rec_slot[new]).to(DEV), kc, vc)
    out = pk.paged_attention(inp["query"], inp["block_table"], inp["context_lens"], kc, vc,
                             w.scale, max_context_len=w.max_context_len, partition_size=part)
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc), ref_k.view(bits(kc).dtype))
    assert np.array_equal(bits(vc), ref_v.view(bits(vc).dtype))
    ref = oracle_out(w, ref_k, ref_v)
    stats = check_close(to_f64(out), ref, w.dtype, name)
    say(f"  {name}: {stats}")


# ---------------------------------------------------------------------------
# fused step (pa_decode_step): same caches and output as the two calls
# ---------------------------------------------------------------------------
FUSED_CASES = [("cfg0", lambda: make_config(0), 0),
               ("cfg1", lambda: make_config(1), 0),
               ("cfg2-bs8", lambda: make_config(2, block_size=8), 0),
               ("cfg2-bs32-P1024", lambda: make_config(2, block_size=32), 1024),
               ("cfg3-prefix", lambda: make_config(3), 0),
               ("cfg3-parallel-sampling", lambda: make_config(3, variant="parallel-sampling"), 0),
               ("cfg4", lambda: make_config(4), 512),
               ("tiny-f32-P64", lambda: tiny("f32", LENS, 8, 2, 128, 16, seed=31), 64),
               ("tiny-bf16-bs8-P128", lambda: tiny("bf16", LENS, 16, 2, 64, 8, seed=32), 128),
               ("tiny-bf16-paired", lambda: tiny("bf16", LENS, 16, 2, 64, 32, seed=33), 0),
               ("many-seqs-unpaired", lambda: tiny("bf16", np.random.default_rng(34).integers(
                   1, 90, size=600), 8, 2, 128, 16, seed=34), 128),
               ("long-tail-P512", lambda: tiny("bf16", long_tail_lens(37), 32, 8, 128, 16,
                                               seed=37), 512),
               ("long-tail-f32-bs8-P64", lambda: tiny("f32", long_tail_lens(38), 32, 8, 64, 8,
                                                      seed=38), 64)]


def fused_inputs(w):
    """The new token of every sequence: its record at position L - 1."""
    new = np.array([w.seq_records[s][-1] for s in range(w.num_seqs)], dtype=np.int64)
    return new, w.rec_slot[new].copy()


@pytest.mark.parametrize("name,make,part", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_decode_step_matches_two_calls_and_oracle(name, make, part):
    w = make()
    say(f"fused step {name} S={w.num_seqs} BS={w.block_size} P={part}")
    new, slots = fused_inputs(w)
    assert set(new.tolist()) == set(w.new_records.tolist())
    hist_k, hist_v = build_pools(w, include_new=False)
    ref_k, ref_v = oracle.reshape_and_cache(w.rec_key[new], w.rec_value[new], slots, hist_k, hist_v)
    ref = oracle_out(w, ref_k, ref_v)
    inp = upload_inputs(w, DEV)
    key, val = to_dev(w.rec_key[new], w.dtype, DEV), to_dev(w.rec_value[new], w.dtype, DEV)
    slot_t = torch.from_numpy(slots).to(DEV)
    kc, vc = to_dev(hist_k, w.dtype, DEV), to_dev(hist_v, w.dtype, DEV)
    out = pk.decode_step(inp["query"], key, val, slot_t, inp["block_table"], inp["context_lens"],
                         kc, vc, w.scale, max_context_len=w.max_context_len, partition_size=part)
    kc2, vc2 = to_dev(hist_k, w.dtype, DEV), to_dev(hist_v, w.dtype, DEV)
    pk.reshape_and_cache(key, val, slot_t, kc2, vc2)
    out2 = pk.paged_attention(inp["query"], inp["block_table"], inp["context_lens"], kc2, vc2,
                              w.scale, max_context_len=w.max_context_len, partition_size=part)
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc), ref_k.view(bits(kc).dtype))
    assert np.array_equal(bits(vc), ref_v.view(bits(vc).dtype))
    assert np.array_equal(bits(out), bits(out2))
    stats = check_close(to_f64(out), ref, w.dtype, name)
    say(f"  {name}: {stats}")


def test_fused_decode_step_skips_negative_slots():
    """A negative slot writes nothing: the cache keeps what it held."""
    w = tiny("bf16", (5, 40, 17, 64), 8, 2, 128, 16, seed=35)
    kc_np, vc_np = build_pools(w)                     # every token already stored
    new, slots = fused_inputs(w)
    slots[1] = -1
    key = w.rec_key[new].copy()
    key[1] = 0                                        # would change the result if written
    inp = upload_inputs(w, DEV)
    kc, vc = to_dev(kc_np, w.dtype, DEV), to_dev(vc_np, w.dtype, DEV)
    say("fused step with a negative slot")
    out = pk.decode_step(inp["query"], to_dev(key, w.dtype, DEV),
                         to_dev(w.rec_value[new], w.dtype, DEV), torch.from_numpy(slots).to(DEV),
                         inp["block_table"], inp["context_lens"], kc, vc, w.scale,
                         max_context_len=w.max_context_len)
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc), kc_np.view(np.uint16))
    check_close(to_f64(out), oracle_out(w, kc_np, vc_np), "bf16", "negative-slot")


def test_cfg1_shape_in_f32_is_exact_to_1e5():
    """The Llama-3-8B decode shape with f32 data: a tighter check of indexing."""
    base = make_config(1)
    w = make_workload(name="cfg1-f32", context_lens=base.context_lens, num_heads=32, num_kv_heads=8,
                      head_dim=128, block_size=16, dtype="f32", seed=1)
    say("decode cfg1 shape f32")
    kc, vc = build_pools(w)
    check_close(to_f64(run_gpu(w, kc, vc)), oracle_out(w, kc, vc), "f32", "cfg1-f32")


# ---------------------------------------------------------------------------
# small shapes: every compiled variant, ragged lengths, several partition sizes
# ---------------------------------------------------------------------------
LENS = (1, 2, 7, 31, 32, 33, 63, 64, 65, 130, 257, 511, 700)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("BS", [8, 16, 32])
@pytest.mark.parametrize("g", [1, 4, 8])
def test_variants_ragged(dtype, D, BS, g):
    Hkv = 2
    w = tiny(dtype, LENS, g * Hkv, Hkv, D, BS, seed=D + BS + g, scale=0.6 / np.sqrt(D) * 4)
    kc, vc = build_pools(w)
    ref = oracle_out(w, kc, vc)
    for part in (0, 64, 128, 768):
        say(f"variant {dtype} D={D} BS={BS} g={g} P={part}")
        check_close(to_f64(run_gpu(w, kc, vc, part)), ref, dtype, f"{dtype}/{D}/{BS}/{g}/{part}")


def test_paired_mode_odd_count_and_uneven_pairs():
    """One partition per sequence, few sequences: workgroups pair the r-th longest with the
    r-th shortest sequence; with an odd count the middle sequence runs alone."""
    w = tiny("bf16", (700, 3, 64, 1, 333, 129, 40), 32, 8, 128, 16, seed=21)
    kc, vc = build_pools(w)
    say("paired mode, 7 sequences")
    check_close(to_f64(run_gpu(w, kc, vc, 768)), oracle_out(w, kc, vc), "bf16", "paired-odd")


def long_tail_lens(seed: int) -> np.ndarray:
    """64 sequences: 58 short, 6 long, three at exact multiples of 512."""
    rng = np.random.default_rng(seed)
    lens = np.concatenate([rng.integers(1, 300, size=58), rng.integers(2000, 4500, size=6)])
    lens[3], lens[10], lens[60] = 512, 1024, 4096
    return rng.permutation(lens)


@pytest.mark.parametrize("dtype,D,BS", [("bf16", 128, 16), ("bf16", 64, 8), ("f32", 64, 32),
                                        ("f32", 128, 16)])
def test_full_batch_with_a_long_tail(dtype, D, BS):
    """A batch whose (sequence, kv head) pairs alone fill the GPU (64 x 8), with a few
    sequences far longer than the partition, an empty one and lengths at exact multiples of
    the partition: partitions from 64 to 2048 tokens, merged by the log-sum-exp reduce."""
    lens = long_tail_lens(50 + D + BS)
    w = tiny(dtype, lens, 32, 8, D, BS, seed=51 + D + BS)
    kc, vc = build_pools(w)
    w.context_lens = w.context_lens.copy()
    w.context_lens[7] = 0
    ref = oracle_out(w, kc, vc)
    for part in (64, 512, 1024, 2048):
        say(f"long tail {dtype} D={D} BS={BS} P={part}")
        out = run_gpu(w, kc, vc, part)
        assert np.array_equal(bits(out)[7], np.zeros_like(bits(out)[7]))
        check_close(to_f64(out), ref, dtype, f"long-tail/{dtype}/{D}/{BS}/{part}")


def test_many_sequences_single_partition_unpaired():
    """More sequences than the in-kernel ordering handles: one workgroup per
    (kv head, sequence) with no pairing."""
    rng = np.random.default_rng(22)
    w = tiny("bf16", rng.integers(1, 100, size=600), 8, 2, 128, 16, seed=22)
    kc, vc = build_pools(w)
    say("600 sequences, one partition each")
    check_close(to_f64(run_gpu(w, kc, vc, 128)), oracle_out(w, kc, vc), "bf16", "unpaired")


def test_group_of_sixteen_f32():
    w = tiny("f32", (5, 40, 129), 32, 2, 64, 16, seed=3)
    kc, vc = build_pools(w)
    say("f32 g=16")
    check_close(to_f64(run_gpu(w, kc, vc, 64)), oracle_out(w, kc, vc), "f32", "g16")


# ---------------------------------------------------------------------------
# edge cases and invariances
# ---------------------------------------------------------------------------
def test_empty_and_single_token_sequences():
    w = tiny("bf16", (1, 5, 1, 40), 8, 2, 128, 16, seed=4)
    kc, vc = build_pools(w)
    lens = w.context_lens.copy()
    lens[2] = 0
    w.context_lens = lens
    say("edge L=0 / L=1")
    out = run_gpu(w, kc, vc)
    assert np.array_equal(bits(out)[2], np.zeros_like(bits(out)[2]))
    # one token: the weight is exactly 1, so the output is that token's V row
    g = 4
    v0 = w.rec_value[w.seq_records[0][0]]
    for h in range(8):
        assert np.array_equal(bits(out)[0, h], v0[h // g])
    check_close(to_f64(out), oracle_out(w, kc, vc), "bf16", "edge")


def test_maximum_context_fills_the_table():
    BS, MB = 16, 40
    w = tiny("bf16", (MB * BS, MB * BS - 1, 3), 32, 8, 128, BS, seed=6, max_blocks_per_seq=MB)
    kc, vc = build_pools(w)
    ref = oracle_out(w, kc, vc)
    for part in (0, 64, 8192):
        say(f"max context P={part}")
        check_close(to_f64(run_gpu(w, kc, vc, part)), ref, "bf16", f"maxctx/{part}")


def test_deterministic_and_block_permutation_invariant_bitwise():
    w = make_config(1)
    kc, vc = build_pools(w)
    say("determinism + permutation cfg1")
    a = bits(run_gpu(w, kc, vc))
    b = bits(run_gpu(w, kc, vc))
    assert np.array_equal(a, b)
    perm = np.random.default_rng(9).permutation(w.num_blocks)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    w.block_table = perm[w.block_table].astype(np.int32)
    assert np.array_equal(bits(run_gpu(w, kc2, vc2)), a)


def test_shared_prefix_equals_private_copies_bitwise():
    w = make_config(3)
    kc, vc = build_pools(w)
    say("sharing cfg3")
    shared = bits(run_gpu(w, kc, vc))
    npre = 1024 // w.block_size
    extra = npre * w.num_seqs
    kc2 = np.concatenate([kc, np.empty((extra,) + kc.shape[1:], kc.dtype)])
    vc2 = np.concatenate([vc, np.empty((extra,) + vc.shape[1:], vc.dtype)])
    table = w.block_table.copy()
    nxt = w.num_blocks
    for s in range(w.num_seqs):
        for j in range(npre):
            kc2[nxt], vc2[nxt] = kc[table[s, j]], vc[table[s, j]]
            table[s, j] = nxt
            nxt += 1
    w.block_table, w.num_blocks = table, nxt
    assert np.array_equal(bits(run_gpu(w, kc2, vc2)), shared)


def test_block_size_does_not_change_the_result_bitwise():
    outs = []
    base = tiny("bf16", (5, 31, 64, 300, 777), 32, 8, 128, 8, seed=12)
    for BS in (8, 16, 32):
        w = tiny("bf16", base.context_lens, 32, 8, 128, BS, seed=13)
        w.query[:] = base.query
        for s in range(w.num_seqs):
            w.rec_key[w.seq_records[s]] = base.rec_key[base.seq_records[s]]
            w.rec_value[w.seq_records[s]] = base.rec_value[base.seq_records[s]]
        kc, vc = build_pools(w)
        say(f"block size invariance BS={BS}")
        outs.append(bits(run_gpu(w, kc, vc, 256)))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_partition_sizes_agree_with_each_other():
    w = make_config(4)
    w.context_lens = w.context_lens[:4].copy()
    w.block_table = w.block_table[:4].copy()
    w.query = w.query[:4].copy()
    w.seq_records = w.seq_records[:4]
    w.num_seqs = 4
    kc, vc = build_pools(w)
    ref = oracle_out(w, kc, vc)
    for part in (512, 1024, 4096, 0):
        say(f"cfg4 subset P={part}")
        check_close(to_f64(run_gpu(w, kc, vc, part)), ref, "bf16", f"cfg4/{part}")


def test_binding_rejects_bad_inputs():
    w = make_config(0)
    kc, vc = build_pools(w)
    inp = upload_inputs(w, DEV)
    kd, vd = to_dev(kc, "f32", DEV), to_dev(vc, "f32", DEV)
    with pytest.raises(TypeError):
        pk.paged_attention(inp["query"].to(torch.bfloat16), inp["block_table"], inp["context_lens"],
                           kd, vd, 0.1, max_context_len=64)
    with pytest.raises(ValueError):
        pk.paged_attention(inp["query"], inp["block_table"], inp["context_lens"], kd, vd, 0.1,
                           max_context_len=65)
    with pytest.raises(ValueError):
        pk.paged_attention(inp["query"], inp["block_table"], inp["context_lens"], kd, vd, 0.1,
                           max_context_len=64, partition_size=100)


# ---------------------------------------------------------------------------
# copy-on-write block copies
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,BS,D", [("f32", 8, 64), ("f32", 32, 128), ("bf16", 16, 128),
                                        ("bf16", 8, 64), ("bf16", 32, 128)])
def test_copy_blocks_bit_exact(dtype, BS, D):
    rng = np.random.default_rng(50 + BS + D)
    NB, Hkv = 40, 4
    kc, vc = oracle.empty_pools(NB, Hkv, D, BS, dtype, fill="zero")
    if dtype == "bf16":
        kc[:] = rng.integers(0, 1 << 16, size=kc.shape, dtype=np.uint16)
        vc[:] = rng.integers(0, 1 << 16, size=vc.shape, dtype=np.uint16)
    else:
        kc[:] = rng.standard_normal(kc.shape, dtype=np.float32)
        vc[:] = rng.standard_normal(vc.shape, dtype=np.float32)
    perm = rng.permutation(NB)
    valid = np.stack([perm[:10], perm[10:20]], axis=1).astype(np.int64)
    bad = np.array([[-1, perm[30]], [perm[31], NB], [NB + 5, perm[32]]], dtype=np.int64)
    pairs = np.concatenate([valid, bad])
    ref_k, ref_v = oracle.copy_blocks(kc, vc, valid)
    say(f"copy_blocks {dtype} BS={BS} D={D} pairs={len(pairs)}")
    kd, vd = to_dev(kc, dtype, DEV), to_dev(vc, dtype, DEV)
    pk.copy_blocks(kd, vd, torch.from_numpy(pairs).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(bits(kd), ref_k.view(bits(kd).dtype))
    assert np.array_equal(bits(vd), ref_v.view(bits(vd).dtype))


def test_copy_on_write_step_parallel_sampling():
    """Prompts shared by 4 samples: copy the shared partial last blocks, then run the
    fused decode step; caches bit-exact and output within tolerance of the oracle."""
    w = make_config(3, variant="parallel-sampling")
    keep_after = np.setdiff1d(np.arange(len(w.rec_slot)), w.new_records)
    keep_before = np.setdiff1d(keep_after, w.cow_records)
    kb, vb = oracle.empty_pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, w.dtype)
    oracle.reshape_and_cache(w.rec_key[keep_before], w.rec_value[keep_before],
                             w.rec_slot[keep_before], kb, vb, inplace=True)
    ref_k, ref_v = oracle.copy_blocks(kb, vb, w.cow_pairs)
    new, slots = fused_inputs(w)
    ref_k, ref_v = oracle.reshape_and_cache(w.rec_key[new], w.rec_value[new], slots, ref_k, ref_v)
    ref = oracle_out(w, ref_k, ref_v)
    say(f"copy-on-write step: {len(w.cow_pairs)} copies, {w.num_seqs} sequences")
    kd, vd = to_dev(kb, w.dtype, DEV), to_dev(vb, w.dtype, DEV)
    pk.copy_blocks(kd, vd, torch.from_numpy(w.cow_pairs).to(DEV))
    inp = upload_inputs(w, DEV)
    out = pk.decode_step(inp["query"], to_dev(w.rec_key[new], w.dtype, DEV),
                         to_dev(w.rec_value[new], w.dtype, DEV), torch.from_numpy(slots).to(DEV),
                         inp["block_table"], inp["context_lens"], kd, vd, w.scale,
                         max_context_len=w.max_context_len)
    torch.cuda.synchronize()
    assert np.array_equal(bits(kd), ref_k.view(np.uint16))
    assert np.array_equal(bits(vd), ref_v.view(np.uint16))
    check_close(to_f64(out), ref, "bf16", "cow-step")


# ---------------------------------------------------------------------------
# paged prefill
# ---------------------------------------------------------------------------
from workloads import make_prefill, make_prefill_config  # noqa: E402


def run_prefill(w, pb, kc_np, vc_np):
    kc, vc = to_dev(kc_np, w.dtype, DEV), to_dev(vc_np, w.dtype, DEV)
    out = pk.paged_prefill(to_dev(pb.query, w.dtype, DEV),
                           torch.from_numpy(pb.query_start_loc).to(DEV),
                           torch.from_numpy(w.block_table).to(DEV),
                           torch.from_numpy(w.context_lens).to(DEV), kc, vc, w.scale,
                           max_query_len=pb.max_query_len)
    torch.cuda.synchronize()
    return out


PREFILL_LENS = (1, 5, 31, 33, 64, 97, 200, 300)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("BS", [8, 16, 32])
@pytest.mark.parametrize("g", [1, 4, 8])
def test_prefill_variants_ragged(dtype, D, BS, g):
    Hkv = 2
    w = tiny(dtype, PREFILL_LENS, g * Hkv, Hkv, D, BS, seed=70 + D + BS + g,
             scale=0.6 / np.sqrt(D) * 4)
    chunks = [1, 5, 17, 33, 64, 40, 200, 129]      # whole context, partial tiles, one token
    pb = make_prefill(w, chunks, 70)
    kc, vc = build_pools(w)
    say(f"prefill {dtype} D={D} BS={BS} g={g} T={len(pb.chunk_records)}")
    got = run_prefill(w, pb, kc, vc)
    ref = oracle.paged_prefill(pb.query, pb.query_start_loc, w.block_table, w.context_lens,
                               kc, vc, w.scale, dtype)
    check_close(to_f64(got), ref, dtype, f"prefill/{dtype}/{D}/{BS}/{g}")


@pytest.mark.parametrize("D,BS,g", [(128, 16, 4), (64, 8, 1), (128, 32, 2)])
def test_prefill_with_large_v_magnitudes(D, BS, g):
    """Large V magnitudes: V of every third physical block scaled by 16 (exact in bf16) and
    one element set to 2^17 (beyond fp16's range).  The weights' hi + lo split keeps P.V
    exact to ~2^-16 of each weight whatever V holds; the result must meet the bar against
    the oracle."""
    Hkv = 2
    w = tiny("bf16", PREFILL_LENS, g * Hkv, Hkv, D, BS, seed=75 + D + BS + g,
             scale=0.6 / np.sqrt(D) * 4)
    pb = make_prefill(w, [1, 5, 17, 33, 64, 40, 200, 129], 75)
    kc, vc = build_pools(w)
    v = (vc.astype(np.uint32) << 16).view(np.float32).copy()      # bf16 bits -> values
    v[::3] *= 16.0
    b, kvh = int(w.block_table[6, 2]), 1                            # a block sequence 6 reads
    v[b, kvh, 0, 5, 3] = 2.0 ** 17                                 # token 3, channel 5
    vc = (v.view(np.uint32) >> 16).astype(np.uint16)
    assert np.abs(np.nan_to_num(v)).max() > 65504
    say(f"prefill with large V, D={D} BS={BS} g={g}")
    got = run_prefill(w, pb, kc, vc)
    ref = oracle.paged_prefill(pb.query, pb.query_start_loc, w.block_table, w.context_lens,
                               kc, vc, w.scale, "bf16")
    check_close(to_f64(got), ref, "bf16", f"prefill-large-v/{D}/{BS}/{g}")


def test_prefill_long_context_reloads_the_table_window():
    """More than 1024 blocks before the chunk (BS 8, 9000 tokens)."""
    w = tiny("bf16", (9000, 40), 8, 2, 128, 8, seed=75)
    pb = make_prefill(w, [70, 40], 75)
    kc, vc = build_pools(w)
    say("prefill long context, 1125 blocks")
    got = run_prefill(w, pb, kc, vc)
    ref = oracle.paged_prefill(pb.query, pb.query_start_loc, w.block_table, w.context_lens,
                               kc, vc, w.scale, "bf16")
    check_close(to_f64(got), ref, "bf16", "prefill-long")


def test_prefill_rising_scores_move_the_running_max():
    """Keys of one sign grow along the sequence (x(1 + t/35) at position t) and the
    queries have one sign too, so each row's maximum score climbs by about 9.5 (log2
    units) per 32-key step: the running max moves on most steps and the accumulators
    are rescaled, which random keys of one scale almost never cause.  bf16 only: at
    these logits (up to ~100) fp32 rounding of the score alone nears the f32 bar."""
    from workloads.configs import f32_to_bf16_bits
    w = tiny("bf16", (300, 130, 77), 8, 2, 128, 16, seed=81, scale=1.0 / np.sqrt(128))
    for recs in w.seq_records:
        f = 1.0 + np.arange(len(recs)) / 35.0
        kf = (w.rec_key[recs].astype(np.uint32) << 16).view(np.float32)
        w.rec_key[recs] = f32_to_bf16_bits(np.abs(kf) * f[:, None, None].astype(np.float32))
    pb = make_prefill(w, [300, 64, 77], 81)
    pb.query = pb.query & np.uint16(0x7FFF)
    kc, vc = build_pools(w)
    say("prefill rising scores")
    got = run_prefill(w, pb, kc, vc)
    ref = oracle.paged_prefill(pb.query, pb.query_start_loc, w.block_table, w.context_lens,
                               kc, vc, w.scale, "bf16")
    check_close(to_f64(got), ref, "bf16", "prefill-rising")


@pytest.mark.parametrize("name", ["prefix-cache-prefill", "chunked-prefill-llama3-8b"])
def test_prefill_named_cases_every_row(name):
    """Full-size batches; the oracle checks every row of every sequence."""
    w, pb = make_prefill_config(name)
    hist = pb.history_records(w)
    kc_np, vc_np = oracle.empty_pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size,
                                      w.dtype)
    oracle.reshape_and_cache(w.rec_key[hist], w.rec_value[hist], w.rec_slot[hist], kc_np, vc_np,
                             inplace=True)
    kc, vc = to_dev(kc_np, w.dtype, DEV), to_dev(vc_np, w.dtype, DEV)
    # the chunks' own K/V go in through the library's scatter, as a prefill step does
    rec = pb.chunk_records
    pk.reshape_and_cache(to_dev(w.rec_key[rec], w.dtype, DEV), to_dev(w.rec_value[rec], w.dtype, DEV),
                         torch.from_numpy(w.rec_slot[rec]).to(DEV), kc, vc)
    say(f"prefill {name}: S={w.num_seqs} T={len(rec)} max chunk {pb.max_query_len}")
    out = pk.paged_prefill(to_dev(pb.query, w.dtype, DEV),
                           torch.from_numpy(pb.query_start_loc).to(DEV),
                           torch.from_numpy(w.block_table).to(DEV),
                           torch.from_numpy(w.context_lens).to(DEV), kc, vc, w.scale,
                           max_query_len=pb.max_query_len)
    torch.cuda.synchronize()
    oracle.reshape_and_cache(w.rec_key[rec], w.rec_value[rec], w.rec_slot[rec], kc_np, vc_np,
                             inplace=True)
    assert np.array_equal(bits(kc), kc_np.view(bits(kc).dtype))
    assert np.array_equal(bits(vc), vc_np.view(bits(vc).dtype))
    got = to_f64(out)
    del kc, vc, out
    ref = prefill_reference(w, pb, kc_np, vc_np)
    stats = check_close(got, ref, w.dtype, name)
    say(f"  {name}: {stats}")


# ---------------------------------------------------------------------------
# every group size the host check admits (g <= 8 for bf16, <= 16 for f32)
# ---------------------------------------------------------------------------
GROUP_CASES = ([("bf16", g) for g in (2, 3, 5, 6, 7)] +
               [("f32", g) for g in (2, 3, 5, 6, 7, 9, 11, 12, 13, 15, 16)])


@pytest.mark.parametrize("D,BS", [(128, 16), (64, 8), (128, 32)])
@pytest.mark.parametrize("dtype,g", GROUP_CASES, ids=[f"{d}-g{g}" for d, g in GROUP_CASES])
def test_every_accepted_group_size(dtype, g, D, BS):
    """The group sizes beyond 1, 4 and 8 run the same lane code with other row counts:
    the hi/lo rows [g, 2g) of the bf16 MFMA, the head of each row (n % g), the fold of
    the lo rows (a shuffle by g) and the merge's g rows.  Decode in the paired mode, with
    the merge kernel and one partition per wave, and the fused step (caches bit-exact,
    output equal to the two calls)."""
    Hkv = 2
    w = tiny(dtype, LENS, g * Hkv, Hkv, D, BS, seed=900 + 16 * g + D + BS,
             scale=0.6 / np.sqrt(D) * 4)
    kc, vc = build_pools(w)
    ref = oracle_out(w, kc, vc)
    for part in (0, 64, 768):
        say(f"group {dtype} g={g} D={D} BS={BS} P={part}")
        check_close(to_f64(run_gpu(w, kc, vc, part)), ref, dtype, f"g{g}/{dtype}/{D}/{BS}/{part}")
    new, slots = fused_inputs(w)
    hist_k, hist_v = build_pools(w, include_new=False)
    ref_k, ref_v = oracle.reshape_and_cache(w.rec_key[new], w.rec_value[new], slots, hist_k, hist_v)
    inp = upload_inputs(w, DEV)
    key, val = to_dev(w.rec_key[new], w.dtype, DEV), to_dev(w.rec_value[new], w.dtype, DEV)
    slot_t = torch.from_numpy(slots).to(DEV)
    for part in (0, 64):
        say(f"group fused step {dtype} g={g} D={D} BS={BS} P={part}")
        kd, vd = to_dev(hist_k, w.dtype, DEV), to_dev(hist_v, w.dtype, DEV)
        out = pk.decode_step(inp["query"], key, val, slot_t, inp["block_table"],
                             inp["context_lens"], kd, vd, w.scale,
                             max_context_len=w.max_context_len, partition_size=part)
        kd2, vd2 = to_dev(hist_k, w.dtype, DEV), to_dev(hist_v, w.dtype, DEV)
        pk.reshape_and_cache(key, val, slot_t, kd2, vd2)
        out2 = pk.paged_attention(inp["query"], inp["block_table"], inp["context_lens"], kd2,
                                  vd2, w.scale, max_context_len=w.max_context_len,
                                  partition_size=part)
        torch.cuda.synchronize()
        assert np.array_equal(bits(kd), ref_k.view(bits(kd).dtype))
        assert np.array_equal(bits(vd), ref_v.view(bits(vd).dtype))
        assert np.array_equal(bits(out), bits(out2))
        check_close(to_f64(out), ref, dtype, f"fused g{g}/{dtype}/{D}/{BS}/{part}")


def test_group_sizes_past_the_limit_are_refused():
    """g = 9 in bf16 and g = 17 in f32 are not built: refused before any launch."""
    for dtype, g in (("bf16", 9), ("f32", 17)):
        w = tiny(dtype, (5, 9), g, 1, 64, 16, seed=950)
        kc, vc = build_pools(w)
        with pytest.raises(NotImplementedError):
            run_gpu(w, kc, vc)


def test_prefill_group_sizes_two_and_sixteen():
    """The prefill's other admitted group sizes (its tile of 128 rows takes g in
    {1, 2, 4, 8, 16}); g = 3 is refused."""
    for dtype, g, D, BS in (("bf16", 2, 128, 16), ("bf16", 16, 64, 8), ("f32", 2, 64, 32),
                            ("f32", 16, 128, 16), ("bf16", 2, 64, 32), ("bf16", 16, 128, 32)):
        Hkv = 2
        w = tiny(dtype, PREFILL_LENS, g * Hkv, Hkv, D, BS, seed=960 + g + D + BS,
                 scale=0.6 / np.sqrt(D) * 4)
        chunks = [1, 5, 17, 33, 64, 40, 200, 129]
        pb = make_prefill(w, chunks, 960 + g)
        kc, vc = build_pools(w)
        say(f"prefill group {dtype} g={g} D={D} BS={BS}")
        got = run_prefill(w, pb, kc, vc)
        ref = oracle.paged_prefill(pb.query, pb.query_start_loc, w.block_table, w.context_lens,
                                   kc, vc, w.scale, dtype)
        check_close(to_f64(got), ref, dtype, f"prefill g{g}/{dtype}/{D}/{BS}")
    w = tiny("bf16", (5, 9), 6, 2, 64, 16, seed=969)
    pb = make_prefill(w, [5, 9], 969)
    kc, vc = build_pools(w)
    with pytest.raises(NotImplementedError):
        run_prefill(w, pb, kc, vc)


# ---------------------------------------------------------------------------
# a caller's side stream: memory the binding allocates is not reused too early
# ---------------------------------------------------------------------------
def test_side_stream_with_binding_allocated_workspace_and_output():
    """The binding allocates out and the partition workspace on torch's current stream
    while the kernels run on the caller's stream.  Right after the call the test
    allocates and fills other tensors on the current stream: had the binding not marked
    its tensors as used on the side stream, the caching allocator could hand their memory
    to those tensors while the decode still writes and reads it."""
    w = tiny("bf16", long_tail_lens(71), 32, 8, 128, 16, seed=71)
    kc_np, vc_np = build_pools(w)
    ref = oracle_out(w, kc_np, vc_np)
    inp = upload_inputs(w, DEV)
    kc, vc = to_dev(kc_np, w.dtype, DEV), to_dev(vc_np, w.dtype, DEV)
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    say("side stream: decode with binding-allocated out and workspace")
    outs = []
    for rep in range(3):
        out = pk.paged_attention(inp["query"], inp["block_table"], inp["context_lens"], kc, vc,
                                 w.scale, max_context_len=w.max_context_len, partition_size=64,
                                 stream=side)
        outs.append(out)
        # freed workspace and other allocations on the current stream, filled at once
        junk = [torch.full((1 << 20,), float("nan"), dtype=torch.float32, device=DEV)
                for _ in range(16)]
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for out in outs:
        check_close(to_f64(out), ref, "bf16", "side-stream")
