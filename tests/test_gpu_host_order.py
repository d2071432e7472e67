"""GPU: decode calls given a host copy of the context lengths (host_context_lens).

With the host copy, the library orders the sequences for the paired mode on the
host and the workgroups skip ranking the lengths.  The order uses the same keys
as the in-kernel ranking, so:
* with a matching host copy, out and both caches are the same bit for bit as
  without it (fused and two-call steps, bf16, f32 and FP8 pools), and the output
  meets the oracle bar;
* with a host copy that does not match the device lengths, the work is spread
  differently but every sequence is still computed once: the output still meets
  the oracle bar and the caches are still bit-exact;
* launches that do not use the paired mode (several partitions per sequence)
  ignore the copy;
* over FP8 pools, whose first step per wave is read with the host's block count, a
  stale copy (a block short or long, or unrelated) still gives the oracle's caches and
  an output within the bar.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_425_amd as pk
from tests.gpu_util import bits, check_close, to_dev, to_f64, upload_inputs
from tests.helpers import build_pools, oracle_out
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
K_SCALE, V_SCALE = 0.0135, 0.0121


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def tiny(dtype, lens, Hq, Hkv, D, BS, seed=0):
    return make_workload(name="host-order", context_lens=list(lens), num_heads=Hq,
                         num_kv_heads=Hkv, head_dim=D, block_size=BS, dtype=dtype, seed=seed)


LENS = (1, 2, 7, 31, 32, 33, 63, 64, 65, 130, 257, 511, 700)

STEP_CASES = [("cfg0", lambda: make_config(0), True),
              ("cfg1", lambda: make_config(1), True),
              ("cfg2-bs8", lambda: make_config(2, block_size=8), False),
              ("cfg2-bs16", lambda: make_config(2, block_size=16), False),
              ("cfg2-bs32", lambda: make_config(2, block_size=32), False),
              ("cfg3-prefix", lambda: make_config(3), False),
              ("cfg3-parallel-sampling", lambda: make_config(3, variant="parallel-sampling"),
               True),
              ("tiny-bf16-ragged", lambda: tiny("bf16", LENS, 16, 2, 64, 32, seed=401), True),
              ("tiny-f32-ragged", lambda: tiny("f32", LENS, 32, 2, 128, 8, seed=402), True),
              ("equal-lengths", lambda: tiny("bf16", [97] * 40, 32, 8, 128, 16, seed=403), True),
              ("odd-count", lambda: tiny("bf16", (700, 3, 64, 1, 333, 129, 40), 32, 8, 128, 16,
                                          seed=404), True)]


def _fused_step(w, hist_k, hist_v, host_lens):
    new = np.array([w.seq_records[s][-1] for s in range(w.num_seqs)], dtype=np.int64)
    inp = upload_inputs(w, DEV)
    kc, vc = to_dev(hist_k, w.dtype, DEV), to_dev(hist_v, w.dtype, DEV)
    out = pk.decode_step(inp["query"], to_dev(w.rec_key[new], w.dtype, DEV),
                         to_dev(w.rec_value[new], w.dtype, DEV),
                         torch.from_numpy(w.rec_slot[new]).to(DEV), inp["block_table"],
                         inp["context_lens"], kc, vc, w.scale,
                         max_context_len=w.max_context_len, host_context_lens=host_lens)
    torch.cuda.synchronize()
    return out, kc, vc, new


@pytest.mark.parametrize("name,make,with_oracle", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_fused_step_with_host_lengths_is_bitwise_unchanged(name, make, with_oracle):
    w = make()
    say(f"host order: fused step {name} S={w.num_seqs} BS={w.block_size}")
    hist_k, hist_v = build_pools(w, include_new=False)
    out0, kc0, vc0, new = _fused_step(w, hist_k, hist_v, None)
    out1, kc1, vc1, _ = _fused_step(w, hist_k, hist_v, w.context_lens.copy())
    assert np.array_equal(bits(out1), bits(out0))
    assert np.array_equal(bits(kc1), bits(kc0))
    assert np.array_equal(bits(vc1), bits(vc0))
    if with_oracle:
        ref_k, ref_v = oracle.reshape_and_cache(w.rec_key[new], w.rec_value[new],
                                                w.rec_slot[new], hist_k, hist_v)
        assert np.array_equal(bits(kc1), ref_k.view(bits(kc1).dtype))
        stats = check_close(to_f64(out1), oracle_out(w, ref_k, ref_v), w.dtype, name)
        say(f"  {name}: {stats}")


@pytest.mark.parametrize("dtype,D,BS,g", [("f32", 64, 8, 1), ("bf16", 128, 16, 4),
                                          ("bf16", 64, 32, 8), ("f32", 128, 32, 16)])
def test_attention_with_host_lengths_is_bitwise_unchanged(dtype, D, BS, g):
    w = tiny(dtype, LENS, 2 * g, 2, D, BS, seed=410 + D + BS + g)
    kc_np, vc_np = build_pools(w)
    inp = upload_inputs(w, DEV)
    kc, vc = to_dev(kc_np, dtype, DEV), to_dev(vc_np, dtype, DEV)
    say(f"host order: attention {dtype} D={D} BS={BS} g={g}")
    outs = [pk.paged_attention(inp["query"], inp["block_table"], inp["context_lens"], kc, vc,
                               w.scale, max_context_len=w.max_context_len, host_context_lens=h)
            for h in (None, w.context_lens.copy(), torch.from_numpy(w.context_lens.copy()))]
    torch.cuda.synchronize()
    assert np.array_equal(bits(outs[1]), bits(outs[0]))
    assert np.array_equal(bits(outs[2]), bits(outs[0]))
    check_close(to_f64(outs[1]), oracle_out(w, kc_np, vc_np), dtype, "host-order")


@pytest.mark.parametrize("how", ["reversed", "shuffled", "zeros", "too-long"])
def test_stale_host_lengths_still_meet_the_bar(how):
    """A host copy that does not match the device lengths changes the pairing only."""
    w = make_config(1)
    rng = np.random.default_rng(420)
    host = w.context_lens.copy()
    if how == "reversed":
        host = host[::-1].copy()
    elif how == "shuffled":
        host = rng.permutation(host)
    elif how == "zeros":
        host[:] = 0
    else:
        host[:] = 10 ** 6
    say(f"host order: stale host copy ({how}) on the Llama-3-8B batch")
    hist_k, hist_v = build_pools(w, include_new=False)
    out, kc, vc, new = _fused_step(w, hist_k, hist_v, host)
    ref_k, ref_v = oracle.reshape_and_cache(w.rec_key[new], w.rec_value[new], w.rec_slot[new],
                                            hist_k, hist_v)
    assert np.array_equal(bits(kc), ref_k.view(bits(kc).dtype))
    assert np.array_equal(bits(vc), ref_v.view(bits(vc).dtype))
    stats = check_close(to_f64(out), oracle_out(w, ref_k, ref_v), w.dtype, how)
    say(f"  {how}: {stats}")


def test_partition_mode_ignores_host_lengths():
    """Several partitions per sequence (no paired mode): the copy is not used."""
    w = make_config(4)
    say("host order: long-context batch at 512-token partitions")
    kc_np, vc_np = build_pools(w)
    inp = upload_inputs(w, DEV)
    kc, vc = to_dev(kc_np, w.dtype, DEV), to_dev(vc_np, w.dtype, DEV)
    outs = [pk.paged_attention(inp["query"], inp["block_table"], inp["context_lens"], kc, vc,
                               w.scale, max_context_len=w.max_context_len, partition_size=512,
                               host_context_lens=h)
            for h in (None, np.zeros_like(w.context_lens))]
    torch.cuda.synchronize()
    assert np.array_equal(bits(outs[1]), bits(outs[0]))


@pytest.mark.parametrize("D,BS,g", [(128, 16, 4), (64, 8, 8), (128, 32, 1)])
def test_fp8_step_with_host_lengths_is_bitwise_unchanged(D, BS, g):
    w = tiny("bf16", LENS + (1500, 9), 2 * g, 2, D, BS, seed=430 + D + BS + g)
    kc_np, vc_np = oracle.empty_fp8_pools(w.num_blocks, w.num_kv_heads, w.head_dim,
                                          w.block_size)
    hist = w.history_records
    oracle.reshape_and_cache_fp8(w.rec_key[hist], w.rec_value[hist], w.rec_slot[hist], kc_np,
                                 vc_np, w.dtype, K_SCALE, V_SCALE, inplace=True)
    new = np.array([w.seq_records[s][-1] for s in range(w.num_seqs)], dtype=np.int64)
    inp = upload_inputs(w, DEV)
    key, val = to_dev(w.rec_key[new], w.dtype, DEV), to_dev(w.rec_value[new], w.dtype, DEV)
    slot_t = torch.from_numpy(w.rec_slot[new]).to(DEV)
    say(f"host order: FP8 fused step D={D} BS={BS} g={g}")
    res = []
    for h in (None, w.context_lens.copy()):
        kc = torch.from_numpy(kc_np.copy()).to(DEV)
        vc = torch.from_numpy(vc_np.copy()).to(DEV)
        out = pk.decode_step_fp8(inp["query"], key, val, slot_t, inp["block_table"],
                                 inp["context_lens"], kc, vc, w.scale, K_SCALE, V_SCALE,
                                 max_context_len=w.max_context_len, host_context_lens=h)
        att = pk.paged_attention_fp8(inp["query"], inp["block_table"], inp["context_lens"], kc,
                                     vc, w.scale, K_SCALE, V_SCALE,
                                     max_context_len=w.max_context_len, host_context_lens=h)
        torch.cuda.synchronize()
        res.append((bits(out), bits(att), kc.cpu().numpy(), vc.cpu().numpy()))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)
    oracle.reshape_and_cache_fp8(w.rec_key[new], w.rec_value[new], w.rec_slot[new], kc_np,
                                 vc_np, w.dtype, K_SCALE, V_SCALE, inplace=True)
    assert np.array_equal(res[1][2], kc_np) and np.array_equal(res[1][3], vc_np)
    ref = oracle.paged_attention_fp8(w.query, w.block_table, w.context_lens, kc_np, vc_np,
                                     w.scale, K_SCALE, V_SCALE, "bf16")
    out1 = res[1][0].view(np.uint16).astype(np.uint32) << 16
    check_close(out1.view(np.float32).astype(np.float64), ref, "bf16", "fp8-host-order")


STALE = ["reversed", "shuffled", "zeros", "too-long", "one-block-short", "one-block-long"]


@pytest.mark.parametrize("D,BS,g", [(128, 16, 4), (64, 8, 8)])
@pytest.mark.parametrize("how", STALE)
def test_fp8_stale_host_lengths_still_meet_the_bar(how, D, BS, g):
    """FP8 pools read each wave's first step from table entries taken before the lengths
    are known, among them the entry of the last block by the host's block count: with a
    stale copy (shorter or longer by a block, or unrelated) the caches must still be the
    oracle's and the output within the bar."""
    w = tiny("bf16", LENS + (1500, 9, 48, 49), 2 * g, 2, D, BS, seed=450 + D + BS + g)
    rng = np.random.default_rng(451)
    host = w.context_lens.copy()
    if how == "reversed":
        host = host[::-1].copy()
    elif how == "shuffled":
        host = rng.permutation(host)
    elif how == "zeros":
        host[:] = 0
    elif how == "too-long":
        host[:] = 10 ** 6
    elif how == "one-block-short":
        host = np.maximum(host - BS, 0)
    else:
        host = host + BS
    kc_np, vc_np = oracle.empty_fp8_pools(w.num_blocks, w.num_kv_heads, w.head_dim,
                                          w.block_size)
    hist = w.history_records
    oracle.reshape_and_cache_fp8(w.rec_key[hist], w.rec_value[hist], w.rec_slot[hist], kc_np,
                                 vc_np, w.dtype, K_SCALE, V_SCALE, inplace=True)
    new = np.array([w.seq_records[s][-1] for s in range(w.num_seqs)], dtype=np.int64)
    inp = upload_inputs(w, DEV)
    kc = torch.from_numpy(kc_np.copy()).to(DEV)
    vc = torch.from_numpy(vc_np.copy()).to(DEV)
    say(f"host order: FP8 fused step, stale host copy ({how}) D={D} BS={BS} g={g}")
    out = pk.decode_step_fp8(inp["query"], to_dev(w.rec_key[new], w.dtype, DEV),
                             to_dev(w.rec_value[new], w.dtype, DEV),
                             torch.from_numpy(w.rec_slot[new]).to(DEV), inp["block_table"],
                             inp["context_lens"], kc, vc, w.scale, K_SCALE, V_SCALE,
                             max_context_len=w.max_context_len, host_context_lens=host)
    torch.cuda.synchronize()
    oracle.reshape_and_cache_fp8(w.rec_key[new], w.rec_value[new], w.rec_slot[new], kc_np,
                                 vc_np, w.dtype, K_SCALE, V_SCALE, inplace=True)
    assert np.array_equal(kc.cpu().numpy(), kc_np) and np.array_equal(vc.cpu().numpy(), vc_np)
    ref = oracle.paged_attention_fp8(w.query, w.block_table, w.context_lens, kc_np, vc_np,
                                     w.scale, K_SCALE, V_SCALE, "bf16")
    got = bits(out).view(np.uint16).astype(np.uint32) << 16
    say(f"  {check_close(got.view(np.float32).astype(np.float64), ref, 'bf16', how)}")
