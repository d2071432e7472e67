"""GPU parity of the paired decode at 4 waves per workgroup.

The paired mode (every sequence one partition) runs 8 waves per workgroup, or 4 when the
pairs outnumber the compute units and the two longest sequences together fit in 32 steps
(32 tokens a step for bf16, 16 for f32, 64 for FP8 pools), so that two workgroups share a
compute unit.  These batches take the 4-wave launch: attention over the K/V reassembled from
the block table ("core architecture" page, section 2.2.2) must meet the oracle bar, with and
without the host copy of the lengths, the two bit-identical, and the fused step's caches
must be bit-exact.  One batch has more sequences (512) than a 4-wave workgroup has threads,
which the in-kernel ranking of the lengths must handle.
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
from workloads import make_workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
K_SCALE, V_SCALE = 0.0135, 0.0121


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def batch(dtype, S, Hkv, g, D, BS, max_len, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len + 1, size=S)
    lens[0] = max_len
    lens[1] = 1
    return make_workload(name="pair-waves", context_lens=lens, num_heads=g * Hkv,
                         num_kv_heads=Hkv, head_dim=D, block_size=BS, dtype=dtype, seed=seed)


# (dtype, S, Hkv, g, D, BS, max_len): ceil(S / 2) * Hkv > 256 workgroups and
# 2 * max_len <= 32 * step
CASES = [("bf16", 128, 8, 4, 128, 16, 512),
         ("bf16", 512, 2, 1, 64, 8, 300),
         ("bf16", 96, 8, 8, 128, 32, 480),
         ("f32", 160, 8, 2, 128, 16, 256),
         ("f32", 100, 6, 4, 64, 8, 200)]


@pytest.mark.parametrize("dtype,S,Hkv,g,D,BS,max_len", CASES)
def test_four_wave_pairs_meet_the_bar(dtype, S, Hkv, g, D, BS, max_len):
    w = batch(dtype, S, Hkv, g, D, BS, max_len, seed=1200 + S + D + BS)
    kc_np, vc_np = build_pools(w)
    inp = upload_inputs(w, DEV)
    kc, vc = to_dev(kc_np, dtype, DEV), to_dev(vc_np, dtype, DEV)
    say(f"4-wave pairs: {dtype} S={S} Hkv={Hkv} g={g} D={D} BS={BS} max={max_len}")
    outs = [pk.paged_attention(inp["query"], inp["block_table"], inp["context_lens"], kc, vc,
                               w.scale, max_context_len=w.max_context_len, host_context_lens=h)
            for h in (None, w.context_lens.copy())]
    torch.cuda.synchronize()
    assert np.array_equal(bits(outs[1]), bits(outs[0]))
    say(f"  {check_close(to_f64(outs[1]), oracle_out(w, kc_np, vc_np), dtype, 'pair-waves')}")


@pytest.mark.parametrize("dtype,S,Hkv,g,D,BS,max_len", CASES[:3])
def test_four_wave_fused_step(dtype, S, Hkv, g, D, BS, max_len):
    w = batch(dtype, S, Hkv, g, D, BS, max_len, seed=1300 + S + D + BS)
    new = np.array([w.seq_records[s][-1] for s in range(w.num_seqs)], dtype=np.int64)
    hist_k, hist_v = build_pools(w, include_new=False)
    ref_k, ref_v = oracle.reshape_and_cache(w.rec_key[new], w.rec_value[new], w.rec_slot[new],
                                            hist_k, hist_v)
    inp = upload_inputs(w, DEV)
    kc, vc = to_dev(hist_k, dtype, DEV), to_dev(hist_v, dtype, DEV)
    say(f"4-wave fused step: {dtype} S={S} Hkv={Hkv} g={g} D={D} BS={BS}")
    out = pk.decode_step(inp["query"], to_dev(w.rec_key[new], dtype, DEV),
                         to_dev(w.rec_value[new], dtype, DEV),
                         torch.from_numpy(w.rec_slot[new]).to(DEV), inp["block_table"],
                         inp["context_lens"], kc, vc, w.scale,
                         max_context_len=w.max_context_len, host_context_lens=w.context_lens)
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc), ref_k.view(bits(kc).dtype))
    assert np.array_equal(bits(vc), ref_v.view(bits(vc).dtype))
    check_close(to_f64(out), oracle_out(w, ref_k, ref_v), dtype, "pair-waves-fused")


def test_four_wave_pairs_fp8():
    """FP8 pools (64-token steps): 128 sequences up to 1024 tokens over 8 kv heads."""
    w = batch("bf16", 128, 8, 4, 128, 16, 1024, seed=1400)
    kc, vc = oracle.empty_fp8_pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size)
    oracle.reshape_and_cache_fp8(w.rec_key, w.rec_value, w.rec_slot, kc, vc, w.dtype, K_SCALE,
                                 V_SCALE, inplace=True)
    say("4-wave pairs: FP8 S=128 Hkv=8 g=4")
    outs = [pk.paged_attention_fp8(to_dev(w.query, w.dtype, DEV),
                                   torch.from_numpy(w.block_table).to(DEV),
                                   torch.from_numpy(w.context_lens).to(DEV),
                                   torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV),
                                   w.scale, K_SCALE, V_SCALE, max_context_len=w.max_context_len,
                                   host_context_lens=h)
            for h in (None, w.context_lens.copy())]
    torch.cuda.synchronize()
    assert np.array_equal(bits(outs[1]), bits(outs[0]))
    ref = oracle.paged_attention_fp8(w.query, w.block_table, w.context_lens, kc, vc, w.scale,
                                     K_SCALE, V_SCALE, "bf16")
    check_close(to_f64(outs[1]), ref, "bf16", "pair-waves-fp8")
