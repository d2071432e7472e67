"""The allocation-free decode step (pa_decode_step_noalloc) against pa_decode_step.

pa_decode_step_noalloc keeps the partitions' partial results in a fixed scratch
array inside the library instead of a caller's workspace.  Two calls in a row,
the second with a smaller batch, must give the output and caches of
pa_decode_step with a workspace bit for bit, and meet the parity bar against
the oracle.  The second call finds the first call's partials in the scratch.
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


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def batch(n_short: int, n_long: int, seed: int, dtype: str = "bf16"):
    rng = np.random.default_rng(seed)
    lens = rng.permutation(np.concatenate([rng.integers(1, 300, size=n_short),
                                           rng.integers(1500, 3000, size=n_long)]))
    return make_workload(name="noalloc", context_lens=list(lens), num_heads=32, num_kv_heads=8,
                         head_dim=128, block_size=16, dtype=dtype, seed=seed)


def step_both_ways(w, part):
    """(out of pa_decode_step, out of pa_decode_step_noalloc, caches of each, oracle)."""
    new = np.array([w.seq_records[s][-1] for s in range(w.num_seqs)], dtype=np.int64)
    slots = w.rec_slot[new].copy()
    hist_k, hist_v = build_pools(w, include_new=False)
    ref_k, ref_v = oracle.reshape_and_cache(w.rec_key[new], w.rec_value[new], slots, hist_k,
                                            hist_v)
    inp = upload_inputs(w, DEV)
    key, val = to_dev(w.rec_key[new], w.dtype, DEV), to_dev(w.rec_value[new], w.dtype, DEV)
    slot_t = torch.from_numpy(slots).to(DEV)
    kc, vc = to_dev(hist_k, w.dtype, DEV), to_dev(hist_v, w.dtype, DEV)
    out = pk.decode_step(inp["query"], key, val, slot_t, inp["block_table"], inp["context_lens"],
                         kc, vc, w.scale, max_context_len=w.max_context_len, partition_size=part)
    kc2, vc2 = to_dev(hist_k, w.dtype, DEV), to_dev(hist_v, w.dtype, DEV)
    out2 = torch.empty_like(inp["query"])
    pk.decode_step_noalloc(inp["query"], key, val, slot_t, inp["block_table"],
                           inp["context_lens"], kc2, vc2, w.scale,
                           max_context_len=w.max_context_len, out=out2, partition_size=part)
    torch.cuda.synchronize()
    return out, out2, (kc, vc), (kc2, vc2), (ref_k, ref_v), oracle_out(w, ref_k, ref_v)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_step_equals_step_with_workspace_two_calls(dtype):
    first = batch(58, 6, 1200, dtype)           # 64 sequences, partitions of 64 tokens
    second = batch(20, 3, 1201, dtype)          # fewer and shorter: a smaller input
    for label, w, part in (("first", first, 64), ("second", second, 64),
                           ("one partition, no scratch", second, 4096)):
        need = pk.workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                 w.max_context_len, part, torch.float32 if dtype == "f32"
                                 else torch.bfloat16)
        say(f"noalloc {dtype} {label}: S={w.num_seqs} max L={w.max_context_len} P={part} "
            f"workspace {need} B")
        out, out2, (kc, vc), (kc2, vc2), (ref_k, ref_v), ref = step_both_ways(w, part)
        assert np.array_equal(bits(out), bits(out2)), f"{label}: output differs"
        assert np.array_equal(bits(kc2), ref_k.view(bits(kc2).dtype)), f"{label}: K pool"
        assert np.array_equal(bits(vc2), ref_v.view(bits(vc2).dtype)), f"{label}: V pool"
        assert np.array_equal(bits(kc), bits(kc2)) and np.array_equal(bits(vc), bits(vc2))
        check_close(to_f64(out2), ref, dtype, f"noalloc {dtype} {label}")


def test_noalloc_step_refuses_more_than_the_scratch():
    """A batch whose partials exceed the scratch is refused before any launch, and the
    next call still works."""
    w = batch(6, 2, 1202)
    inp = upload_inputs(w, DEV)
    new = np.array([w.seq_records[s][-1] for s in range(w.num_seqs)], dtype=np.int64)
    kc, vc = (to_dev(a, w.dtype, DEV) for a in build_pools(w, include_new=False))
    key, val = to_dev(w.rec_key[new], w.dtype, DEV), to_dev(w.rec_value[new], w.dtype, DEV)
    slot_t = torch.from_numpy(w.rec_slot[new]).to(DEV)
    out = torch.empty_like(inp["query"])
    # claim a maximum length of 1M tokens (table wide enough) in 64-token partitions:
    # 8 x 32 x 16384 partial rows of 130 floats, far past 64 MiB
    wide = torch.zeros((w.num_seqs, (1 << 20) // 16), dtype=torch.int32, device=DEV)
    wide[:, :w.block_table.shape[1]] = inp["block_table"]
    say("noalloc refusal")
    with pytest.raises(ValueError):
        pk.decode_step_noalloc(inp["query"], key, val, slot_t, wide, inp["context_lens"], kc, vc,
                               w.scale, max_context_len=1 << 20, out=out, partition_size=64)
    pk.decode_step_noalloc(inp["query"], key, val, slot_t, inp["block_table"],
                           inp["context_lens"], kc, vc, w.scale,
                           max_context_len=w.max_context_len, out=out, partition_size=64)
    torch.cuda.synchronize()
    kr, vr = build_pools(w)
    check_close(to_f64(out), oracle_out(w, kr, vr), "bf16", "noalloc after refusal")
