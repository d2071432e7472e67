"""Seeded synthetic decode workloads for paged attention.

A workload is everything a decode step consumes, built the way a serving
engine would lay it out, with random contents:

* ``query``        [S, Hq, D]   one query token per sequence;
* ``block_table``  [S, MB]      int32, logical block -> physical block;
* ``context_lens`` [S]          int32, tokens each query attends over
                                (the step's new token included);
* token records: the K and V vectors of every token that lives in the pool,
  with the slot (physical_block * block_size + offset) each one occupies.
  ``new_records`` are the tokens written by the decode step itself
  (the reshape_and_cache input); every other record is history already in
  the pool when the step starts.
* ``seq_records[s]``: record index of each logical position 0..L_s-1 of
  sequence s, i.e. the contiguous, never-paged K/V of that sequence.

Values are drawn N(0, 1) in float32.  For bfloat16 workloads they are then
rounded to the nearest bfloat16 (ties to even) and kept as raw 16-bit
patterns in uint16 arrays, because NumPy has no bfloat16 type; consumers on
both sides decode those same bits.

The five named workloads mirror the shapes the pages discuss: a tiny float32
case, a Llama-3-8B-shaped decode batch (32 query / 8 KV heads, head size 128),
a continuous-batching mix of short and long requests with block size 8/16/32,
prefix sharing and parallel sampling with copy-on-write, and a long-context
Llama-3-70B-shaped batch (64 query / 8 KV heads) split into 512-token
partitions.

This module holds no attention arithmetic: it only draws numbers and builds
integer tables (see ``block_pool`` for the allocator).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .block_pool import BlockPool, SequenceBlocks, append_token

BF16_NAN_BITS = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even).

    Returns the raw 16-bit patterns.  Inputs here are N(0,1) draws, so NaN
    and overflow handling is not needed.
    """
    flat = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 22
    for i in range(0, flat.size, step):
        u = flat[i:i + step].view(np.uint32).copy()
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        u += np.uint32(0x7FFF)
        u += lsb
        u >>= np.uint32(16)
        out[i:i + step] = u
    return out.reshape(np.shape(x))


def element_size(dtype: str) -> int:
    return {"f32": 4, "bf16": 2}[dtype]


@dataclass
class Workload:
    name: str
    dtype: str                      # "f32" or "bf16"
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    query: np.ndarray               # [S, Hq, D] float32 or uint16 (bf16 bits)
    block_table: np.ndarray         # [S, MB] int32
    context_lens: np.ndarray        # [S] int32
    rec_key: np.ndarray             # [R, Hkv, D]
    rec_value: np.ndarray           # [R, Hkv, D]
    rec_slot: np.ndarray            # [R] int64
    seq_records: list               # S arrays of int64, length L_s
    new_records: np.ndarray         # [T] int64, written by the decode step
    partition_size: int | None = None
    # copy-on-write block copies, [n, 2] int64 (source block, destination block): the
    # records that duplicate a source block's tokens into its copy are listed in
    # cow_records (they exist before the step only once the blocks are copied)
    cow_pairs: np.ndarray = field(default_factory=lambda: np.zeros((0, 2), dtype=np.int64))
    cow_records: np.ndarray = field(default_factory=lambda: np.zeros(0, dtype=np.int64))
    blocks_allocated: int = 0
    info: dict = field(default_factory=dict)

    # ---- derived views -------------------------------------------------
    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def history_records(self) -> np.ndarray:
        mask = np.ones(len(self.rec_slot), dtype=bool)
        mask[self.new_records] = False
        return np.nonzero(mask)[0]

    @property
    def kv_bytes_logical(self) -> int:
        """K+V bytes one decode step reads if every position is fetched."""
        return int(self.context_lens.astype(np.int64).sum()) * 2 * \
            self.num_kv_heads * self.head_dim * element_size(self.dtype)

    @property
    def kv_bytes_unique(self) -> int:
        """K+V bytes of the distinct physical token slots one step reads."""
        slots = set()
        for s in range(self.num_seqs):
            slots.update(self.rec_slot[self.seq_records[s]].tolist())
        return len(slots) * 2 * self.num_kv_heads * self.head_dim * \
            element_size(self.dtype)


# ---------------------------------------------------------------------------
def _draw(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) float32 draws, bf16-rounded if asked.

    Large arrays are drawn in fixed chunks of rows, chunk k from its own
    generator seeded by (one number taken from ``rng``, k), on a thread pool;
    the result depends only on ``rng``'s state, never on the thread count.
    """
    shape = tuple(int(n) for n in shape)
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    if out.size == 0:
        return out
    flat = out.reshape(shape[0], -1)
    rows = max(1, (1 << 21) // max(1, flat.shape[1]))
    base = int(rng.integers(0, 2**63 - 1))

    def fill(k: int) -> None:
        r = k * rows
        n = min(rows, shape[0] - r)
        x = np.random.default_rng([base, k]).standard_normal((n, flat.shape[1]),
                                                             dtype=np.float32)
        flat[r:r + n] = f32_to_bf16_bits(x) if dtype == "bf16" else x

    chunks = -(-shape[0] // rows)
    if chunks == 1:
        fill(0)
    else:
        workers = min(16, len(os.sched_getaffinity(0)), chunks)
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(chunks)))
    return out


def make_workload(*, name: str, context_lens, num_heads: int, num_kv_heads: int,
                  head_dim: int, block_size: int, dtype: str, seed: int,
                  rng: np.random.Generator | None = None, scale: float | None = None,
                  num_blocks: int | None = None, pool_factor: float = 1.2,
                  max_blocks_per_seq: int | None = None,
                  shared_prefix_len: int = 0, samples_per_prompt: int = 1,
                  partition_size: int | None = None) -> Workload:
    """Lay out a batch of sequences in a paged pool and draw its contents.

    ``context_lens`` are the per-sequence lengths including the step's new
    token.  With ``shared_prefix_len`` > 0 every sequence starts with the same
    prefix stored once.  With ``samples_per_prompt`` = n > 1 the lengths are
    prompt lengths; each prompt is forked into n samples that each append one
    new token, copying a shared partial last block first (copy-on-write).
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    rng = rng if rng is not None else np.random.default_rng(seed)
    lens_in = np.asarray(context_lens, dtype=np.int64)
    BS = int(block_size)
    nblk = lambda n: -(-int(n) // BS)  # noqa: E731  ceil division

    # ---- pool size ------------------------------------------------------
    if samples_per_prompt > 1:
        need = sum(nblk(L) + samples_per_prompt for L in lens_in)
    elif shared_prefix_len:
        need = nblk(shared_prefix_len) + sum(nblk(L) - shared_prefix_len // BS
                                             for L in lens_in)
    else:
        need = sum(nblk(L) for L in lens_in)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(pool_factor * need))
    pool = BlockPool(num_blocks, rng)

    # ---- allocation + records --------------------------------------------
    # records are appended as (slot, source-record-or--1); source >= 0 marks a
    # copy-on-write duplicate of an existing record.
    rec_slot: list = []
    rec_src: list = []
    cow_pairs: list = []
    seqs: list = []
    seq_records: list = []
    new_records: list = []

    def add_record(slot: int, src: int = -1) -> int:
        rec_slot.append(slot)
        rec_src.append(src)
        return len(rec_slot) - 1

    if samples_per_prompt > 1:
        for Lp in lens_in:
            prompt = SequenceBlocks()
            recs = [add_record(append_token(prompt, pool, BS).slot) for _ in range(int(Lp))]
            for _ in range(samples_per_prompt):
                seqs.append(prompt.fork(pool))
                seq_records.append(list(recs))
            for b in prompt.blocks:          # the template itself holds no reference
                pool.release(b)
        for i, seq in enumerate(seqs):
            w = append_token(seq, pool, BS)
            if w.copy_from >= 0:
                cow_pairs.append((w.copy_from, w.copy_to))
                # duplicate the stored tokens of the shared block into the copy
                stored = seq.num_tokens - 1 - (seq.num_tokens - 1) // BS * BS
                logical = (seq.num_tokens - 1) // BS
                for off in range(stored):
                    pos = logical * BS + off
                    src = seq_records[i][pos]
                    seq_records[i][pos] = add_record(w.copy_to * BS + off, src)
            r = add_record(w.slot)
            seq_records[i].append(r)
            new_records.append(r)
    elif shared_prefix_len:
        if shared_prefix_len % BS:
            raise ValueError("shared_prefix_len must be a whole number of blocks")
        if (lens_in <= shared_prefix_len).any():
            raise ValueError("every sequence must extend past the shared prefix")
        prompt = SequenceBlocks()
        prefix = [add_record(append_token(prompt, pool, BS).slot)
                  for _ in range(shared_prefix_len)]
        for L in lens_in:
            seq = prompt.fork(pool)
            recs = list(prefix)
            for _ in range(int(L) - shared_prefix_len):
                recs.append(add_record(append_token(seq, pool, BS).slot))
            seqs.append(seq)
            seq_records.append(recs)
            new_records.append(recs[-1])
        for b in prompt.blocks:
            pool.release(b)
    else:
        start = 0
        for L in lens_in:
            seq = SequenceBlocks(blocks=[pool.allocate() for _ in range(nblk(L))],
                                 num_tokens=int(L))
            t = np.arange(int(L), dtype=np.int64)
            slots = np.asarray(seq.blocks, dtype=np.int64)[t // BS] * BS + t % BS \
                if L else np.zeros(0, dtype=np.int64)
            rec_slot.extend(slots.tolist())
            rec_src.extend([-1] * int(L))
            recs = list(range(start, start + int(L)))
            start += int(L)
            seqs.append(seq)
            seq_records.append(recs)
            if L:
                new_records.append(recs[-1])

    S = len(seqs)
    lens = np.array([s.num_tokens for s in seqs], dtype=np.int32)
    MB = max_blocks_per_seq if max_blocks_per_seq is not None else \
        max(1, max(len(s.blocks) for s in seqs))
    if any(len(s.blocks) > MB for s in seqs):
        raise ValueError("a sequence needs more blocks than max_blocks_per_seq")

    # ---- block table: unused entries hold valid ids of other blocks -------
    allocated = np.nonzero(pool.refcount)[0]
    table = rng.choice(allocated, size=(S, MB)).astype(np.int32)
    for i, s in enumerate(seqs):
        table[i, :len(s.blocks)] = s.blocks

    # ---- contents ---------------------------------------------------------
    Hq, Hkv, D = num_heads, num_kv_heads, head_dim
    query = _draw(rng, (S, Hq, D), dtype)
    src = np.asarray(rec_src, dtype=np.int64)
    fresh = np.nonzero(src < 0)[0]
    R = len(rec_slot)
    kdt = np.uint16 if dtype == "bf16" else np.float32
    rec_key = np.empty((R, Hkv, D), dtype=kdt)
    rec_value = np.empty((R, Hkv, D), dtype=kdt)
    rec_key[fresh] = _draw(rng, (len(fresh), Hkv, D), dtype)
    rec_value[fresh] = _draw(rng, (len(fresh), Hkv, D), dtype)
    dup = np.nonzero(src >= 0)[0]
    rec_key[dup] = rec_key[src[dup]]
    rec_value[dup] = rec_value[src[dup]]

    return Workload(
        name=name, dtype=dtype, num_seqs=S, num_heads=Hq, num_kv_heads=Hkv,
        head_dim=D, block_size=BS, num_blocks=int(num_blocks), max_blocks_per_seq=int(MB),
        scale=float(scale if scale is not None else 1.0 / math.sqrt(D)),
        query=query, block_table=table, context_lens=lens,
        rec_key=rec_key, rec_value=rec_value,
        rec_slot=np.asarray(rec_slot, dtype=np.int64),
        seq_records=[np.asarray(r, dtype=np.int64) for r in seq_records],
        new_records=np.asarray(new_records, dtype=np.int64),
        partition_size=partition_size,
        blocks_allocated=int(np.count_nonzero(pool.refcount)),
        info={"seed": seed, "shared_prefix_len": int(shared_prefix_len)},
        cow_pairs=np.asarray(cow_pairs, dtype=np.int64).reshape(-1, 2),
        cow_records=np.nonzero(src >= 0)[0].astype(np.int64),
    )


# ---------------------------------------------------------------------------
CONFIG_NAMES = {
    0: "tiny-f32",
    1: "llama3-8b-decode-bf16",
    2: "continuous-batching-mix-bf16",
    3: "prefix-sharing-bf16",
    4: "llama3-70b-long-context-bf16",
}


def make_config(index: int, *, seed: int | None = None, block_size: int | None = None,
                variant: str | None = None) -> Workload:
    """The five named workloads; ``seed`` defaults to the config index."""
    seed = index if seed is None else seed
    rng = np.random.default_rng(seed)
    if index == 0:
        return make_workload(name=CONFIG_NAMES[0], context_lens=[5, 17, 33, 64],
                             num_heads=4, num_kv_heads=4, head_dim=64, block_size=16,
                             dtype="f32", seed=seed, rng=rng, scale=1.0 / 8.0,
                             num_blocks=64, max_blocks_per_seq=4)
    if index == 1:
        lens = rng.integers(128, 2048 + 1, size=64)
        return make_workload(name=CONFIG_NAMES[1], context_lens=lens, num_heads=32,
                             num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
                             seed=seed, rng=rng, max_blocks_per_seq=2048 // 16)
    if index == 2:
        BS = 16 if block_size is None else block_size
        S, n_long = 256, 26          # 10% of 256, rounded: an exact count
        is_long = np.zeros(S, dtype=bool)
        is_long[rng.permutation(S)[:n_long]] = True
        lens = np.where(is_long, rng.integers(2000, 8192 + 1, size=S),
                        rng.integers(50, 400 + 1, size=S))
        w = make_workload(name=f"{CONFIG_NAMES[2]}-bs{BS}", context_lens=lens, num_heads=32,
                          num_kv_heads=8, head_dim=128, block_size=BS, dtype="bf16",
                          seed=seed, rng=rng, max_blocks_per_seq=-(-8192 // BS))
        return w
    if index == 3:
        variant = variant or "prefix"
        if variant == "prefix":
            suffix = rng.integers(32, 512 + 1, size=128)
            return make_workload(name=f"{CONFIG_NAMES[3]}-prefix", context_lens=1024 + suffix,
                                 num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                                 dtype="bf16", seed=seed, rng=rng, shared_prefix_len=1024)
        if variant == "parallel-sampling":
            prompts = rng.integers(32, 512 + 1, size=32)
            return make_workload(name=f"{CONFIG_NAMES[3]}-parallel-sampling",
                                 context_lens=prompts, num_heads=32, num_kv_heads=8,
                                 head_dim=128, block_size=16, dtype="bf16", seed=seed,
                                 rng=rng, samples_per_prompt=4)
        raise ValueError(f"unknown variant {variant!r}")
    if index == 4:
        lens = rng.integers(16384, 32768 + 1, size=16)
        return make_workload(name=CONFIG_NAMES[4], context_lens=lens, num_heads=64,
                             num_kv_heads=8, head_dim=128, block_size=32, dtype="bf16",
                             seed=seed, rng=rng, max_blocks_per_seq=32768 // 32,
                             partition_size=512)
    raise ValueError(f"no config {index}")


# ---------------------------------------------------------------------------
# prefill chunks: the last n tokens of each sequence are new query tokens
# ---------------------------------------------------------------------------
@dataclass
class PrefillBatch:
    """New query tokens of a workload's sequences (their K/V records are in the workload).

    Sequence s owns rows query_start_loc[s] .. query_start_loc[s+1] - 1 of ``query``; they
    are its last n_s context positions, whose K/V records are ``chunk_records`` (in row
    order).  Every other record is history already in the pool.
    """
    query: np.ndarray               # [T, Hq, D]
    query_start_loc: np.ndarray     # [S + 1] int32
    chunk_records: np.ndarray       # [T] int64
    max_query_len: int

    def history_records(self, w: Workload) -> np.ndarray:
        mask = np.ones(len(w.rec_slot), dtype=bool)
        mask[self.chunk_records] = False
        return np.nonzero(mask)[0]


def make_prefill(w: Workload, chunk_lens, seed: int) -> PrefillBatch:
    """Chunks of chunk_lens[s] new tokens at the end of each sequence of ``w``."""
    n = np.minimum(np.asarray(chunk_lens, dtype=np.int64), w.context_lens.astype(np.int64))
    qsl = np.zeros(w.num_seqs + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(n)
    recs = np.concatenate([w.seq_records[s][len(w.seq_records[s]) - n[s]:]
                           for s in range(w.num_seqs)]) if w.num_seqs else np.zeros(0, np.int64)
    rng = np.random.default_rng([seed, 7919])
    query = _draw(rng, (int(qsl[-1]), w.num_heads, w.head_dim), w.dtype)
    return PrefillBatch(query=query, query_start_loc=qsl, chunk_records=recs.astype(np.int64),
                        max_query_len=int(n.max()) if len(n) else 0)


PREFILL_NAMES = {
    "prefix-cache-prefill": "the prefix-sharing batch; each sequence's private suffix "
                            "(32..512 tokens) is prefilled over the cached 1024-token prefix",
    "chunked-prefill-llama3-8b": "the Llama-3-8B-shaped batch; the last min(L, 512) tokens of "
                                 "each sequence are one prefill chunk",
}


def make_prefill_config(name: str, seed: int | None = None):
    """(workload, prefill batch) of a named prefill case."""
    if name == "prefix-cache-prefill":
        w = make_config(3, seed=seed)
        return w, make_prefill(w, w.context_lens.astype(np.int64) - 1024, w.info["seed"])
    if name == "chunked-prefill-llama3-8b":
        w = make_config(1, seed=seed)
        return w, make_prefill(w, np.minimum(w.context_lens, 512), w.info["seed"])
    raise ValueError(f"no prefill case {name!r}")
