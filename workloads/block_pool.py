"""Host-side physical block pool with reference counts and copy-on-write.

This is the bookkeeping the pages attach to the paged KV cache, done on the
host so that synthetic workloads can be laid out the way a serving engine
would lay them out:

* the cache is cut into fixed-size physical blocks that are handed out on
  demand, one more whenever a sequence's last block is full
  ("core architecture" page, section 2.2.1 table and the on-demand-allocation
  bullet; "core inference engine" page, section 2.2);
* a sequence's block table maps its logical blocks to physical ones, and
  producing a token appends one mapping ("core features" page, section 4.1);
* several sequences may point at the same physical block (a shared system
  prompt, parallel sampling, beam search: "core features" page 4.1,
  "core architecture" page 2.2.1, "architecture & core features" page 3.1).

Reference counts and copy-on-write are the plainest way to keep shared blocks
correct when one of the sharers appends into a partially filled block; the
pages imply them through sharing but do not spell them out.

Free blocks are handed out in the order of one seeded random permutation of
the pool, so physical placement is scattered and reproducible.

Nothing here computes attention; the module only produces integer tables.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


class PoolExhausted(RuntimeError):
    """Raised when an allocation finds no free physical block."""


class BlockPool:
    """A pool of ``num_blocks`` physical blocks with per-block reference counts."""

    def __init__(self, num_blocks: int, rng: np.random.Generator):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        self.num_blocks = int(num_blocks)
        # free list: one seeded random permutation, handed out front to back
        self._free = [int(b) for b in rng.permutation(self.num_blocks)]
        self._free.reverse()  # pop() from the end == take from the front
        self.refcount = np.zeros(self.num_blocks, dtype=np.int64)

    @property
    def num_free(self) -> int:
        return len(self._free)

    def allocate(self) -> int:
        if not self._free:
            raise PoolExhausted(
                f"no free physical block left in a pool of {self.num_blocks}")
        b = self._free.pop()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def share(self, block: int) -> None:
        if self.refcount[block] <= 0:
            raise ValueError(f"block {block} is not allocated")
        self.refcount[block] += 1

    def release(self, block: int) -> None:
        if self.refcount[block] <= 0:
            raise ValueError(f"block {block} released more often than held")
        self.refcount[block] -= 1
        if self.refcount[block] == 0:
            self._free.append(block)

    def utilisation(self, tokens_stored: int, block_size: int) -> float:
        """Stored tokens over the token capacity of all allocated blocks."""
        used = int(np.count_nonzero(self.refcount))
        return tokens_stored / max(1, used * block_size)


@dataclass
class SequenceBlocks:
    """One sequence's logical-to-physical block list and token count."""
    blocks: list = field(default_factory=list)
    num_tokens: int = 0

    def fork(self, pool: BlockPool) -> "SequenceBlocks":
        """A new sequence that shares every block of this one."""
        for b in self.blocks:
            pool.share(b)
        return SequenceBlocks(blocks=list(self.blocks), num_tokens=self.num_tokens)


@dataclass
class SlotWrite:
    """Where the next token of a sequence goes, plus any copy it needs first.

    ``copy_from`` / ``copy_to`` name a physical block whose stored tokens must
    be duplicated before the write (copy-on-write); both are -1 otherwise.
    """
    slot: int
    copy_from: int = -1
    copy_to: int = -1


def append_token(seq: SequenceBlocks, pool: BlockPool, block_size: int) -> SlotWrite:
    """Reserve the slot of ``seq``'s next token (allocating or copying a block).

    slot = physical_block * block_size + offset_in_block.
    """
    pos = seq.num_tokens
    logical = pos // block_size
    offset = pos % block_size
    copy_from = copy_to = -1
    if logical == len(seq.blocks):
        seq.blocks.append(pool.allocate())
    else:
        phys = seq.blocks[logical]
        if pool.refcount[phys] > 1:
            # the last block is shared and partially filled: copy before writing
            new = pool.allocate()
            pool.release(phys)
            seq.blocks[logical] = new
            copy_from, copy_to = phys, new
    seq.num_tokens += 1
    return SlotWrite(slot=seq.blocks[logical] * block_size + offset,
                     copy_from=copy_from, copy_to=copy_to)
