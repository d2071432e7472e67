"""CPU: the paired mode's host plan (pa_plan_pairs), which the decode calls make from
host_context_lens and the kernel makes again from context_lens when no host copy is given.

* Pairs: pair r holds the r-th longest and the r-th shortest sequence of the clamped
  lengths, ties to the lower index; every sequence is in exactly one pair; an odd count
  leaves the middle sequence alone (sB = 0xFFFF).
* Blocks: each unit's table entries to stage, ceil(L / BS) of its clamped length.
* Waves: with two units, the first keeps between 1 and waves - 1 waves, and the split is
  the first that minimises the larger of the two units' steps per unit of wave weight
  (weights 3, 2, 3, 2, ... by rank at 8 waves, 1 each at 4); a single unit keeps all.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import paged_kv_cache_425_amd as pk

NONE = 0xFFFF


def weight(rank: int, waves: int) -> int:
    return (3 if rank % 2 == 0 else 2) if waves == 8 else 1


def unpack(plan):
    x, y = plan[:, 0].astype(np.int64), plan[:, 1].astype(np.int64)
    return x & 0xFFFF, x >> 16, y & 0xFFF, (y >> 12) & 0xFFF, y >> 24


def cases():
    rng = np.random.default_rng(2024)
    yield "uniform", rng.integers(1, 2049, size=64)
    yield "ties", rng.choice([0, 16, 17, 500], size=33)
    yield "past-the-clamp", np.concatenate([rng.integers(0, 9000, size=40), [-5, 10 ** 6]])
    yield "two", np.array([3, 3])
    yield "three", np.array([0, 9, 1])
    yield "many", rng.integers(0, 8193, size=512)


@pytest.mark.parametrize("waves,step", [(8, 32), (4, 32), (8, 64), (8, 16)])
@pytest.mark.parametrize("BS", [8, 16, 32])
def test_plan_pairs(waves, step, BS):
    cap = 8192
    for name, lens in cases():
        lens = np.asarray(lens, dtype=np.int64)
        S = lens.size
        plan = pk.plan_pairs(lens, BS, cap, step, waves)
        sA, sB, bA, bB, nA = unpack(plan)
        L = np.clip(lens, 0, cap)
        order = sorted(range(S), key=lambda t: (-L[t], t))       # longest first, ties by index
        npairs = (S + 1) // 2
        assert plan.shape == (npairs, 2), name
        seen = []
        for r in range(npairs):
            assert sA[r] == order[r], (name, r)
            if r == S - 1 - r:
                assert sB[r] == NONE and bB[r] == 0 and nA[r] == waves, (name, r)
            else:
                assert sB[r] == order[S - 1 - r], (name, r)
                seen.append(int(sB[r]))
            seen.append(int(sA[r]))
            assert bA[r] == -(-L[sA[r]] // BS), (name, r)
            if sB[r] != NONE:
                assert bB[r] == -(-L[sB[r]] // BS), (name, r)
        assert sorted(seen) == list(range(S)), name
        for r in range(npairs):
            if sB[r] == NONE:
                continue
            stA, stB = -(-L[sA[r]] // step), -(-L[sB[r]] // step)

            def cost(c):
                capA = sum(weight(k, waves) for k in range(c))
                capB = sum(weight(k, waves) for k in range(c, waves))
                return max(Fraction(int(stA), capA), Fraction(int(stB), capB))

            best = min(range(1, waves), key=lambda c: (cost(c), c))
            assert nA[r] == best, (name, r, stA, stB)


def test_plan_pairs_needs_a_valid_call():
    with pytest.raises(ValueError):
        pk.plan_pairs(np.zeros((2, 2)), 16, 8192, 32, 8)
    for bad in (dict(block_size=12), dict(max_len=8193), dict(max_len=-1), dict(waves=6),
                dict(step_tokens=0)):
        args = dict(block_size=16, max_len=8192, step_tokens=32, waves=8)
        args.update(bad)
        with pytest.raises(ValueError):
            pk.plan_pairs([1, 2, 3], **args)
    with pytest.raises(ValueError):
        pk.plan_pairs([1], 16, 8192, 32, 8)                       # one sequence: no pairs
    with pytest.raises(ValueError):
        pk.plan_pairs(np.ones(513), 16, 8192, 32, 8)              # more than 512
