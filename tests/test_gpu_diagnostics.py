"""GPU: the two diagnostics beside the decode path run and compute what they claim.

* pa_read_probe reads every listed piece exactly once: the XOR of its checksums equals the
  XOR of every 32-bit word of the pieces, computed on the host, for the in-order and the
  shuffled piece lists and both load policies.
* pa_coexec_probe runs every mode at 4 and 8 waves per workgroup, writes one finite value
  per thread, and gives the same values on a second launch.  Its placement mode shows the
  placement the split mode relies on: the four waves 0..3 of an 8-wave workgroup run on
  four different SIMDs, and wave w + 4 on the SIMD of wave w.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_425_amd as pk

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("in_flight", [4, 8, 16])
@pytest.mark.parametrize("nontemporal", [False, True])
def test_read_probe_reads_every_piece_once(in_flight, nontemporal):
    rng = np.random.default_rng(1500 + in_flight)
    piece = 4096
    n = 48 * in_flight                                   # whole groups of pieces
    host = rng.integers(0, 1 << 32, size=(n + 7) * piece // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.uint8)).to(DEV)
    want = np.bitwise_xor.reduce(host[: n * piece // 4].reshape(n, -1), axis=None)
    for order in ("stream", "gather"):
        idx = np.arange(n) if order == "stream" else rng.permutation(n)
        offs = torch.from_numpy((idx * piece).astype(np.int64)).to(DEV)
        for wgs in (1, 7, 64):
            say(f"read probe {order} in_flight={in_flight} nt={nontemporal} workgroups={wgs}")
            sink = torch.zeros(wgs * 256, dtype=torch.int32, device=DEV)
            pk.read_probe(buf, offs, piece, wgs, in_flight, sink, nontemporal=nontemporal)
            torch.cuda.synchronize()
            got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
            assert got == want


@pytest.mark.parametrize("waves", [4, 8])
def test_coexec_probe_runs_every_mode(waves):
    wgs = 3
    for mode in ("mfma", "valu", "interleaved", "split"):
        say(f"coexec probe {mode} waves={waves}")
        a = torch.full((wgs * waves * 64,), float("nan"), dtype=torch.float32, device=DEV)
        b = torch.full_like(a, float("nan"))
        pk.coexec_probe(mode, wgs, waves, 64, a)
        pk.coexec_probe(mode, wgs, waves, 64, b)
        torch.cuda.synchronize()
        assert torch.isfinite(a).all()
        assert torch.equal(a, b)


def test_coexec_probe_placement():
    wgs, waves = 16, 8
    say(f"coexec probe placement workgroups={wgs} waves={waves}")
    out = torch.full((wgs * waves * 64,), -1.0, dtype=torch.float32, device=DEV)
    pk.coexec_probe("placement", wgs, waves, 1, out)
    torch.cuda.synchronize()
    simd = out.cpu().numpy().reshape(wgs, waves, 64)
    assert (simd == simd[:, :, :1]).all()              # one SIMD per wave
    first = simd[:, :, 0].astype(np.int64)
    assert set(np.unique(first)) <= {0, 1, 2, 3}
    for w in first:
        assert sorted(w[:4]) == [0, 1, 2, 3]
        assert (w[4:] == w[:4]).all()
