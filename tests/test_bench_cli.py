"""CPU: the host-side parts of bench.py that need no GPU.

* `--gpus N` with N > 1 exits with status 2 and says that only one GPU is measured, before
  anything touches a device;
* `--help` names every `--op` the driver and the profiles use;
* the balanced-pairs rearrangement keeps the longer half of the lengths and gives each its
  partner so that the pair holds twice the mean;
* a traffic record counts only when it names the workload and was taken on the current
  kernel source (its digest), else the bench line reports `traffic: null`.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*argv: str) -> subprocess.CompletedProcess:
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_help_names_every_op():
    r = _run("--help")
    assert r.returncode == 0
    text = " ".join(r.stdout.split())
    for op in ("step", "copy_blocks", "prefill", "fp8", "swap", "ceiling", "math", "balance",
               "coexec", "writes", "suffixes"):
        assert f"{op}:" in text, op                           # the op and its description


def test_balanced_pair_lengths():
    rng = np.random.default_rng(7)
    for n in (2, 7, 64):
        lens = rng.integers(128, 2049, size=n)
        out = bench.balanced_pair_lengths(lens)
        assert out.shape == lens.shape and (out >= 1).all()
        total = 2 * int(round(float(lens.mean())))
        head = n - n // 2
        assert (out[:head] == np.sort(lens)[::-1][:head]).all()      # the longer half kept
        for r in range(n // 2):
            assert out[r] + out[n - 1 - r] == total or out[n - 1 - r] == 1


def test_traffic_record_needs_the_current_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    wl = "some-workload"
    rec = {"workload": wl, "bytes_per_launch": 12345, "source_sha256": bench.source_digest()}
    path = tmp_path / f"traffic_{wl}.json"
    path.write_text(json.dumps(rec))
    assert bench.load_traffic(wl) == 12345
    path.write_text(json.dumps(dict(rec, source_sha256="0" * 64)))
    assert bench.load_traffic(wl) is None                     # another kernel
    path.write_text(json.dumps(dict(rec, workload="other")))
    assert bench.load_traffic(wl) is None                     # another workload
    path.write_text("not json")
    assert bench.load_traffic(wl) is None
    assert bench.load_traffic("missing") is None
