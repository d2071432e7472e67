"""Moving workloads and pools between NumPy (oracle side) and the GPU."""
from __future__ import annotations

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_dev(arr: np.ndarray, dtype: str, dev) -> torch.Tensor:
    """Upload float32 values or bf16 bit patterns (uint16) without any rounding."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a device tensor, for bit-exact comparisons."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.cpu().numpy()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def upload_inputs(w, dev) -> dict:
    return {
        "query": to_dev(w.query, w.dtype, dev),
        "block_table": torch.from_numpy(w.block_table).to(dev),
        "context_lens": torch.from_numpy(w.context_lens).to(dev),
    }


# bf16 outputs: the absolute bound holds where bf16 can meet it.  From |x| = 4 up, half a
# bf16 ulp is 2^-6 = 0.0156 > 1e-2, so even the exact result rounded to bf16 (the output
# format) can miss 1e-2 there; the relative bound governs those elements.
BF16_ABS_LIMIT = 4.0


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    """The parity bar: f32 max |err| <= 1e-5; bf16 max |err| <= 1e-2 wherever |ref| < 4,
    and |err| / |ref| <= 2e-2 wherever |ref| >= 1e-2.  Below 1e-2 the relative error of
    N(0,1) data near zero crossings is meaningless and the absolute bound governs; from 4
    up the output format's own rounding (half an ulp, 0.0156 at 4) exceeds 1e-2 and the
    relative bound governs."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    stats = {"max_abs": float(err.max()) if err.size else 0.0}
    if dtype == "f32":
        assert stats["max_abs"] <= 1e-5, f"{what}: max abs err {stats['max_abs']:.3e} > 1e-5"
    else:
        mag = np.abs(ref)
        big = mag >= 1e-2
        rel = err[big] / mag[big]
        stats["max_rel"] = float(rel.max()) if rel.size else 0.0
        small = err[mag < BF16_ABS_LIMIT]
        stats["max_abs_below_4"] = float(small.max()) if small.size else 0.0
        assert stats["max_abs_below_4"] <= 1e-2, \
            f"{what}: max abs err {stats['max_abs_below_4']:.3e} > 1e-2 (|ref| < 4)"
        assert stats["max_rel"] <= 2e-2, f"{what}: max rel err {stats['max_rel']:.3e} > 2e-2"
    return stats
