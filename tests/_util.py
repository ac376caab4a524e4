"""Helpers shared by the tests (not a test module)."""
from __future__ import annotations

import numpy as np

import rvq_inputs as RI


def analytic_first_frame(cfg: dict, n: int) -> int:
    """Earliest frame that output sample n depends on (walk back through the
    layers: causal conv i -> i - (k-1) d; transposed conv i -> floor(i/s) - 1;
    windowed attention i -> i - (window - 1) per layer)."""
    i = n - 6
    for s in reversed(cfg["strides"]):
        i -= 18
        i -= 6
        i = i // s - 1
    i -= 6
    i -= cfg["tf_layers"] * max(cfg["tf_window"] - 1, 0)
    return i


def analytic_left_context(cfg: dict) -> int:
    H = RI.hop(cfg)
    return max(n // H - analytic_first_frame(cfg, n) for n in range(4 * H, 5 * H))


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    """max|gpu - ref| / max|ref| (the bar) and / max|ref - mean(ref)| (reported)."""
    err = float(np.max(np.abs(gpu.astype(np.float64) - ref)))
    peak = float(np.max(np.abs(ref)))
    ac = float(np.max(np.abs(ref - ref.mean())))
    return err / peak, err / max(ac, 1e-300)


def tol_for(cfg: dict) -> float:
    return 2e-3 if cfg["weight_dtype"] == "bf16" else 1e-5


def host_weights(cfg: dict, w: dict) -> dict:
    """What the GPU library is given: bf16 bit patterns or fp32 arrays."""
    return RI.weight_bits(w) if cfg["weight_dtype"] == "bf16" else w
