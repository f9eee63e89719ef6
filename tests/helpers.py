"""Shared helpers of the GPU parity tests: running the HIP path through the C
ABI, running the oracle on the same inputs, and the tolerance of each dtype."""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch

import oracle
from transformer_attention_variant_amd import binding
from transformer_attention_variant_amd import inputs as I

# Tolerances, element by element: 1e-4 in float32; in bfloat16 2e-2 times the
# RMS of the oracle's output, plus the bf16 unit roundoff (2^-8) times the
# element's own magnitude.  The second term is the rounding of the result to the
# output format, which the float64 oracle does not have: near 4-5 x RMS one
# bf16 step is already as large as 2e-2 x RMS, so without it the bar would
# measure the output format rather than the computation.  One rule for every
# bf16 case.
F32_TOL = 1e-4
BF16_REL_TOL = 2e-2
BF16_UNIT_ROUNDOFF = 2.0 ** -8


def to_dev(inp: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
    return {k: v.cuda() for k, v in inp.items()}


def run_gpu(cfg: I.MTAConfig, inp: Dict[str, torch.Tensor], dev=None) -> torch.Tensor:
    dev = dev or to_dev(inp)
    out = binding.forward_cfg(cfg, dev)
    torch.cuda.synchronize()
    return out


def tolerance(cfg: I.MTAConfig, ref: np.ndarray):
    """The bar of each compared element (a scalar in float32, an array like
    ``ref`` in bfloat16)."""
    if cfg.dtype == "f32":
        return F32_TOL
    return bf16_tolerance(ref)


def bf16_tolerance(ref: np.ndarray) -> np.ndarray:
    ref = ref.astype(np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    return BF16_REL_TOL * rms + BF16_UNIT_ROUNDOFF * np.abs(ref)


def compare(cfg: I.MTAConfig, got: torch.Tensor, ref: np.ndarray, mask: Optional[np.ndarray] = None,
            what: str = "") -> Tuple[float, float]:
    g = got.detach().cpu().double().numpy()
    if mask is not None:
        g, ref = g[mask], ref[mask]
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    assert np.isfinite(ref).all(), f"{what}: non-finite oracle output"
    if not g.size:
        return 0.0, 0.0
    diff = np.abs(g - ref)
    tol = np.broadcast_to(tolerance(cfg, ref), diff.shape)
    worst = int(np.argmax(diff - tol))
    err = float(diff.flat[worst])
    assert diff.flat[worst] <= tol.flat[worst], \
        f"{what} {cfg.short()}: abs err {err:.3e} > tol {float(tol.flat[worst]):.3e} at flat index {worst} " \
        f"(max abs err {float(diff.max()):.3e})"
    # the margin of the closest element: its error and its bar
    return err, float(tol.flat[worst])


def sample_plan(cfg: I.MTAConfig, n_units: int = 2, rows: int = 64) -> Tuple[Sequence[Tuple[int, int]], Sequence[int]]:
    """Row ranges (start, middle, end of the sequence) and (b, group) units to
    check at full size; the middle range straddles a 64-row tile boundary."""
    T = cfg.T
    mid = max(0, min(T - rows, T // 2 - rows // 2 - 7))
    ranges = sorted({(0, min(rows, T)), (mid, mid + min(rows, T)), (max(0, T - rows), T)})
    U = cfg.B * cfg.groups
    units = sorted({0, U - 1} if n_units >= 2 else {U - 1})
    return ranges, units


def oracle_sampled(cfg: I.MTAConfig, inp, ranges, units) -> Tuple[np.ndarray, np.ndarray]:
    """Oracle output on the sampled rows/units (NaN elsewhere) and the mask of
    the sampled entries."""
    ref = np.full((cfg.B, cfg.H, cfg.T, cfg.d), np.nan)
    mask = np.zeros(ref.shape, dtype=bool)
    for (r0, r1) in ranges:
        o = oracle.forward_cfg(cfg, inp, rows=(r0, r1), units=units, chunk=16)
        for u in units:
            b, g = divmod(u, cfg.groups)
            hs = slice(g * cfg.c_h, (g + 1) * cfg.c_h)
            ref[b, hs, r0:r1] = o[b, hs, r0:r1]
            mask[b, hs, r0:r1] = True
    return ref, mask
