"""The range-clipping calibrators of "Building a From-Scratch Group-Wise INT4
Quantization Layer for LLaMA Weights", Step 4, evaluated group by group with
the PyTorch calls that step names (torch.quantile, torch.linspace, float32
division, round, clamp, F.mse_loss).  Test infrastructure: these give the
values the oracle's calibrators must reproduce bit for bit.  They run on one
group at a time and are slow by design."""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def _group(vals) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(vals, np.float32)))


def percentile(vals, p: float) -> np.float32:
    """The "percentile" calibrator: torch.quantile of |w| at p / 100."""
    return np.float32(torch.quantile(_group(vals).abs(), p / 100).item())


def mse_search(vals, n: int) -> np.float32:
    """The "mse" calibrator for one group: the candidate steps are
    torch.linspace(min|w|, max|w|, n); a step below 1e-10 is passed over; a
    step's error is F.mse_loss between the group and its reconstruction from
    codes round(w / step) clamped to [-7, 7]; a later step replaces the one
    held only with a strictly smaller error; 1e-8 if no step is eligible."""
    w = _group(vals)
    mags = w.abs()
    steps = torch.linspace(mags.min(), mags.max(), n)
    held, held_err = None, None
    for i in range(n):
        step = steps[i]
        if bool(step < 1e-10):
            continue
        recon = torch.clamp(torch.round(w / step), -7, 7) * step
        err = F.mse_loss(recon, w)
        if held is None or bool(err < held_err):
            held, held_err = i, err
    return np.float32(1e-8) if held is None else np.float32(steps[held].item())
