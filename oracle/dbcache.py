"""The DBCache reuse decision, float64. Test infrastructure only.

The AMD RDNA 4 xDiT blog (section "Skip Transformer Work Only When the Model
Has Enough Steps") enables DBCache step caching with a residual diff
threshold (0.12 in its example): consecutive denoising steps produce similar
transformer outputs, and after the first Fn blocks of a step the cache
decides whether the rest of the step can reuse the previous step's work. A
higher threshold allows more reuse. The page names the threshold but not the
formula; the reading here is the relative L1 difference of the residuals that
the first blocks produce in the previous and the current step,

    diff = sum_i |cur_i - prev_i| / sum_i |prev_i|,    reuse = diff < threshold,

with diff = +inf (never reuse) when the previous residual is all zero.
"""
from __future__ import annotations

import math

import numpy as np


def residual_diff(prev, cur) -> float:
    prev = np.asarray(prev, np.float64).ravel()
    cur = np.asarray(cur, np.float64).ravel()
    if prev.shape != cur.shape:
        raise ValueError("residuals must have the same size")
    den = float(np.sum(np.abs(prev)))
    num = float(np.sum(np.abs(cur - prev)))
    return math.inf if den == 0.0 else num / den


def can_reuse(prev, cur, threshold: float) -> bool:
    return residual_diff(prev, cur) < threshold
