"""Multi-axis rotary position embedding, float64. Test infrastructure only.

The pages never define RoPE. They name its users (FLUX.1-dev in the AMD
MXFP4-with-Quark-on-MI350 blog, FLUX.2 / Wan 2.2 in the AMD RDNA 4 xDiT
blog, section "How to Scale Diffusion Inference Across AMD RDNA 4 GPUs") and
nothing of its form. This file takes the plainest reading:

* the head dimension D is split into consecutive per-axis blocks of
  ``axes_dim[a]`` dims (for example 16/56/56 for text-index/height/width);
* inside axis a, local pair i (0 <= i < d_a/2) has angular frequency
  omega_i = theta ** (-2 i / d_a), and its angle at a token is
  pos[token, a] * omega_i;
* pair j of the head (j = offset_a/2 + i) rotates dims (2j, 2j+1) as the
  complex number x[2j] + i x[2j+1] multiplied by exp(i * angle).
"""
from __future__ import annotations

import numpy as np


def rope_angles(pos: np.ndarray, axes_dim, theta: float) -> np.ndarray:
    """Angles in float64, shape [S, sum(axes_dim)/2].

    pos: integer [S, n_axes] token coordinates (text tokens all 0).
    """
    pos = np.asarray(pos)
    if pos.ndim != 2 or pos.shape[1] != len(axes_dim):
        raise ValueError("pos must be [S, n_axes]")
    blocks = []
    for a, d_a in enumerate(axes_dim):
        if d_a % 2:
            raise ValueError("each axis needs an even number of dims")
        i = np.arange(d_a // 2, dtype=np.float64)
        omega = np.power(np.float64(theta), -2.0 * i / d_a)
        blocks.append(pos[:, a].astype(np.float64)[:, None] * omega[None, :])
    return np.concatenate(blocks, axis=1)


def rope_apply(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate interleaved pairs of x [..., S, D] by angles [S, D/2], float64."""
    x = np.asarray(x, dtype=np.float64)
    c = np.cos(angles)
    s = np.sin(angles)
    even = x[..., 0::2]
    odd = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out
