"""Non-causal joint self-attention, float64. Test infrastructure only.

The plain definition of scaled dot-product attention ("Attention Is All You
Need", in the xDiT paper's reference list) applied to the whole joint
sequence: every query row attends to every key row, text and image alike, with
no mask (the xDiT abstract: attention over long image/video token sequences is
the growing cost). The flash/online-softmax form (FlashAttention-2, same
reference list) reaches this same result; the oracle does not tile keys.

Rows are independent, so the oracle processes query rows in blocks only to
bound memory. ``rows`` selects a subset of query rows for sampled checks at
large sizes; each selected row still sees every key.
"""
from __future__ import annotations

import math

import numpy as np

from .rope import rope_apply

_ROW_BLOCK = 2048


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be rank 4: [B, H, S, D]")
    if q.shape[:2] != k.shape[:2] or k.shape[:3] != v.shape[:3] or q.shape[3] != k.shape[3]:
        raise ValueError("q [B,H,Sq,D], k [B,H,Sk,D], v [B,H,Sk,Dv] shapes disagree")


def _scores(qb: np.ndarray, kh: np.ndarray, scale: float) -> np.ndarray:
    return scale * (qb @ kh.T)


def softmax_probs(q, k, scale, rows=None):
    """P = softmax(scale * q k^T) per (b, h): [B, H, R, S_k]. For small inputs."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    B, H = q.shape[:2]
    rsel = np.arange(q.shape[2]) if rows is None else np.asarray(rows)
    out = np.empty((B, H, len(rsel), k.shape[2]))
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, h, rsel], k[b, h], scale)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            out[b, h] = p / p.sum(axis=1, keepdims=True)
    return out


def attention(q, k, v, scale=None, rows=None, return_lse=False):
    """softmax(scale * q k^T) v, float64, [B, H, R, Dv] (R = all rows or ``rows``).

    With ``return_lse`` also returns the natural-log row log-sum-exp of the
    scaled scores, [B, H, R].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    _check(q, k, v)
    B, H, S_q, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rsel = np.arange(S_q) if rows is None else np.asarray(rows)
    out = np.empty((B, H, len(rsel), v.shape[3]))
    lses = np.empty((B, H, len(rsel)))
    for b in range(B):
        for h in range(H):
            kh, vh = k[b, h], v[b, h]
            for r0 in range(0, len(rsel), _ROW_BLOCK):
                idx = rsel[r0:r0 + _ROW_BLOCK]
                s = _scores(q[b, h, idx], kh, scale)
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                denom = p.sum(axis=1, keepdims=True)
                out[b, h, r0:r0 + len(idx)] = (p @ vh) / denom
                lses[b, h, r0:r0 + len(idx)] = (m + np.log(denom))[:, 0]
    return (out, lses) if return_lse else out


def lse(q, k, scale=None):
    return attention(q, k, np.zeros(k.shape[:3] + (1,)), scale, return_lse=True)[1]


def joint_attention(q, k, v, angles=None, scale=None, rows=None):
    """RoPE on Q and K (when ``angles`` is given), then attention. V is not rotated.

    q, k, v: [B, H, S, D] (any float dtype; promoted to float64).
    angles: [S, D/2] float64 from ``rope_angles``, or None for no RoPE.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    rsel = None if rows is None else np.asarray(rows)
    if rsel is not None:
        q = q[:, :, rsel]
    if angles is not None:
        q = rope_apply(q, angles if rsel is None else angles[rsel])
        k = rope_apply(k, angles)
    return attention(q, k, v, scale)
