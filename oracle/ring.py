"""Blockwise attention with row log-sum-exp, and the exact merge of partial
results. Test infrastructure only.

Ring attention ("Ring Attention with Blockwise Transformers for Near-Infinite
Context", in the xDiT paper page's reference list; the xDiT runner
configuration in the MXFP4/Quark on MI350 blog carries a ring degree) splits
the keys of a sequence into blocks held by different ranks. A rank attends its
query shard to one key/value block at a time and folds the partial results
together.

The partial result over key block b is O_b = softmax over the keys of b,
applied to V_b, together with the row log-sum-exp L_b = log sum_{j in b}
exp(s_ij) of the scaled scores s_ij. Softmax over the union of the blocks
gives block b the total weight exp(L_b) / sum_c exp(L_c), so the merged row is

    O = sum_b exp(L_b - L) O_b,   L = log sum_b exp(L_b),

which is exact by the definition of softmax; this module writes it out for two
partial results. RoPE is applied to a query shard with the shard's positions
and to a key block with the block's positions (the rotation depends only on a
token's own position), so a block result needs both angle tables.
"""
from __future__ import annotations

import numpy as np

from .attention import attention
from .rope import rope_apply


def block_attention(q, k, v, q_angles=None, k_angles=None, scale=None, rows=None):
    """Attention of query rows q [B, H, Sq, D] over one key/value block
    k, v [B, H, Sk, D]; q rotated with q_angles [Sq, D/2], k with k_angles
    [Sk, D/2] (both None: no RoPE). Returns (O [B, H, R, D], L [B, H, R]),
    float64, L the natural-log row log-sum-exp of the scaled scores."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    if (q_angles is None) != (k_angles is None):
        raise ValueError("give both angle tables or neither")
    rsel = None if rows is None else np.asarray(rows)
    if rsel is not None:
        q = q[:, :, rsel]
    if q_angles is not None:
        q = rope_apply(q, q_angles if rsel is None else np.asarray(q_angles)[rsel])
        k = rope_apply(k, k_angles)
    return attention(q, k, v, scale, return_lse=True)


def merge_lse(o_a, l_a, o_b, l_b):
    """Fold two partial results over disjoint key blocks: (O, L) as above.
    A row with L = -inf on one side (an empty block) takes the other side."""
    o_a = np.asarray(o_a, np.float64)
    o_b = np.asarray(o_b, np.float64)
    l_a = np.asarray(l_a, np.float64)
    l_b = np.asarray(l_b, np.float64)
    L = np.logaddexp(l_a, l_b)
    w_a = np.exp(l_a - L)[..., None]
    w_b = np.exp(l_b - L)[..., None]
    return w_a * o_a + w_b * o_b, L
