"""Pure-Python scalar version of RoPE + joint attention. Test infrastructure only.

Written loop by loop from the definitions (see ``oracle.rope`` and
``oracle.attention``), with ``math.cos``/``math.sin``/``math.exp`` and
``math.fsum``, so that it shares no numpy code with the vectorised oracle. It
is meant for tiny inputs (S <= 16 with small D, or D = 128 with S <= 4).
"""
from __future__ import annotations

import math


def angle(pos_row, axes_dim, theta, pair):
    """Angle of global pair index ``pair`` for one token's coordinates."""
    offset = 0
    for a, d_a in enumerate(axes_dim):
        if pair < offset + d_a // 2:
            i = pair - offset
            return pos_row[a] * theta ** (-2.0 * i / d_a)
        offset += d_a // 2
    raise IndexError(pair)


def rotate_row(x_row, pos_row, axes_dim, theta):
    out = list(x_row)
    for j in range(len(x_row) // 2):
        a = angle(pos_row, axes_dim, theta, j)
        c, s = math.cos(a), math.sin(a)
        x0, x1 = x_row[2 * j], x_row[2 * j + 1]
        out[2 * j] = x0 * c - x1 * s
        out[2 * j + 1] = x0 * s + x1 * c
    return out


def joint_attention(q, k, v, pos=None, axes_dim=None, theta=10000.0, scale=None):
    """q, k, v: nested lists [B][H][S][D]; pos: [S][n_axes] or None (no RoPE)."""
    B, H, S, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = []
    for b in range(B):
        ob = []
        for h in range(H):
            qs = [list(map(float, r)) for r in q[b][h]]
            ks = [list(map(float, r)) for r in k[b][h]]
            vs = [list(map(float, r)) for r in v[b][h]]
            if pos is not None:
                qs = [rotate_row(qs[i], pos[i], axes_dim, theta) for i in range(S)]
                ks = [rotate_row(ks[i], pos[i], axes_dim, theta) for i in range(S)]
            oh = []
            for i in range(S):
                s = [scale * math.fsum(qs[i][d] * ks[j][d] for d in range(D)) for j in range(S)]
                m = max(s)
                p = [math.exp(x - m) for x in s]
                z = math.fsum(p)
                oh.append([math.fsum(p[j] * vs[j][e] for j in range(S)) / z for e in range(len(vs[0]))])
            ob.append(oh)
        out.append(ob)
    return out


def row_lse(q, k, pos_q=None, pos_k=None, axes_dim=None, theta=10000.0, scale=None):
    """Natural-log log-sum-exp of each query row's scaled scores, nested lists
    [B][H][Sq] from q [B][H][Sq][D] and k [B][H][Sk][D]; pos_q / pos_k are the
    token coordinates of the rows (both None: no RoPE)."""
    B, H, Sq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = []
    for b in range(B):
        ob = []
        for h in range(H):
            qs = [list(map(float, r)) for r in q[b][h]]
            ks = [list(map(float, r)) for r in k[b][h]]
            if pos_q is not None:
                qs = [rotate_row(qs[i], pos_q[i], axes_dim, theta) for i in range(Sq)]
                ks = [rotate_row(ks[j], pos_k[j], axes_dim, theta) for j in range(len(ks))]
            oh = []
            for i in range(Sq):
                s = [scale * math.fsum(qs[i][d] * ks[j][d] for d in range(D)) for j in range(len(ks))]
                m = max(s)
                oh.append(m + math.log(math.fsum(math.exp(x - m) for x in s)))
            ob.append(oh)
        out.append(ob)
    return out


def residual_diff(prev, cur):
    """The DBCache relative L1 difference of two flat residuals, scalar loops."""
    den = math.fsum(abs(float(p)) for p in prev)
    num = math.fsum(abs(float(c) - float(p)) for p, c in zip(prev, cur))
    return math.inf if den == 0.0 else num / den
