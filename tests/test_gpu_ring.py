"""Ring-attention building blocks on the GPU (dit_attn_core_lse, dit_attn_merge_lse)
against the float64 oracle (oracle.ring), through the C ABI.

Gates.
* O after a ring of key blocks: the bf16 attention gates (max 1e-2, mean 1e-3,
  relative mean 1%), since each block's O carries the attention kernel's error
  and the merge adds one bf16 rounding (relative 2^-8, bf16's unit roundoff)
  of values of size |O|.
* Row log-sum-exp L: a score on the GPU is scale * sum_d q'_d k'_d with q'
  (times scale * log2 e) and k' each rounded to bf16 (relative error <= 2^-8),
  so a logit moves by at most 2^-7 * scale * sum_d |q'_d k'_d|; for
  unit-variance rows with D = 128 that sum is about 0.64 * 128 * scale = 7.2,
  i.e. 0.056. L moves by the softmax-weighted average of its row's logit
  errors, and the weight sum l (bf16 weights) by at most 2^-8 = 0.004
  relative: max |dL| <= 0.06. Rounding errors of random sign average down
  over the dims and the keys; the mean gate 3e-3 is ten times the means
  observed. Gates: max |dL| <= 6e-2, mean |dL| <= 3e-3.
* The merge alone, on the GPU's own partial results: fp32 arithmetic and one
  bf16 RNE rounding, so |out - exact| <= 2^-8 |exact| + 1e-6 element-wise and
  |L_out - exact| <= 1e-5 (1 + |exact|).
"""
import math

import numpy as np
import pytest

import dit_workloads as W
from oracle import block_attention, joint_attention, merge_lse, rope_angles
from tests.gpu_inputs import bf16_f64, err_stats, from_device_bf16, sample_rows, to_device_bf16

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, REL_MEAN = 1e-2, 1e-3, 1e-2
LSE_MAX, LSE_MEAN = 6e-2, 3e-3


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _dj():
    import dit_joint_self_amd as dj
    return dj


def _tables(w, rows):
    torch = _torch()
    pos = torch.from_numpy(np.ascontiguousarray(W.positions(w)[rows])).to("cuda")
    return _dj().dit_rope_tables(pos, w.axes_dim, w.theta)


def _block_result(w, q, k, v, qrows, krows):
    """(O, L) on the GPU of query rows qrows over the key/value block krows
    (each rotated with its own positions); tensors on the device."""
    torch = _torch()
    dj = _dj()
    n = len(qrows)
    assert len(krows) == n
    cq, sq = _tables(w, qrows)
    ck, sk = _tables(w, krows)
    ws = torch.empty(dj.dit_attn_workspace_bytes(w.B, w.H, n, w.D), dtype=torch.uint8, device="cuda")
    kk = k[:, :, krows[0]:krows[-1] + 1].contiguous()
    vv = v[:, :, krows[0]:krows[-1] + 1].contiguous()
    qq = q[:, :, qrows[0]:qrows[-1] + 1].contiguous()
    dj.dit_attn_prepare_k(kk, ck, sk, ws)
    out = torch.empty_like(qq)
    return dj.dit_attn_core_lse(qq, vv, cq, sq, ws, out)


def _lse_close(got, want, tag):
    d = np.abs(got - want)
    print(f"[lse parity] {tag}: max {d.max():.3g} mean {d.mean():.3g}", flush=True)
    assert np.all(np.isfinite(got)), tag
    assert d.max() <= LSE_MAX and d.mean() <= LSE_MEAN, (tag, float(d.max()), float(d.mean()))


def _o_close(got, want, tag):
    e = err_stats(got, want)
    print(f"[ring parity] {tag}: {e}", flush=True)
    assert np.all(np.isfinite(got)), tag
    assert e["max_abs"] <= MAX_ABS and e["mean_abs"] <= MEAN_ABS and e["rel_mean"] <= REL_MEAN, (tag, e)


@pytest.mark.parametrize("name,S_txt,grid,B,H", [("tiny", None, None, None, None),
                                                 ("edge", 1, (0, 0), 1, 1),      # S = 1: L = the one score
                                                 ("edge", 1, (4, 8), 1, 2),      # S = 33, one ragged tile
                                                 ("edge", 13, (12, 20), 2, 2),   # S = 253, split key ranges
                                                 ("edge", 0, (8, 8), 1, 256),    # 256 items: one whole round
                                                 ("edge", 0, (30, 60), 2, 20)])  # 320 items: round + 64 x 4 pieces
def test_core_lse_matches_oracle(name, S_txt, grid, B, H):
    torch = _torch()
    dj = _dj()
    if name == "tiny":
        w = W.get("tiny")
    else:
        w = W.Workload("edge", B=B, H=H, D=128, S_txt=S_txt, grid=grid, axes_dim=(64, 64), theta=10000.0,
                       seed=300 + S_txt)
    qb, kb, vb = W.make_bf16_inputs(w)
    q, k, v = to_device_bf16(qb), to_device_bf16(kb), to_device_bf16(vb)
    rows = np.arange(w.S)
    out, lse = _block_result(w, q, k, v, rows, rows)
    out_plain = torch.empty_like(out)
    cos, sin = _tables(w, rows)
    ws = torch.empty(dj.dit_attn_workspace_bytes(w.B, w.H, w.S, w.D), dtype=torch.uint8, device="cuda")
    dj.dit_attn_prepare_k(k, cos, sin, ws)
    dj.dit_attn_core(q, v, cos, sin, ws, out_plain)
    torch.cuda.synchronize()
    # the LSE variant writes the same O as the plain call
    assert torch.equal(out.view(torch.int16), out_plain.view(torch.int16))
    ang = rope_angles(W.positions(w), w.axes_dim, w.theta)
    o_ref, l_ref = block_attention(bf16_f64(qb), bf16_f64(kb), bf16_f64(vb), ang, ang)
    got_l = lse.cpu().numpy().astype(np.float64)
    _lse_close(got_l, l_ref, f"{name} S={w.S}")
    if w.S == 1:  # a single key: L is its scaled score
        q1 = bf16_f64(qb)[:, :, 0]
        k1 = bf16_f64(kb)[:, :, 0]
        s = np.einsum("bhd,bhd->bh", q1, k1) / math.sqrt(w.D)   # position 0: RoPE is the identity
        assert np.max(np.abs(got_l[:, :, 0] - s)) <= LSE_MAX
    e = err_stats(from_device_bf16(out), o_ref)
    assert e["max_abs"] <= max(MAX_ABS, 0.25 * float(np.abs(o_ref).max())), e


def _ring_fold(w, q, k, v, qrows, blocks, inplace):
    dj = _dj()
    o = l = None
    for krows in blocks:
        ob, lb = _block_result(w, q, k, v, qrows, krows)
        if o is None:
            o, l = ob, lb
        elif inplace:
            dj.dit_attn_merge_lse(o, l, ob, lb, out=o, lse_out=l)
        else:
            o, l = dj.dit_attn_merge_lse(o, l, ob, lb)
    return o, l


@pytest.mark.parametrize("name,P", [("tiny", 2), ("flux1024x768", 2), ("flux1024x768", 4)])
def test_ring_of_blocks_equals_joint_attention(name, P):
    """Each of the P query shards attends to all P key/value blocks in ring
    order; the folded result equals attention over the whole joint sequence."""
    torch = _torch()
    w = W.get(name)
    assert w.S % P == 0
    n = w.S // P
    qb, kb, vb = W.make_bf16_inputs(w)
    q, k, v = to_device_bf16(qb), to_device_bf16(kb), to_device_bf16(vb)
    ang = rope_angles(W.positions(w), w.axes_dim, w.theta)
    blocks = [np.arange(b * n, (b + 1) * n) for b in range(P)]
    for r in range(P):
        qrows = blocks[r]
        order = blocks[r:] + blocks[:r]               # the ring: own block first, then the others in turn
        o, l = _ring_fold(w, q, k, v, qrows, order, inplace=(r % 2 == 0))
        torch.cuda.synchronize()
        sel = qrows if w.S <= 4096 else qrows[sample_rows(n, 0, 24, seed=r)]
        want_o = joint_attention(bf16_f64(qb), bf16_f64(kb), bf16_f64(vb), ang, rows=sel)
        _, want_l = block_attention(bf16_f64(qb), bf16_f64(kb), bf16_f64(vb), ang, ang, rows=sel)
        loc = sel - qrows[0]
        _o_close(from_device_bf16(o)[:, :, loc], want_o, f"{name} P={P} shard {r}")
        _lse_close(l.cpu().numpy().astype(np.float64)[:, :, loc], want_l, f"{name} P={P} shard {r}")


def test_merge_alone_matches_exact_fold_and_in_place():
    """The merge kernel on the GPU's own partial results against the exact fold
    of those same values; in-place folding gives the same bits."""
    torch = _torch()
    dj = _dj()
    w = W.get("tiny")
    n = w.S // 2
    qb, kb, vb = W.make_bf16_inputs(w)
    q, k, v = to_device_bf16(qb), to_device_bf16(kb), to_device_bf16(vb)
    rows_a, rows_b = np.arange(n), np.arange(n, w.S)
    oa, la = _block_result(w, q, k, v, rows_a, rows_a)
    ob, lb = _block_result(w, q, k, v, rows_a, rows_b)
    out, lo = dj.dit_attn_merge_lse(oa, la, ob, lb)
    oa2, la2 = oa.clone(), la.clone()
    dj.dit_attn_merge_lse(oa2, la2, ob, lb, out=oa2, lse_out=la2)
    ob2, lb2 = ob.clone(), lb.clone()
    dj.dit_attn_merge_lse(oa, la, ob2, lb2, out=ob2, lse_out=lb2)
    torch.cuda.synchronize()
    want_o, want_l = merge_lse(from_device_bf16(oa), la.cpu().numpy(), from_device_bf16(ob), lb.cpu().numpy())
    got_o = from_device_bf16(out)
    assert np.all(np.abs(got_o - want_o) <= 2.0 ** -8 * np.abs(want_o) + 1e-6)
    got_l = lo.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got_l - want_l) <= 1e-5 * (1.0 + np.abs(want_l)))
    for o2, l2 in ((oa2, la2), (ob2, lb2)):
        assert torch.equal(o2.view(torch.int16), out.view(torch.int16)) and torch.equal(l2, lo)


def test_ring_full_size_sampled():
    """flux2048 (S = 16896) as a ring of two ranks: shard 1 over both blocks,
    sampled rows against the oracle."""
    _torch()
    w = W.get("flux2048")
    n = w.S // 2
    qb, kb, vb = W.make_bf16_inputs(w)
    q, k, v = to_device_bf16(qb), to_device_bf16(kb), to_device_bf16(vb)
    blocks = [np.arange(0, n), np.arange(n, w.S)]
    qrows = blocks[1]
    o, l = _ring_fold(w, q, k, v, qrows, [blocks[1], blocks[0]], inplace=True)
    sel = qrows[sample_rows(n, 0, 32, seed=5)]
    ang = rope_angles(W.positions(w), w.axes_dim, w.theta)
    want_o, want_l = block_attention(bf16_f64(qb), bf16_f64(kb), bf16_f64(vb), ang, ang, rows=sel)
    loc = sel - n
    _o_close(from_device_bf16(o)[:, :, loc], want_o, "flux2048 P=2 shard 1")
    _lse_close(l.cpu().numpy().astype(np.float64)[:, :, loc], want_l, "flux2048 P=2 shard 1")
