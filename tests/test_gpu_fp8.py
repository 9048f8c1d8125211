"""Parity of the fp8 (OCP e4m3, per-tensor scales) path with the float64 oracle
on the dequantised inputs.

Gates for unit-variance data quantised per tensor: max |gpu - oracle| <= 5e-2,
mean <= 5e-3, and mean|diff| / mean|oracle| <= 8%.  The relative gate comes
from the arithmetic: besides the inputs, the path rounds three things to e4m3
(3 mantissa bits, RMS relative error 2^-4 / sqrt(3) ~ 3.6%): the rotated K', the
rotated and scaled Q'' and the weights P.  The first two move each base-2
logit by ~ sqrt(2) * 3.6% of its size (|s| ~ 1.5 here), i.e. a weight by
~ ln2 * 0.076 ~ 5%; with P's own 3.6% the weights move by ~ 6% RMS, which
averages down in O but not below a few percent of |O|.  Short sequences (S <= 256)
average few V rows, so |O| is O(1): there e4m3's 2^-4 relative rounding of the
re-quantised Q'', K' and of P dominates and the gates are max(5e-2, 2^-2 max|O|)
and max(5e-3, 2^-4 mean|O|).  The same holds for sharpened logits (Q x 3): the
softmax then puts its mass on a few keys, so O is again a short average of V
rows, and the logit error (proportional to |s|) grows threefold; those cases
take the |O|-relative gates too, with the same 8% relative-mean gate.
"""
import math

import numpy as np
import pytest

import dit_workloads as W
from oracle import joint_attention, rope_angles
from oracle.fp8 import dequantize
from tests.gpu_inputs import err_stats, from_device_bf16, sample_rows, tile_rows

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, REL_MEAN = 5e-2, 5e-3, 8e-2


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _quantized(w, qmul=1.0):
    q, k, v = W.draw_qkv_f32(w)
    return [W.fp8_e4m3_quantize(x) for x in (q * qmul, k, v)]


def _run(w, qkv8, rope=True, split=False, scale=None):
    torch = _torch()
    import dit_joint_self_amd as dj
    (q8, sq), (k8, sk), (v8, sv) = qkv8
    dev = lambda c: torch.from_numpy(np.ascontiguousarray(c)).to("cuda")
    q, k, v = dev(q8), dev(k8), dev(v8)
    cos = sin = None
    if rope:
        cos, sin = dj.dit_rope_tables(torch.from_numpy(W.positions(w)).to("cuda"), w.axes_dim, w.theta)
    if split:
        nb = dj.dit_attn_workspace_bytes_fp8(w.B, w.H, w.S, w.D)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
        dj.dit_attn_prepare_kv_fp8(k, v, sk, sv, cos, sin, ws)
        dj.dit_attn_core_fp8(q, sq, cos, sin, ws, out, scale=scale)
    else:
        out = dj.dit_attn_forward_fp8(q, k, v, sq, sk, sv, cos, sin, S_txt=w.S_txt, scale=scale)
    torch.cuda.synchronize()
    return from_device_bf16(out)


def _oracle(w, qkv8, rope=True, rows=None, scale=None):
    (q8, sq), (k8, sk), (v8, sv) = qkv8
    ang = rope_angles(W.positions(w), w.axes_dim, w.theta) if rope else None
    return joint_attention(dequantize(q8, sq), dequantize(k8, sk), dequantize(v8, sv), ang, scale=scale, rows=rows)


def _assert_close(got, want, tag, few_rows=False):
    e = err_stats(got, want)
    print(f"[fp8 parity] {tag}: {e}", flush=True)
    assert np.all(np.isfinite(got)), tag
    mg, ng = MAX_ABS, MEAN_ABS
    if few_rows:
        mg = max(MAX_ABS, 0.25 * float(np.abs(want).max()))
        ng = max(MEAN_ABS, 2.0 ** -4 * float(np.abs(want).mean()))
    assert e["max_abs"] <= mg and e["mean_abs"] <= ng and e["rel_mean"] <= REL_MEAN, (tag, e)


@pytest.mark.parametrize("name", ["tiny", "flux1024x768"])
def test_fp8_full_parity(name):
    w = W.get(name)
    qkv8 = _quantized(w)
    _assert_close(_run(w, qkv8), _oracle(w, qkv8), name)


def test_fp8_whole_ranges_and_key_range_pieces_in_one_launch():
    """37 heads x ceil(1800 / 256) = 296 items: 256 whole-range workgroups and 40
    items x 6 key ranges in one launch of the fp8 kernel (its two wave groups
    half a tile apart), with 8-row and 8-key tails; every row compared."""
    w = W.Workload("edge8", B=1, H=37, D=128, S_txt=0, grid=(30, 60), axes_dim=(64, 64), theta=10000.0, seed=1801)
    qkv8 = _quantized(w)
    want = _oracle(w, qkv8)
    for split in (False, True):
        _assert_close(_run(w, qkv8, split=split), want, f"S={w.S} H={w.H} split={split}")


def test_fp8_every_element_flux2048():
    """The fp8 variant of the 2048 x 2048 FLUX shape (24 heads of 16896 tokens)
    in the benchmark's launch configuration: every output against the oracle
    on the dequantised inputs."""
    w = W.get("flux2048_fp8")
    qkv8 = _quantized(w)
    got = _run(w, qkv8)
    _assert_close(got, _oracle(w, qkv8), f"flux2048_fp8 every element ({got.size} outputs)")


def test_fp8_every_query_tile_video_share():
    """The video head share (10 heads of 76112 tokens) on the fp8 path: first,
    last and two random rows of every 256-row query tile of every head."""
    w = W.get("video_ulysses4")
    (q8, sq), (k8, sk), (v8, sv) = qkv8 = _quantized(w)
    got = _run(w, qkv8)
    assert np.all(np.isfinite(got))
    ang = rope_angles(W.positions(w), w.axes_dim, w.theta)
    gots, wants = [], []
    for h in range(w.H):
        rows = tile_rows(w.S, seed=w.seed * 100 + 50 + h)
        sl = slice(h, h + 1)
        wants.append(joint_attention(dequantize(q8[:, sl], sq), dequantize(k8[:, sl], sk), dequantize(v8[:, sl], sv),
                                     ang, rows=rows))
        gots.append(got[:, sl][:, :, rows])
    _assert_close(np.concatenate(gots, axis=2), np.concatenate(wants, axis=2),
                  f"fp8 video_ulysses4 ({sum(x.shape[2] for x in gots)} rows over {w.H} heads)")


@pytest.mark.parametrize("sign", [-1.0, 1.0])
def test_fp8_scale_of_either_sign(sign):
    """A negative softmax scale on the fp8 path: the Q re-quantisation step is
    chosen from the magnitude of scale * log2(e), so Q'' keeps its codes in the
    normal e4m3 range for either sign.  3 heads of 1000 tokens."""
    w = W.Workload("edge8", B=1, H=3, D=128, S_txt=24, grid=(16, 61), axes_dim=(64, 64), theta=10000.0, seed=91)
    qkv8 = _quantized(w)
    scale = sign / math.sqrt(128)
    want = _oracle(w, qkv8, scale=scale)
    for split in (False, True):
        _assert_close(_run(w, qkv8, split=split, scale=scale), want, f"fp8 scale {scale:+.4f} split={split}")


@pytest.mark.parametrize("S_txt,grid,B,H", [(1, (0, 0), 1, 1), (0, (1, 31), 1, 1), (2, (1, 31), 1, 1),
                                            (0, (7, 9), 1, 2), (1, (8, 8), 1, 3), (13, (12, 20), 1, 2),
                                            (64, (16, 16), 2, 2)])
def test_fp8_ragged_and_small(S_txt, grid, B, H):
    """Includes single-tile sequences shorter than the 32-query MFMA block
    (S = 1, 31, 33): the query lanes past S must still feed every MFMA."""
    w = W.Workload("edge8", B=B, H=H, D=128, S_txt=S_txt, grid=grid, axes_dim=(64, 64), theta=10000.0,
                   seed=77 + S_txt)
    qkv8 = _quantized(w)
    want = _oracle(w, qkv8)
    for split in (False, True):
        _assert_close(_run(w, qkv8, split=split), want, f"S={w.S} split={split}", few_rows=w.S <= 256)


def test_fp8_no_rope_and_sharper_logits():
    w = W.get("tiny").with_(H=2)
    qkv8 = _quantized(w, qmul=3.0)
    _assert_close(_run(w, qkv8, rope=False), _oracle(w, qkv8, rope=False), "no-rope q*3", few_rows=True)


def test_fp8_deterministic_and_forward_equals_split():
    w = W.get("tiny")
    qkv8 = _quantized(w)
    a, b, c = _run(w, qkv8), _run(w, qkv8), _run(w, qkv8, split=True)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_fp8_bitwise_repeatable_with_tile_loop():
    """Repeated calls agree bit for bit on a shape where every workgroup runs
    the pipelined tile loop (56 key tiles) and the key-range split and merge
    run too (3584 tokens x 24 heads = 336 query tiles).  LDS loads landing in
    the operand registers of still-queued fp8 MFMAs once made a version of
    this kernel vary from run to run by up to 6e-2, inside the oracle gates,
    so the parity tests alone did not show it."""
    w = W.get("flux1024x768")
    qkv8 = _quantized(w)
    a = _run(w, qkv8, split=True)
    for _ in range(3):
        assert np.array_equal(a, _run(w, qkv8, split=True))
    assert np.array_equal(a, _run(w, qkv8))


def test_fp8_bitwise_repeatable_full_size():
    """flux2048_fp8: three calls agree bit for bit."""
    torch = _torch()
    import dit_joint_self_amd as dj
    w = W.get("flux2048_fp8")
    (q8, sq), (k8, sk), (v8, sv) = _quantized(w)
    dev = lambda c: torch.from_numpy(np.ascontiguousarray(c)).to("cuda")
    q, k, v = dev(q8), dev(k8), dev(v8)
    cos, sin = dj.dit_rope_tables(torch.from_numpy(W.positions(w)).to("cuda"), w.axes_dim, w.theta)
    outs = [dj.dit_attn_forward_fp8(q, k, v, sq, sk, sv, cos, sin, S_txt=w.S_txt) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


def test_fp8_longest_supported_sequence():
    """S = 2^21 on the fp8 path (one head): the last fp8 tiles sit just below
    the 32-bit byte offsets of the tile addressing.  Sampled rows, including
    the last tile's."""
    torch = _torch()
    import dit_joint_self_amd as dj
    w = W.Workload("max8", B=1, H=1, D=128, S_txt=0, grid=(1, 1024, 2048), axes_dim=(16, 56, 56), theta=10000.0,
                   seed=2022)
    assert w.S == 2 ** 21
    qkv8 = _quantized(w)
    got_all = _run(w, qkv8)
    rows = np.unique(np.concatenate([sample_rows(w.S, 0, 16, seed=4), [2 ** 20, w.S - 64, w.S - 2, w.S - 1]]))
    _assert_close(got_all[:, :, rows], _oracle(w, qkv8, rows=rows), f"fp8 S=2^21 ({len(rows)} rows)")
