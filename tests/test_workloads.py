"""The seeded input generator: shapes, positions reading, bf16 rounding (no GPU)."""
import numpy as np
import pytest
import torch

import dit_workloads as W


def test_sequence_lengths():
    assert W.get("tiny").S == 320
    assert W.get("flux1024x768").S == 3584
    assert W.get("flux2048").S == 16896
    assert W.get("video_ulysses4").S == 76112
    assert W.get("flux2048_fp8").S == 16896
    for w in W.WORKLOADS.values():
        assert sum(w.axes_dim) == w.D == 128
        assert len(w.axes_dim) == len(w.grid)


def test_flops_formula():
    assert W.get("flux2048").flops == 4 * 24 * 16896 ** 2 * 128 == 3507914539008


def test_positions_text_zero_then_raster():
    w = W.get("flux1024x768")
    pos = W.positions(w)
    assert pos.shape == (3584, 3) and pos.dtype == np.int32
    assert not pos[:512].any()
    # token 512 + r*64 + c is image row r, column c (48 rows x 64 columns)
    for r, c in [(0, 0), (0, 63), (1, 0), (47, 63), (20, 33)]:
        assert tuple(pos[512 + r * 64 + c]) == (0, r, c)
    v = W.get("video_ulysses4")
    pv = W.positions(v)
    t, h, x = 13, 44, 79
    assert tuple(pv[512 + (t * 45 + h) * 80 + x]) == (t, h, x)
    tiny = W.positions(W.get("tiny"))
    assert tuple(tiny[64 + 5 * 16 + 9]) == (5, 9)


def test_bf16_round_to_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -1.0 - 2 ** -8, 3.0], np.float32)
    got = W.bf16_bits_to_f32(W.bf16_round_bits(x))
    assert got.tolist() == [1.0, 1.015625, 1.0078125, -1.0, 3.0]
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 100
    ref = torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.bf16_round_bits(r), ref)


def test_draws_are_seeded_and_ordered():
    w = W.get("tiny")
    a = W.make_bf16_inputs(w)
    b = W.make_bf16_inputs(w)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    q, k, v = W.draw_qkv_f32(w)
    rng = np.random.default_rng(1001)
    assert np.array_equal(q, rng.standard_normal((1, 2, 320, 128), dtype=np.float32))
    assert abs(float(q.std()) - 1.0) < 0.02


def test_fp8_quantize_roundtrip():
    x = np.random.default_rng(1).standard_normal(4096).astype(np.float32)
    codes, scale = W.fp8_e4m3_quantize(x)
    assert codes.dtype == np.uint8 and scale == np.float32(np.abs(x).max() / 448.0)
    deq = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy() * scale
    # e4m3 has 3 mantissa bits: relative error at most 2^-4 for normal codes
    big = np.abs(x) > scale * 2 ** -6
    assert np.all(np.abs(deq - x)[big] <= np.abs(x)[big] * 2 ** -4 + 1e-12)
    assert np.max(np.abs(deq)) == pytest.approx(np.abs(x).max(), rel=1e-6)
