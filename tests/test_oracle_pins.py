"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: a
pure-Python brute force, torch's float64 SDPA, a complex-number RoPE,
hand-derived closed forms (tests/golden/closed_forms.json) or an invariant
that the mathematics fixes.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, brute, joint_attention, rope_angles, rope_apply, softmax_probs

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _as4(x):
    return np.asarray(x, np.float64)[None, None]


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("B,H,S,D,axes", [
    (1, 2, 7, 8, (4, 4)),
    (2, 1, 16, 6, (2, 2, 2)),
    (1, 1, 3, 128, (16, 56, 56)),
    (1, 1, 4, 128, (64, 64)),
    (1, 1, 4, 128, (44, 42, 42)),
])
def test_brute_force_matches(B, H, S, D, axes):
    rng = np.random.default_rng(S * 100 + D)
    q, k, v = _rand(rng, B, H, S, D), _rand(rng, B, H, S, D), _rand(rng, B, H, S, D)
    pos = rng.integers(0, 9, size=(S, len(axes)))
    scale = 0.7 / math.sqrt(D) * 3
    got = joint_attention(q, k, v, rope_angles(pos, axes, 10000.0), scale=scale)
    want = np.array(brute.joint_attention(q.tolist(), k.tolist(), v.tolist(), pos.tolist(), axes, 10000.0, scale))
    assert np.max(np.abs(got - want)) <= 1e-12


def test_brute_force_no_rope_default_scale():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 1, 2, 9, 12), _rand(rng, 1, 2, 9, 12), _rand(rng, 1, 2, 9, 5)
    got = joint_attention(q, k, v)
    want = np.array(brute.joint_attention(q.tolist(), k.tolist(), v.tolist()))
    assert np.max(np.abs(got - want)) <= 1e-12


# ---------------------------------------------------------------- library routines

@pytest.mark.parametrize("scale", [None, 0.3])
def test_attention_matches_torch_sdpa_fp64(scale):
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 2, 3, 37, 16), _rand(rng, 2, 3, 53, 16), _rand(rng, 2, 3, 53, 8)
    got = attention(q, k, v, scale=scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=scale).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(12)
    S, axes = 40, (16, 56, 56)
    pos = rng.integers(0, 128, size=(S, 3))
    ang = rope_angles(pos, axes, 10000.0)
    x = _rand(rng, 2, 3, S, 128)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * ang)
    want = np.empty_like(x)
    want[..., 0::2], want[..., 1::2] = z.real, z.imag
    assert np.max(np.abs(rope_apply(x, ang) - want)) <= 1e-12


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("case", ["attention_3key", "attention_uniform"])
def test_golden_attention(case):
    g = GOLDEN[case]
    out = attention(_as4(g["q"]), _as4(g["k"]), _as4(g["v"]), scale=g["scale"])[0, 0]
    assert np.max(np.abs(out - np.array(g["out"]))) <= 1e-12
    if "probs" in g:
        p = softmax_probs(_as4(g["q"]), _as4(g["k"]), g["scale"])[0, 0]
        assert np.max(np.abs(p - np.array(g["probs"]))) <= 1e-15


def test_golden_rope_angles():
    g = GOLDEN["rope_angles"]
    for c in g["cases"]:
        ang = rope_angles(np.array([c["pos"]]), c["axes_dim"], g["theta"])
        assert abs(ang[0, c["pair"]] - c["angle"]) <= 1e-12, c


def test_golden_rope_rotation():
    g = GOLDEN["rope_rotation"]
    out = rope_apply(np.array([[g["x"]]]), np.array([[g["angle"]]]))
    assert np.max(np.abs(out[0, 0] - np.array(g["out"]))) <= 1e-15


# ---------------------------------------------------------------- invariants

def _joint(rng, S=24, D=32, axes=(8, 12, 12), H=2):
    q, k, v = _rand(rng, 1, H, S, D), _rand(rng, 1, H, S, D), _rand(rng, 1, H, S, D)
    pos = rng.integers(0, 20, size=(S, len(axes)))
    return q, k, v, pos, axes


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(20)
    p = softmax_probs(_rand(rng, 1, 2, 17, 8) * 3, _rand(rng, 1, 2, 29, 8) * 3, 0.9)
    assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-14
    assert np.all(p >= 0)


def test_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(21)
    q = _rand(rng, 1, 1, 6, 8)
    k = np.repeat(_rand(rng, 1, 1, 1, 8), 10, axis=2)
    v = _rand(rng, 1, 1, 10, 8)
    out = attention(q, k, v)
    assert np.max(np.abs(out - v.mean(axis=2, keepdims=True))) <= 1e-14
    # with RoPE: all tokens at one position (text tokens) rotate identically
    ang = rope_angles(np.zeros((10, 2), int), (4, 4), 10000.0)
    out2 = joint_attention(_rand(rng, 1, 1, 10, 8), k, v, ang)
    assert np.max(np.abs(out2 - v.mean(axis=2, keepdims=True))) <= 1e-14


def test_scale_zero_gives_mean_of_v():
    rng = np.random.default_rng(22)
    q, k, v, pos, axes = _joint(rng)
    out = joint_attention(q, k, v, rope_angles(pos, axes, 10000.0), scale=0.0)
    assert np.max(np.abs(out - v.mean(axis=2, keepdims=True))) <= 1e-14


def test_constant_v_gives_constant():
    rng = np.random.default_rng(23)
    q, k, v, pos, axes = _joint(rng)
    v[:] = 0.625
    out = joint_attention(q, k, v, rope_angles(pos, axes, 10000.0))
    assert np.max(np.abs(out - 0.625)) <= 1e-14


def test_single_token_returns_v():
    rng = np.random.default_rng(24)
    q, k, v = _rand(rng, 1, 3, 1, 128), _rand(rng, 1, 3, 1, 128), _rand(rng, 1, 3, 1, 128)
    ang = rope_angles(np.array([[0, 7, 3]]), (16, 56, 56), 10000.0)
    assert np.array_equal(joint_attention(q, k, v, ang), v)


def test_joint_kv_permutation_leaves_output_unchanged():
    rng = np.random.default_rng(25)
    q, k, v = _rand(rng, 1, 2, 9, 16), _rand(rng, 1, 2, 31, 16), _rand(rng, 1, 2, 31, 16)
    perm = rng.permutation(31)
    a = attention(q, k, v)
    b = attention(q, k[:, :, perm], v[:, :, perm])
    assert np.max(np.abs(a - b)) <= 1e-13


def test_token_permutation_with_positions_permutes_output():
    rng = np.random.default_rng(26)
    q, k, v, pos, axes = _joint(rng)
    perm = rng.permutation(q.shape[2])
    a = joint_attention(q, k, v, rope_angles(pos, axes, 10000.0))
    b = joint_attention(q[:, :, perm], k[:, :, perm], v[:, :, perm], rope_angles(pos[perm], axes, 10000.0))
    assert np.max(np.abs(a[:, :, perm] - b)) <= 1e-13


def test_shift_invariance_with_overflowing_logits():
    # adding the same vector c to every key adds q.c to a whole score row;
    # softmax must not change even when q.c alone would overflow exp
    rng = np.random.default_rng(27)
    q, k, v = _rand(rng, 1, 1, 5, 8), _rand(rng, 1, 1, 12, 8), _rand(rng, 1, 1, 12, 8)
    c = np.sign(q[0, 0].sum(0))[None, None, None, :] * 2000.0
    a = attention(q, k, v)
    b = attention(q, k + c, v)
    assert np.all(np.isfinite(b))
    assert np.max(np.abs(a - b)) <= 1e-9


def test_lse_merge_of_key_halves_equals_whole():
    rng = np.random.default_rng(28)
    q, k, v = _rand(rng, 1, 2, 7, 16), _rand(rng, 1, 2, 40, 16), _rand(rng, 1, 2, 40, 16)
    o, l = attention(q, k, v, return_lse=True)
    o1, l1 = attention(q, k[:, :, :17], v[:, :, :17], return_lse=True)
    o2, l2 = attention(q, k[:, :, 17:], v[:, :, 17:], return_lse=True)
    m = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - m)[..., None], np.exp(l2 - m)[..., None]
    merged = (w1 * o1 + w2 * o2) / (w1 + w2)
    assert np.max(np.abs(merged - o)) <= 1e-13
    assert np.max(np.abs(m + np.log(np.exp(l1 - m) + np.exp(l2 - m)) - l)) <= 1e-13


def test_linear_in_v():
    rng = np.random.default_rng(29)
    q, k = _rand(rng, 1, 1, 6, 8), _rand(rng, 1, 1, 11, 8)
    v1, v2 = _rand(rng, 1, 1, 11, 8), _rand(rng, 1, 1, 11, 8)
    a = attention(q, k, 2.5 * v1 - v2)
    b = 2.5 * attention(q, k, v1) - attention(q, k, v2)
    assert np.max(np.abs(a - b)) <= 1e-13


def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(30)
    x = _rand(rng, 1, 2, 5, 128)
    ang = rope_angles(np.zeros((5, 3), int), (16, 56, 56), 10000.0)
    assert np.array_equal(rope_apply(x, ang), x)


def test_rope_preserves_pair_norms_and_composes():
    rng = np.random.default_rng(31)
    x = _rand(rng, 1, 1, 8, 128)
    pa = rng.integers(0, 100, size=(8, 3))
    pb = rng.integers(0, 100, size=(8, 3))
    A, Bn = rope_angles(pa, (16, 56, 56), 10000.0), rope_angles(pb, (16, 56, 56), 10000.0)
    y = rope_apply(x, A)
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.max(np.abs(n0 - n1)) <= 1e-12
    # R(b) R(a) = R(a + b), and R(-a) undoes R(a)
    assert np.max(np.abs(rope_apply(y, Bn) - rope_apply(x, A + Bn))) <= 1e-11
    assert np.max(np.abs(rope_apply(y, -A) - x)) <= 1e-12
    # angles are linear in position, so R(a + b) is the rotation at position pa + pb
    assert np.max(np.abs(rope_angles(pa + pb, (16, 56, 56), 10000.0) - (A + Bn))) <= 1e-12


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_shifting_all_positions_on_an_axis_leaves_output_unchanged(axis):
    # <R_m q, R_n k> depends only on n - m
    rng = np.random.default_rng(32 + axis)
    q, k, v, pos, axes = _joint(rng, S=20, D=32, axes=(8, 12, 12))
    shifted = pos.copy()
    shifted[:, axis] += 37
    a = joint_attention(q, k, v, rope_angles(pos, axes, 10000.0))
    b = joint_attention(q, k, v, rope_angles(shifted, axes, 10000.0))
    assert np.max(np.abs(a - b)) <= 1e-12


def test_row_sampling_matches_full():
    rng = np.random.default_rng(33)
    q, k, v, pos, axes = _joint(rng, S=30)
    ang = rope_angles(pos, axes, 10000.0)
    full = joint_attention(q, k, v, ang)
    rows = np.array([0, 7, 29, 12])
    # BLAS may sum a row subset in another order: agree to rounding
    assert np.max(np.abs(joint_attention(q, k, v, ang, rows=rows) - full[:, :, rows])) <= 1e-14


def test_oracle_catches_planted_sign_error():
    # a plausible mistake (wrong sign on sin) must fail the complex-rotation pin
    rng = np.random.default_rng(34)
    x = _rand(rng, 1, 1, 6, 16)
    ang = rope_angles(rng.integers(1, 9, size=(6, 2)), (8, 8), 10000.0)
    c, s = np.cos(ang), np.sin(ang)
    bad = np.empty_like(x)
    bad[..., 0::2] = x[..., 0::2] * c + x[..., 1::2] * s
    bad[..., 1::2] = -x[..., 0::2] * s + x[..., 1::2] * c
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * ang)
    assert np.max(np.abs(bad[..., 0::2] - z.real)) > 1e-3
    assert np.max(np.abs(rope_apply(x, ang)[..., 0::2] - z.real)) <= 1e-12


# ---------------------------------------------------------------- fp8 decoding

def test_e4m3_decode_matches_torch_for_every_code():
    from oracle.fp8 import e4m3_decode
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_e4m3_decode_closed_forms():
    from oracle.fp8 import dequantize, e4m3_decode
    # 0x38 = 0 0111 000 -> 2^0; 0x7e = 0 1111 110 -> 1.75 * 2^8; 0x08 -> 2^-6 (smallest normal);
    # 0x01 -> 1/8 * 2^-6 (smallest subnormal); 0xc4 = 1 1000 100 -> -1.5 * 2
    got = e4m3_decode(np.array([0x38, 0x7e, 0x08, 0x01, 0xc4, 0x00, 0x80], np.uint8))
    assert got.tolist() == [1.0, 448.0, 2.0 ** -6, 2.0 ** -9, -3.0, 0.0, -0.0]
    assert np.isnan(e4m3_decode(np.array([0x7f, 0xff], np.uint8))).all()
    assert dequantize(np.array([0x40], np.uint8), 0.25).tolist() == [0.5]


# ---------------------------------------------------------------- ring blocks and the log-sum-exp merge

def _positions_2d(n, width):
    return np.stack([np.arange(n) // width, np.arange(n) % width], axis=1).astype(np.int64)


def test_block_lse_matches_brute_force_with_block_positions():
    from oracle import block_attention
    rng = np.random.default_rng(40)
    q, k, v = _rand(rng, 1, 2, 3, 8), _rand(rng, 1, 2, 5, 8), _rand(rng, 1, 2, 5, 8)
    pos_q = _positions_2d(3, 2) + np.array([1, 0])      # the query shard sits elsewhere in the grid
    pos_k = _positions_2d(5, 3)
    aq, ak = rope_angles(pos_q, (4, 4), 100.0), rope_angles(pos_k, (4, 4), 100.0)
    o, L = block_attention(q, k, v, aq, ak)
    want = brute.row_lse(q.tolist(), k.tolist(), pos_q.tolist(), pos_k.tolist(), (4, 4), 100.0)
    assert np.max(np.abs(L - np.array(want))) <= 1e-12
    # O of the block is ordinary attention of the rotated rows
    qr = np.array(brute.rotate_row(q[0, 1, 2].tolist(), pos_q[2].tolist(), (4, 4), 100.0))
    kr = np.array([brute.rotate_row(k[0, 1, j].tolist(), pos_k[j].tolist(), (4, 4), 100.0) for j in range(5)])
    s = kr @ qr / math.sqrt(8)
    p = np.exp(s - s.max())
    assert np.max(np.abs(o[0, 1, 2] - (p / p.sum()) @ v[0, 1])) <= 1e-12


def test_ring_blocks_merge_to_joint_attention():
    """Three uneven key blocks, each rotated with its own positions, folded in
    ring order: equal to attention over the whole joint sequence."""
    from oracle import block_attention, merge_lse
    rng = np.random.default_rng(41)
    S, D = 37, 16
    q, k, v = _rand(rng, 1, 2, S, D), _rand(rng, 1, 2, S, D), _rand(rng, 1, 2, S, D)
    pos = _positions_2d(S, 6)
    ang = rope_angles(pos, (8, 8), 10000.0)
    whole, L_whole = block_attention(q, k, v, ang, ang)
    bounds = [0, 9, 30, S]
    o = L = None
    for b0, b1 in zip(bounds[:-1], bounds[1:]):
        ob, lb = block_attention(q, k[:, :, b0:b1], v[:, :, b0:b1], ang, ang[b0:b1])
        o, L = (ob, lb) if o is None else merge_lse(o, L, ob, lb)
    assert np.max(np.abs(o - joint_attention(q, k, v, ang))) <= 1e-12
    assert np.max(np.abs(L - L_whole)) <= 1e-12
    # a fold that forgets to renormalise by the merged L fails
    o1, l1 = block_attention(q, k[:, :, :9], v[:, :, :9], ang, ang[:9])
    o2, l2 = block_attention(q, k[:, :, 9:], v[:, :, 9:], ang, ang[9:])
    wrong = 0.5 * (o1 + o2)
    assert np.max(np.abs(wrong - whole)) > 1e-3


def test_merge_lse_closed_forms():
    from oracle import merge_lse
    rng = np.random.default_rng(42)
    o, l = _rand(rng, 1, 2, 4, 8), rng.normal(size=(1, 2, 4))
    m, L = merge_lse(o, l, o, l)                          # a block merged with its copy
    assert np.max(np.abs(m - o)) <= 1e-15 and np.max(np.abs(L - (l + math.log(2.0)))) <= 1e-15
    m, L = merge_lse(o, l, 7.0 * o, np.full_like(l, -np.inf))   # empty second block
    assert np.array_equal(m, o) and np.array_equal(L, l)
    # two blocks of identical keys: weights in proportion to their sizes
    oa, ob = _rand(rng, 1, 1, 1, 8), _rand(rng, 1, 1, 1, 8)
    s = 0.7
    m, L = merge_lse(oa, np.array([[[s + math.log(3)]]]), ob, np.array([[[s + math.log(5)]]]))
    assert np.max(np.abs(m - (3 * oa + 5 * ob) / 8)) <= 1e-15
    assert abs(L[0, 0, 0] - (s + math.log(8))) <= 1e-15


def test_lse_identical_keys_closed_form():
    from oracle import block_attention
    rng = np.random.default_rng(43)
    q = _rand(rng, 1, 1, 3, 8)
    krow = _rand(rng, 1, 1, 1, 8)
    k = np.repeat(krow, 11, axis=2)
    v = _rand(rng, 1, 1, 11, 8)
    o, L = block_attention(q, k, v)
    s = (q[0, 0] @ krow[0, 0, 0]) / math.sqrt(8)
    assert np.max(np.abs(L[0, 0] - (s + math.log(11)))) <= 1e-13
    assert np.max(np.abs(o[0, 0] - v[0, 0].mean(axis=0))) <= 1e-13


# ---------------------------------------------------------------- MXFP4 (OCP MX) quantisation and linear

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # codes 0..7 from sign/exponent/mantissa by hand


def test_e2m1_and_e8m0_decode_tables():
    from oracle.mx import e2m1_decode, e8m0_decode
    got = e2m1_decode(np.arange(16))
    assert got[:8].tolist() == E2M1_TABLE
    assert (-got[8:]).tolist() == E2M1_TABLE and np.signbit(got[8])
    e = e8m0_decode(np.array([0, 1, 126, 127, 128, 254, 255]))
    assert e[:6].tolist() == [2.0 ** -127, 2.0 ** -126, 0.5, 1.0, 2.0, 2.0 ** 127] and np.isnan(e[6])


def test_mxfp4_quantize_closed_forms():
    from oracle.mx import mxfp4_quantize, mxfp4_dequantize
    blk = lambda vals: np.array(vals + [0.0] * (32 - len(vals)))
    # block max 6 * 2^k: scale 2^k, the max maps to code 7, exactly representable values survive
    x = blk([6.0 * 8, 0.5 * 8, -3.0 * 8, 1.5 * 8])
    c, s = mxfp4_quantize(x)
    assert s.tolist() == [127 + 3] and c[:4].tolist() == [7, 1, 8 + 5, 3]
    assert np.array_equal(mxfp4_dequantize(c, s), x)
    # max 7: floor(log2 7) - 2 = 0, 7 saturates to 6
    c, s = mxfp4_quantize(blk([7.0, 1.0]))
    assert s.tolist() == [127] and c[:2].tolist() == [7, 2]
    # ties go to the even code: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, -0.25->-0 (scale 2^0: max 4)
    c, s = mxfp4_quantize(blk([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 4.0, -0.25]))
    assert s.tolist() == [127] and c[:9].tolist() == [6, 0, 2, 2, 4, 4, 6, 6, 8]
    c, s = mxfp4_quantize(blk([6.0, 5.0]))                  # 5 is halfway between 4 and 6
    assert c[:2].tolist() == [7, 6]
    # zero block: smallest scale, zero codes; tiny block: scale clamped to 2^-127
    c, s = mxfp4_quantize(np.zeros(32))
    assert s.tolist() == [0] and not c.any()
    c, s = mxfp4_quantize(blk([2.0 ** -130]))
    assert s.tolist() == [0] and c[0] == 0


def test_mxfp4_quantize_picks_the_nearest_code_by_search():
    """Property pin: the scale obeys 2^X <= max|V| / 4 < 2^(X+1), and every code
    is the one of all 16 whose value times 2^X is nearest (ties: even code)."""
    from oracle.mx import mxfp4_quantize
    rng = np.random.default_rng(44)
    x = rng.standard_normal((6, 128)) * np.exp2(rng.integers(-8, 8, size=(6, 1)))
    c, s = mxfp4_quantize(x)
    table = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])
    for r in range(6):
        for b in range(4):
            blk = x[r, 32 * b:32 * b + 32]
            sc = 2.0 ** (int(s[r, b]) - 127)
            assert sc <= np.abs(blk).max() / 4 < 2 * sc
            for i, v in enumerate(blk):
                y = min(abs(v) / sc, 6.0) * (1 if v >= 0 else -1)
                d = np.abs(table - y)
                ok = np.flatnonzero(d == d.min())
                want = ok[0] if len(ok) == 1 or ok[0] % 2 == 0 else ok[1]
                if abs(table[want]) == 0.0:
                    want = 8 if v < 0 else 0
                assert c[r, 32 * b + i] == want, (r, b, i, v)


def test_mx_linear_exact_on_representable_values():
    """Codes and scales chosen so every product is a dyadic rational: the oracle
    must equal the exact sum computed with Python fractions."""
    from fractions import Fraction
    from oracle.mx import mx_linear
    rng = np.random.default_rng(45)
    M, N, K = 3, 4, 64
    ac, wc = rng.integers(0, 16, size=(M, K)), rng.integers(0, 16, size=(N, K))
    asc, wsc = rng.integers(120, 134, size=(M, K // 32)), rng.integers(120, 134, size=(N, K // 32))
    val = lambda code: (Fraction(E2M1_TABLE[code & 7]) * (-1 if code & 8 else 1))
    got = mx_linear(ac, asc, wc, wsc)
    for m in range(M):
        for n in range(N):
            exact = sum(val(int(ac[m, k])) * Fraction(2) ** (int(asc[m, k // 32]) - 127) *
                        val(int(wc[n, k])) * Fraction(2) ** (int(wsc[n, k // 32]) - 127) for k in range(K))
            assert got[m, n] == float(exact)


# ---------------------------------------------------------------- DBCache reuse decision

def test_residual_diff_closed_forms():
    from oracle.dbcache import can_reuse, residual_diff
    rng = np.random.default_rng(46)
    p = rng.standard_normal(1000)
    assert residual_diff(p, p) == 0.0
    assert abs(residual_diff(p, 1.25 * p) - 0.25) <= 1e-15          # cur = (1 + a) prev -> |a|
    assert abs(residual_diff(p, 0.9 * p) - 0.1) <= 1e-15
    assert residual_diff(p, np.zeros_like(p)) == 1.0                 # cur = 0 -> 1
    assert residual_diff(p, -p) == 2.0
    c = p + 0.05 * rng.standard_normal(1000)
    assert abs(residual_diff(3.0 * p, 3.0 * c) - residual_diff(p, c)) <= 1e-15   # scale invariance
    assert residual_diff(np.zeros(5), np.ones(5)) == math.inf and not can_reuse(np.zeros(5), np.zeros(5), 0.12)
    assert can_reuse(p, 1.1 * p, 0.12) and not can_reuse(p, 1.2 * p, 0.12)


def test_residual_diff_matches_brute_force():
    from oracle.dbcache import residual_diff
    rng = np.random.default_rng(47)
    p, c = rng.standard_normal(257), rng.standard_normal(257)
    assert abs(residual_diff(p, c) - brute.residual_diff(p.tolist(), c.tolist())) <= 1e-14


def test_residual_diff_nan_and_size_mismatch():
    from oracle.dbcache import can_reuse, residual_diff
    p = np.ones(64)
    c = np.ones(64)
    c[5] = np.nan
    assert math.isnan(residual_diff(p, c)) and not can_reuse(p, c, 1e300)
    with pytest.raises(ValueError):
        residual_diff(np.ones(3), np.ones(4))


# ---------------------------------------------------------------- pins of the remaining exported helpers

def test_oracle_lse_matches_brute_force_and_closed_form():
    """oracle.attention.lse (natural-log row log-sum-exp of the scaled scores)
    against the pure-Python math.fsum version, and the identical-keys closed
    form L = s + log n."""
    from oracle import lse
    rng = np.random.default_rng(48)
    q, k = _rand(rng, 2, 2, 5, 8), _rand(rng, 2, 2, 7, 8)
    got = lse(q, k, 0.45)
    want = np.array(brute.row_lse(q.tolist(), k.tolist(), scale=0.45))
    assert got.shape == (2, 2, 5)
    assert np.max(np.abs(got - want)) <= 1e-12
    got = lse(q, k)                                     # default scale 1/sqrt(D)
    want = np.array(brute.row_lse(q.tolist(), k.tolist()))
    assert np.max(np.abs(got - want)) <= 1e-12
    krow = _rand(rng, 1, 1, 1, 8)
    kk = np.repeat(krow, 9, axis=2)
    qq = _rand(rng, 1, 1, 3, 8)
    s = (qq[0, 0] @ krow[0, 0, 0]) / math.sqrt(8)
    assert np.max(np.abs(lse(qq, kk)[0, 0] - (s + math.log(9)))) <= 1e-13


def test_mx_linear_from_float_exact_on_representable_activations():
    """The dynamic-activation path on activations that MXFP4 represents
    exactly (every 32-block holds a +-6 * 2^X element, so the block scale is
    2^X, and the rest are E2M1 magnitudes times 2^X): quantising loses
    nothing, and the result must equal the exact dyadic sum of x times the
    dequantised weight, computed with Python fractions."""
    from fractions import Fraction
    from oracle.mx import mx_linear_from_float
    rng = np.random.default_rng(49)
    M, N, K = 3, 2, 64
    mags = np.array(E2M1_TABLE)
    x = np.empty((M, K))
    for m in range(M):
        for b in range(K // 32):
            ex = int(rng.integers(-6, 6))
            blk = mags[rng.integers(0, 8, size=32)] * rng.choice([-1.0, 1.0], size=32)
            blk[int(rng.integers(0, 32))] = 6.0 * (1 if rng.random() < 0.5 else -1)
            x[m, 32 * b:32 * b + 32] = blk * 2.0 ** ex
    wc = rng.integers(0, 16, size=(N, K))
    wsc = rng.integers(122, 132, size=(N, K // 32))
    val = lambda code: Fraction(E2M1_TABLE[code & 7]) * (-1 if code & 8 else 1)
    got = mx_linear_from_float(x, wc, wsc)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(x[m, kk])) * val(int(wc[n, kk])) * Fraction(2) ** (int(wsc[n, kk // 32]) - 127)
                        for kk in range(K))
            assert got[m, n] == float(exact)


def test_mx_linear_from_float_rounds_the_activations():
    """A hand-worked block: x = (7, 1.25, -0.75, 0, ...) has max 7, so
    X = floor(log2 7) - 2 = 0; 7 saturates to 6, 1.25 ties to the even code
    (1.0) and -0.75 ties to the even code (-1.0).  With a weight row of
    E2M1 1.0 (code 2) at scale 2^1 the product is 2 (6 + 1 - 1) = 12; a
    weight row of -0.5 (code 9) at scale 2^0 gives -0.5 (6 + 1 - 1) = -3."""
    from oracle.mx import mx_linear_from_float
    x = np.zeros((1, 32))
    x[0, :3] = [7.0, 1.25, -0.75]
    wc = np.zeros((2, 32), np.int64)
    wc[0, :3] = 2
    wc[1, :3] = 9
    wsc = np.array([[128], [127]])
    got = mx_linear_from_float(x, wc, wsc)
    assert got.tolist() == [[12.0, -3.0]]
