"""MXFP4 quantiser and A4W4 GEMM on the GPU (through the C ABI) against the
float64 oracle (oracle.mx).

* Quantisation: codes and scales bit-exact. Every decision of the MX rule is
  exact in fp32 for bf16 inputs (power-of-two scaling, comparisons with the
  rounding midpoints), so the GPU and the oracle must agree on every nibble.
* GEMM: the products of E2M1 values and E8M0 scales are exact in fp32; what
  remains is fp32 accumulation and the bf16 rounding of the output. Gate per
  element: |gpu - exact| <= 2^-8 |exact| + K 2^-24 S, with S = sum_k
  |a_k w_k| (the recursive-summation bound gamma_K for K terms).
"""
import numpy as np
import pytest

import dit_workloads as W
from oracle.mx import mx_linear, mxfp4_dequantize, mxfp4_quantize
from tests.gpu_inputs import bf16_f64, from_device_bf16

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _dj():
    import dit_joint_self_amd as dj
    return dj


def _dev_bf16(bits):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def _unpack(codes_bytes):
    """[rows, K/2] bytes -> [rows, K] nibbles (low nibble = even k)."""
    c = np.asarray(codes_bytes)
    return np.stack([c & 15, c >> 4], axis=-1).reshape(c.shape[0], -1)


def _pack(nibbles):
    n = np.asarray(nibbles, np.uint8).reshape(nibbles.shape[0], -1, 2)
    return (n[..., 0] | (n[..., 1] << 4)).astype(np.uint8)


def _gate(got, a_deq, w_deq, tag):
    exact = a_deq @ w_deq.T
    S = np.abs(a_deq) @ np.abs(w_deq).T
    K = a_deq.shape[1]
    bound = 2.0 ** -8 * np.abs(exact) + K * 2.0 ** -24 * S
    err = np.abs(got - exact)
    print(f"[mxfp4 parity] {tag}: max |diff| {err.max():.3g}, max |diff|/bound {(err / np.maximum(bound, 1e-300)).max():.3g}",
          flush=True)
    assert np.all(np.isfinite(got)), tag
    assert np.all(err <= bound), tag


def _quantize_edge_rows():
    """bf16 rows with blocks that exercise every branch of the rule: exact
    ties at the rounding midpoints, saturation, zeros, -0, tiny and huge
    blocks, subnormal bf16 values."""
    rows = []
    mids = [4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -5.0, -0.0, 0.0, 6.0, -6.0, 0.5]
    rows.append(np.array(mids * 2, np.float32))                           # X = 0: values land on midpoints
    rows.append(np.array([7.0, 6.5, -7.5, 1.0] + [0.1] * 28, np.float32))  # saturation above 6
    rows.append(np.zeros(32, np.float32))                                  # zero block
    rows.append(np.array([-0.0] * 32, np.float32))                         # all -0
    rows.append(np.array([2.0 ** -130] + [2.0 ** -133] * 31, np.float32))  # subnormal maxima: X clamps to -127
    rows.append(np.array(mids * 2, np.float32) * np.float32(2.0 ** -127))  # max 2^-125: X = -127 with every
    #                                                                        midpoint (bf16 subnormals, exact)
    rows.append(np.array([3.0e38, -1.0e38] + [1.0] * 30, np.float32))      # largest exponents
    rows.append(np.array([1.5 * 2.0 ** 20, 2.0 ** 18] + [2.0 ** 15] * 30, np.float32))
    x = np.concatenate(rows)
    x = np.tile(x, 2).reshape(2 * len(rows) * 32 // 64, 64)                 # rows of K = 64
    return W.bf16_round_bits(x)


@pytest.mark.parametrize("case", ["edges", "small_ragged", "flux1024x768_qkv"])
def test_quantize_bit_exact(case):
    torch = _torch()
    dj = _dj()
    if case == "edges":
        bits = _quantize_edge_rows()
    else:
        bits, _ = W.make_linear_inputs(W.LINEAR_WORKLOADS[case])
        bits = bits.copy()
        bits[0] = 0                                                        # one all-zero row
        bits[1, :32] = W.bf16_round_bits(np.full(32, 1e-39, np.float32))  # subnormal block
    x = _dev_bf16(bits)
    codes, scales = dj.dit_mxfp4_quantize(x)
    torch.cuda.synchronize()
    want_c, want_s = mxfp4_quantize(bf16_f64(bits))
    got_c = _unpack(codes.cpu().numpy())
    assert np.array_equal(dj.mxfp4_scales_from_tiles(scales.cpu().numpy(), *bits.shape), want_s), case
    bad = np.argwhere(got_c != want_c)
    assert len(bad) == 0, (case, bad[:5], got_c[tuple(bad[0])], want_c[tuple(bad[0])])


@pytest.mark.parametrize("M,N,K", [(128, 256, 128), (1, 4, 128), (200, 100, 384), (1000, 1028, 1024),
                                   (257, 260, 640), (2048, 9116, 384), (2304, 7424, 256)])
def test_gemm_random_codes(M, N, K):
    """Random codes (all 16 nibbles) and scales in 2^-7 .. 2^6: exact products.
    Up to 128 tiles run as 256 x 128 half tiles only (some wholly past N);
    2048 x 9116 has 288 tiles: 256 whole ones, then the last 32 as 64 half
    tiles (dispatched first), with a ragged last column tile and a half K
    step; 2304 x 7424 has 261 tiles: 256 whole ones and 5 tiles as 10 half
    tiles, a count that does not fill the XCDs evenly."""
    torch = _torch()
    dj = _dj()
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    ac, wc = rng.integers(0, 16, size=(M, K), dtype=np.uint8), rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    asc = rng.integers(120, 134, size=(M, K // 32), dtype=np.uint8)
    wsc = rng.integers(120, 134, size=(N, K // 32), dtype=np.uint8)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    tiles = lambda sc: dev(dj.mxfp4_scales_to_tiles(sc))   # the library's scale layout (a permutation)
    out = dj.dit_mxfp4_gemm(dev(_pack(ac)), tiles(asc), dev(_pack(wc)), tiles(wsc))
    torch.cuda.synchronize()
    got = from_device_bf16(out)
    _gate(got, mxfp4_dequantize(ac, asc), mxfp4_dequantize(wc, wsc), f"M={M} N={N} K={K}")
    assert np.array_equal(got, from_device_bf16(dj.dit_mxfp4_gemm(dev(_pack(ac)), tiles(asc), dev(_pack(wc)),
                                                                  tiles(wsc))))


@pytest.mark.parametrize("case", ["small_ragged", "flux1024x768_qkv"])
def test_linear_matches_oracle(case):
    """bf16 activations and weights: the weight quantised once, the activations
    inside dit_mxfp4_linear; against the oracle's quantise-then-multiply."""
    torch = _torch()
    dj = _dj()
    lw = W.LINEAR_WORKLOADS[case]
    xb, wb = W.make_linear_inputs(lw)
    wc, ws = dj.dit_mxfp4_quantize(_dev_bf16(wb))
    out = dj.dit_mxfp4_linear(_dev_bf16(xb), wc, ws)
    torch.cuda.synchronize()
    got = from_device_bf16(out)
    a_c, a_s = mxfp4_quantize(bf16_f64(xb))
    w_c, w_s = mxfp4_quantize(bf16_f64(wb))
    rows = np.arange(lw.M) if lw.M * lw.N <= 4e6 else np.unique(np.r_[0, 1, 127, 128, lw.M - 1,
                                                                        np.random.default_rng(1).integers(0, lw.M, 40)])
    _gate(got[rows], mxfp4_dequantize(a_c[rows], a_s[rows]), mxfp4_dequantize(w_c, w_s), case)
    # and the oracle's direct form agrees with the same reference
    ref = mx_linear(a_c[rows[:4]], a_s[rows[:4]], w_c, w_s)
    assert np.allclose(ref, mxfp4_dequantize(a_c[rows[:4]], a_s[rows[:4]]) @ mxfp4_dequantize(w_c, w_s).T)


def test_linear_full_size_sampled():
    """flux2048 fused QKV projection (M = 16896, N = 9216, K = 3072): the
    launch configuration the benchmark times, sampled rows."""
    torch = _torch()
    dj = _dj()
    lw = W.LINEAR_WORKLOADS["flux2048_qkv"]
    xb, wb = W.make_linear_inputs(lw)
    wc, ws = dj.dit_mxfp4_quantize(_dev_bf16(wb))
    out = dj.dit_mxfp4_linear(_dev_bf16(xb), wc, ws)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 127, 128, 16895, np.random.default_rng(2).integers(0, lw.M, 24)])
    got = from_device_bf16(out[torch.from_numpy(rows).to("cuda")])
    a_c, a_s = mxfp4_quantize(bf16_f64(xb[rows]))
    w_c, w_s = mxfp4_quantize(bf16_f64(wb))
    _gate(got, mxfp4_dequantize(a_c, a_s), mxfp4_dequantize(w_c, w_s), "flux2048_qkv")


def test_linear_full_size_bitwise_repeatable():
    """Two calls of the full-size QKV layer agree bit for bit (the GEMM issues
    its FP4 MFMAs back to back while the next fragments load)."""
    torch = _torch()
    dj = _dj()
    lw = W.LINEAR_WORKLOADS["flux2048_qkv"]
    xb, wb = W.make_linear_inputs(lw)
    x = _dev_bf16(xb)
    wc, ws = dj.dit_mxfp4_quantize(_dev_bf16(wb))
    a = dj.dit_mxfp4_linear(x, wc, ws)
    b = dj.dit_mxfp4_linear(x, wc, ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("M,N,K", [(300, 512, 256), (1, 8, 128)])
def test_gemm_out_only_8byte_aligned(M, N, K):
    """An output that starts 8 bytes past a 16-byte boundary (the interface
    asks for 8-byte alignment) takes the 8-byte store path; N % 8 == 0, so an
    aligned output of the same call takes the 16-byte one: both bit-identical
    and within the gate."""
    torch = _torch()
    dj = _dj()
    rng = np.random.default_rng(M + N + K)
    ac, wc = rng.integers(0, 16, size=(M, K), dtype=np.uint8), rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    asc = rng.integers(120, 134, size=(M, K // 32), dtype=np.uint8)
    wsc = rng.integers(120, 134, size=(N, K // 32), dtype=np.uint8)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    tiles = lambda sc: dev(dj.mxfp4_scales_to_tiles(sc))
    args = (dev(_pack(ac)), tiles(asc), dev(_pack(wc)), tiles(wsc))
    aligned = dj.dit_mxfp4_gemm(*args)
    buf = torch.full((M * N + 8,), float("nan"), dtype=torch.bfloat16, device="cuda")
    assert buf.data_ptr() % 16 == 0
    out8 = buf[4:4 + M * N].view(M, N)
    assert out8.data_ptr() % 16 == 8
    dj.dit_mxfp4_gemm(*args, out=out8)
    torch.cuda.synchronize()
    assert torch.equal(aligned.view(torch.int16), out8.view(torch.int16))
    assert torch.isnan(buf[:4]).all() and torch.isnan(buf[4 + M * N:]).all()   # nothing written outside
    _gate(from_device_bf16(aligned), mxfp4_dequantize(ac, asc), mxfp4_dequantize(wc, wsc), f"M={M} N={N} K={K}")
