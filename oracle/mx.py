"""MXFP4 (OCP Microscaling) quantisation and the block-scaled linear layer,
float64. Test infrastructure only.

The MXFP4/Quark on MI350 blog (section "MXFP4 Quantization") quantises the
FLUX transformer's linear layers to MXFP4 as defined by the OCP Microscaling
(MX) specification: blocks of 32 FP4 elements share one E8M0 scale. Weights
are quantised once (static) and activations per call (dynamic), both in blocks
of 32 along the last axis (the reduction axis K of the linear layer), and the
product runs on the matrix cores (section "MXFP4 Kernel": an activation
quantisation kernel plus an A4W4 GEMM).

Formats, as the MX specification defines them:
* E2M1 element (4 bits): sign, 2 exponent bits (bias 1), 1 mantissa bit.
  Exponent 0 is subnormal (m / 2); the magnitudes are 0, 0.5, 1, 1.5, 2, 3,
  4, 6. No infinities or NaN.
* E8M0 scale (8 bits): 2^(x - 127); 0xFF is NaN.

Conversion of a block V of 32 values (the specification's rule):
    X = floor(log2(max |V_i|)) - emax_elem,  emax_elem = 2 for E2M1
    P_i = V_i / 2^X rounded to E2M1, round to nearest, ties to even, values
          beyond the largest magnitude (6) clamped to +-6.
A block of zeros takes the smallest scale 2^-127 and zero elements. X is
clamped to the E8M0 range [-127, 127].

The block-scaled linear layer is C = deq(A) deq(W)^T with deq(code, X) =
E2M1(code) * 2^X, computed here in float64 (the plain definition).
"""
from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0
EMAX_ELEM = 2
BLOCK = 32


def e2m1_decode(codes) -> np.ndarray:
    """4-bit codes (0..15, any integer dtype) -> float64 values."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return sign * mag


def e8m0_decode(x) -> np.ndarray:
    x = np.asarray(x).astype(np.int64)
    return np.where(x == 255, np.nan, np.exp2(x - 127.0))


_MAGS = e2m1_decode(np.arange(8))          # 0, .5, 1, 1.5, 2, 3, 4, 6 for codes 0..7


def _round_e2m1(y: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code of each float64 value, magnitudes above 6 clamped to
    6; a tie lies between two adjacent magnitudes, one with an even code and
    one with an odd code, and goes to the even one. The sign bit is kept
    (a negative value that rounds to zero gives -0, code 8). Codes 0..15."""
    a = np.minimum(np.abs(y), E2M1_MAX)
    d = np.abs(a[..., None] - _MAGS)
    near = d == d.min(axis=-1, keepdims=True)
    even = near & (np.arange(8) % 2 == 0)
    best = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(near, axis=-1))
    return best + 8 * np.signbit(y)


def mxfp4_quantize(x, block: int = BLOCK):
    """x [..., K] (K a multiple of 32) -> (codes uint8 [..., K] in 0..15,
    scales uint8 [..., K / 32] as E8M0 biased exponents)."""
    x = np.asarray(x, np.float64)
    K = x.shape[-1]
    if K % block:
        raise ValueError("K must be a multiple of the block size")
    xb = x.reshape(x.shape[:-1] + (K // block, block))
    amax = np.max(np.abs(xb), axis=-1)
    # floor(log2(amax)) exactly: amax = f * 2^p with f in [0.5, 1)
    _, p = np.frexp(amax)
    e = np.where(amax > 0, (p - 1).astype(np.float64) - EMAX_ELEM, -127.0)
    e = np.clip(e, -127, 127)
    y = xb / np.exp2(e)[..., None]
    codes = _round_e2m1(y).astype(np.uint8).reshape(x.shape)
    scales = (e + 127).astype(np.uint8)
    return codes, scales


def mxfp4_dequantize(codes, scales, block: int = BLOCK) -> np.ndarray:
    codes = np.asarray(codes)
    K = codes.shape[-1]
    v = e2m1_decode(codes).reshape(codes.shape[:-1] + (K // block, block))
    return (v * e8m0_decode(scales)[..., None]).reshape(codes.shape)


def mx_linear(a_codes, a_scales, w_codes, w_scales) -> np.ndarray:
    """C [M, N] = deq(A) [M, K] @ deq(W) [N, K]^T, float64."""
    a = mxfp4_dequantize(a_codes, a_scales)
    w = mxfp4_dequantize(w_codes, w_scales)
    return a @ w.T


def mx_linear_from_float(x, w_codes, w_scales) -> np.ndarray:
    """The dynamic-activation path: quantise x [M, K] per 1x32 block, then
    the block-scaled product with the already quantised weight."""
    a_codes, a_scales = mxfp4_quantize(x)
    return mx_linear(a_codes, a_scales, w_codes, w_scales)
