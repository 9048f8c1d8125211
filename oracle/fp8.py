"""OCP FP8 E4M3 decoding, float64.  Test infrastructure only.

The AMD RDNA 4 xDiT blog names an fp8 attention backend (and fp8 GEMMs and
communication) without fixing the format; the reading here is the OCP 8-bit
floating point E4M3 encoding: bit 7 sign, bits 6..3 exponent (bias 7), bits
2..0 mantissa; exponent 0 encodes subnormals m/8 * 2^-6; exponent 15 with
mantissa 7 is NaN; there are no infinities, so the largest finite value is
1.75 * 2^8 = 448.  Attention on fp8 inputs is attention on the dequantised
values code * scale (one scale per tensor), so the oracle decodes and then
calls ``oracle.attention.joint_attention`` unchanged.
"""
from __future__ import annotations

import numpy as np


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = sign * np.ldexp(1.0 + man / 8.0, exp - 7)
    subnormal = sign * np.ldexp(man / 8.0, -6)
    out = np.where(exp == 0, subnormal, normal)
    return np.where((exp == 15) & (man == 7), np.nan, out)


def dequantize(codes, scale: float) -> np.ndarray:
    """Real values of e4m3 codes with one per-tensor scale, float64."""
    return e4m3_decode(codes) * float(np.float32(scale))
