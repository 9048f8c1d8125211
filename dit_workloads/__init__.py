"""Seeded synthetic inputs for DiT joint self-attention.

This module is the one piece shared by the CPU oracle, the tests and the
benchmark. It holds workload shapes and seeded random draws only: no RoPE,
no softmax, no attention arithmetic.

The joint sequence is the text tokens followed by the patchified latent
tokens (xDiT / FLUX pipeline pages: the DiT refines a latent of patches and
attends over prompt and image tokens together). Each image token carries its
integer grid coordinates, one per RoPE axis; text tokens carry 0 on every axis.
The grid is walked in raster order, with the last axis fastest.

Q, K and V are drawn as N(0, 1) float32 from ``numpy.random.default_rng(seed)``
in the order Q, K, V, each with shape [B, H, S, D], then rounded to bfloat16
with round-to-nearest-even. The fp8 workload quantises those same draws per
tensor to OCP E4M3 (one fp32 scale per tensor, amax / 448).

The linear-layer workloads (MXFP4 GEMMs on either side of attention) are the
FLUX.1-dev transformer's projections at a token count M: hidden size 3072
(24 heads x 128), MLP width 12288 (the MXFP4/Quark on MI350 blog quantises
these linear layers). The activation x [M, K] is drawn N(0, 1) and the weight
w [N, K] (one row per output feature) N(0, 1/K), float32 from
``default_rng(seed)`` in the order x, w, then rounded to bfloat16.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "positions", "draw_qkv_f32", "bf16_round_bits",
    "bf16_bits_to_f32", "make_bf16_inputs", "fp8_e4m3_quantize", "E4M3_MAX", "LinearWorkload",
    "LINEAR_WORKLOADS", "make_linear_inputs",
]

E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    S_txt: int
    grid: Tuple[int, ...]       # image token grid, slowest axis first
    axes_dim: Tuple[int, ...]   # RoPE dims per axis (sum = D); one axis per grid dim
    theta: float
    seed: int
    dtype: str = "bf16"         # "bf16" or "fp8_e4m3"
    note: str = field(default="", compare=False)

    @property
    def S_img(self) -> int:
        return int(np.prod(self.grid)) if self.grid else 0

    @property
    def S(self) -> int:
        return self.S_txt + self.S_img

    @property
    def flops(self) -> float:
        """QK^T plus PV multiply-adds counted as 2 flops each: 4 B H S^2 D."""
        return 4.0 * self.B * self.H * self.S * self.S * self.D

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny", B=1, H=2, D=128, S_txt=64, grid=(16, 16), axes_dim=(64, 64),
                 theta=10000.0, seed=1001,
                 note="2-D axial RoPE on a 16x16 patch grid, 320 tokens"),
        Workload("flux1024x768", B=1, H=24, D=128, S_txt=512, grid=(1, 48, 64),
                 axes_dim=(16, 56, 56), theta=10000.0, seed=1002,
                 note="1024x768 image: 48 rows x 64 columns of 2x2 latent patches, 3584 tokens"),
        Workload("flux2048", B=1, H=24, D=128, S_txt=512, grid=(1, 128, 128),
                 axes_dim=(16, 56, 56), theta=10000.0, seed=1003,
                 note="2048x2048 image: 128x128 patch grid, 16896 tokens (headline shape)"),
        Workload("video_ulysses4", B=1, H=10, D=128, S_txt=512, grid=(21, 45, 80),
                 axes_dim=(44, 42, 42), theta=10000.0, seed=1004,
                 note="video DiT, one GPU's 10-of-40 head share under 4-way Ulysses, 76112 tokens"),
        Workload("flux2048_fp8", B=1, H=24, D=128, S_txt=512, grid=(1, 128, 128),
                 axes_dim=(16, 56, 56), theta=10000.0, seed=1003, dtype="fp8_e4m3",
                 note="fp8 e4m3 per-tensor-scaled variant of flux2048, same draws"),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def positions(w: Workload) -> np.ndarray:
    """int32 [S, n_axes]: zeros for the S_txt text rows, then the image grid
    coordinates in raster order (last axis fastest)."""
    n_axes = len(w.axes_dim)
    if len(w.grid) != n_axes:
        raise ValueError("grid rank must equal the number of RoPE axes")
    pos = np.zeros((w.S, n_axes), dtype=np.int32)
    if w.S_img:
        coords = np.indices(w.grid, dtype=np.int32).reshape(n_axes, -1).T
        pos[w.S_txt:] = coords
    return pos


def draw_qkv_f32(w: Workload):
    """The raw N(0,1) float32 draws, in the order Q, K, V."""
    rng = np.random.default_rng(w.seed)
    shape = (w.B, w.H, w.S, w.D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    return q, k, v


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.
    Inputs here are finite, so no NaN handling.  Works in place on slices of
    a copy so full-size workloads round in a couple of seconds."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 22
    for i in range(0, flat.size, step):
        b = flat[i:i + step].view(np.uint32).copy()
        bias = b >> 16
        bias &= np.uint32(1)
        bias += np.uint32(0x7FFF)
        b += bias
        b >>= 16
        out[i:i + step] = b
    return out.reshape(x.shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_bf16_inputs(w: Workload):
    """Returns (q_bits, k_bits, v_bits) as uint16 bfloat16 patterns, [B,H,S,D]."""
    q, k, v = draw_qkv_f32(w)
    return bf16_round_bits(q), bf16_round_bits(k), bf16_round_bits(v)


def fp8_e4m3_quantize(x: np.ndarray):
    """Per-tensor OCP E4M3 quantisation of a float32 tensor.

    scale = amax(|x|) / 448 (float32); codes = round-to-nearest-even(x / scale)
    into E4M3 (saturating at +-448). Returns (uint8 codes, float32 scale).
    The encoding itself is torch's CPU float8_e4m3fn cast.
    """
    import torch
    amax = float(np.max(np.abs(x)))
    scale = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    y = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)) / torch.tensor(scale)
    y = torch.clamp(y, -E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


@dataclass(frozen=True)
class LinearWorkload:
    name: str
    M: int      # tokens (rows of x and of the output)
    N: int      # output features (rows of w)
    K: int      # input features (the reduction axis; MX blocks run along it)
    seed: int
    note: str = field(default="", compare=False)

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


LINEAR_WORKLOADS: Dict[str, LinearWorkload] = {
    w.name: w for w in [
        LinearWorkload("flux2048_qkv", M=16896, N=9216, K=3072, seed=2001,
                       note="fused Q, K, V projection of the 16896-token 2048x2048 sequence"),
        LinearWorkload("flux2048_out", M=16896, N=3072, K=3072, seed=2002,
                       note="attention output projection, 16896 tokens"),
        LinearWorkload("flux2048_mlp_up", M=16896, N=12288, K=3072, seed=2003,
                       note="MLP up projection, 16896 tokens"),
        LinearWorkload("flux2048_mlp_down", M=16896, N=3072, K=12288, seed=2004,
                       note="MLP down projection, 16896 tokens"),
        LinearWorkload("flux1024x768_qkv", M=3584, N=9216, K=3072, seed=2005,
                       note="fused Q, K, V projection of the 3584-token 1024x768 sequence"),
        LinearWorkload("small_ragged", M=200, N=100, K=384, seed=2006,
                       note="test shape: partial tiles in M and N, an odd number of K steps"),
    ]
}


def make_linear_inputs(w: LinearWorkload):
    """(x_bits [M, K], w_bits [N, K]) as bfloat16 bit patterns (uint16)."""
    rng = np.random.default_rng(w.seed)
    x = rng.standard_normal((w.M, w.K), dtype=np.float32)
    wt = rng.standard_normal((w.N, w.K), dtype=np.float32) * np.float32(1.0 / np.sqrt(w.K))
    return bf16_round_bits(x), bf16_round_bits(wt)


@dataclass(frozen=True)
class ResidualWorkload:
    """Residuals of the first Fn blocks of a DiT in two consecutive denoising
    steps, for the DBCache reuse decision: [tokens, hidden] bf16 each."""
    name: str
    tokens: int
    hidden: int
    rel_change: float   # scale of the step-to-step change relative to the residual
    seed: int
    note: str = field(default="", compare=False)

    @property
    def n(self) -> int:
        return self.tokens * self.hidden


RESIDUAL_WORKLOADS: Dict[str, ResidualWorkload] = {
    w.name: w for w in [
        ResidualWorkload("flux2048_residual", tokens=16896, hidden=3072, rel_change=0.1, seed=3001,
                         note="hidden state of the 16896-token 2048x2048 joint sequence (24 heads x 128)"),
        ResidualWorkload("flux1024x768_residual", tokens=3584, hidden=3072, rel_change=0.2, seed=3002,
                         note="hidden state of the 3584-token 1024x768 joint sequence"),
        ResidualWorkload("residual_ragged", tokens=333, hidden=1003, rel_change=0.05, seed=3003,
                         note="test shape: n = 333 x 1003, not a multiple of 8"),
    ]
}


def make_residual_inputs(w: ResidualWorkload):
    """(prev_bits, cur_bits), bfloat16 bit patterns [tokens, hidden].  The
    previous residual is Gaussian with a log-normal scale per hidden channel
    (a few channels carry most of the magnitude, as activation outliers do);
    the current one adds an independent Gaussian change of relative size
    rel_change per element, so the relative L1 difference is close to
    rel_change."""
    rng = np.random.default_rng(w.seed)
    ch = np.exp(rng.standard_normal(w.hidden, dtype=np.float32))
    prev = rng.standard_normal((w.tokens, w.hidden), dtype=np.float32)
    prev *= ch
    cur = rng.standard_normal((w.tokens, w.hidden), dtype=np.float32)
    cur *= np.float32(w.rel_change) * ch
    cur += prev
    return bf16_round_bits(prev), bf16_round_bits(cur)
