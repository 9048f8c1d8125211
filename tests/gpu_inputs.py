"""Device-side inputs for the GPU tests: seeded bf16 Q/K/V from dit_workloads
copied to the GPU, and the oracle's float64 view of the same values."""
from __future__ import annotations

import numpy as np

import dit_workloads as W


def to_device_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda")


def from_device_bf16(t) -> np.ndarray:
    """Device bf16 tensor -> float64 numpy (exact)."""
    import torch
    bits = t.detach().to("cpu").view(torch.int16).numpy().view(np.uint16)
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def sample_rows(S: int, S_txt: int, n_random: int, seed: int) -> np.ndarray:
    """Query rows for sampled checks: tile and segment boundaries plus random rows."""
    fixed = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 257, S_txt - 1, S_txt, S_txt + 1, S - 1, S - 2, S // 2}
    rng = np.random.default_rng(seed)
    rand = set(rng.integers(0, S, size=n_random).tolist())
    return np.array(sorted(r for r in fixed | rand if 0 <= r < S), dtype=np.int64)


def err_stats(got: np.ndarray, want: np.ndarray) -> dict:
    d = np.abs(got - want)
    return {"max_abs": float(d.max()), "mean_abs": float(d.mean()),
            "rel_mean": float(d.mean() / max(np.abs(want).mean(), 1e-300))}


def tile_rows(S: int, seed: int, per_tile_random: int = 2, tile: int = 256) -> np.ndarray:
    """First and last row of every `tile`-row query tile of a sequence, plus
    `per_tile_random` seeded random rows inside each tile (the ragged last tile
    included).  Every workgroup of the attention launch owns one such tile, so
    every workgroup's output is compared."""
    rng = np.random.default_rng(seed)
    rows = []
    for t0 in range(0, S, tile):
        t1 = min(S, t0 + tile)
        rows += [t0, t1 - 1] + rng.integers(t0, t1, size=per_tile_random).tolist()
    return np.unique(np.array(rows, dtype=np.int64))
