"""Thin Python binding of libditattn.so (MI355X / gfx950 joint self-attention).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Functions keep the C names (``dit_attn_forward``, ``dit_rope_tables``,
``dit_attn_workspace_bytes``, ``dit_attn_prepare_k``, ``dit_attn_core``,
``dit_attn_core_lse``, ``dit_attn_merge_lse``, the ``_fp8`` entries, the
MXFP4 linear-layer entries and the DBCache decision) and
take torch tensors, whose device pointers are passed after the checks the
C ABI cannot make (dtype, contiguity, shapes, one GPU).  A missing library
raises ``RuntimeError``: there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

__all__ = [
    "LIB_PATH", "DitAttnError", "lib", "lib_loaded", "dit_last_error", "dit_abi_version",
    "dit_rope_tables", "dit_attn_forward", "dit_attn_workspace_bytes", "dit_attn_prepare_k",
    "dit_attn_core", "dit_attn_workspace_bytes_fp8", "dit_attn_prepare_kv_fp8", "dit_attn_core_fp8",
    "dit_attn_forward_fp8", "dit_attn_core_lse", "dit_attn_merge_lse", "dit_mxfp4_scale_bytes",
    "dit_mxfp4_quantize", "dit_mxfp4_gemm", "dit_mxfp4_linear", "mxfp4_scale_shape", "mxfp4_scales_to_tiles",
    "mxfp4_scales_from_tiles", "dit_dbcache_workspace_bytes", "dit_dbcache_residual_diff",
    "dit_dbcache_residual_diff_noalloc", "dit_clock_probe",
    "dit_wall_clock_khz", "EXPORTED_SYMBOLS", "DIT_OK", "DIT_ERR_INVALID_ARG", "DIT_ERR_UNSUPPORTED",
    "DIT_ERR_NO_DEVICE", "DIT_ERR_OUT_OF_MEMORY", "DIT_ERR_LAUNCH", "DIT_DTYPE_BF16",
    "DIT_DTYPE_FP8_E4M3",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libditattn.so")
# Debug build whose attention kernels fill LDS with NaN before their first tile copy.
DEBUG_LDS_NAN_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libditattn_ldsnan.so")

DIT_DTYPE_BF16 = 0
DIT_DTYPE_FP8_E4M3 = 1

DIT_OK = 0
DIT_ERR_INVALID_ARG = 1
DIT_ERR_UNSUPPORTED = 2
DIT_ERR_NO_DEVICE = 3
DIT_ERR_OUT_OF_MEMORY = 4
DIT_ERR_LAUNCH = 5

_STATUS_NAMES = {0: "DIT_OK", 1: "DIT_ERR_INVALID_ARG", 2: "DIT_ERR_UNSUPPORTED", 3: "DIT_ERR_NO_DEVICE",
                 4: "DIT_ERR_OUT_OF_MEMORY", 5: "DIT_ERR_LAUNCH"}

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float

# name -> (restype, argtypes); the same set include/dit_attn.h declares.
_SIGNATURES = {
    "dit_last_error": (ctypes.c_char_p, []),
    "dit_abi_version": (_I, []),
    "dit_rope_tables": (_I, [_P, _I, _I, ctypes.POINTER(ctypes.c_int32), _F, _P, _P, _P]),
    "dit_attn_forward": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "dit_attn_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "dit_attn_prepare_k": (_I, [_P, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _I, _P]),
    "dit_attn_core": (_I, [_P, _P, _P, _P, _P, ctypes.c_size_t, _P, _I, _I, _I, _I, _F, _P]),
    "dit_attn_workspace_bytes_fp8": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "dit_attn_prepare_kv_fp8": (_I, [_P, _P, _F, _F, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _I, _P]),
    "dit_attn_core_fp8": (_I, [_P, _F, _P, _P, _P, ctypes.c_size_t, _P, _I, _I, _I, _I, _F, _P]),
    "dit_attn_forward_fp8": (_I, [_P, _P, _P, _F, _F, _F, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "dit_attn_core_lse": (_I, [_P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P, _I, _I, _I, _I, _F, _P]),
    "dit_attn_merge_lse": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "dit_mxfp4_scale_bytes": (ctypes.c_size_t, [_I, _I]),
    "dit_mxfp4_quantize": (_I, [_P, _P, _P, _I, _I, _P]),
    "dit_mxfp4_gemm": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P]),
    "dit_mxfp4_linear": (_I, [_P, _P, _P, _P, _I, _I, _I, _P]),
    "dit_dbcache_workspace_bytes": (ctypes.c_size_t, []),
    "dit_dbcache_residual_diff": (_I, [_P, _P, ctypes.c_int64, ctypes.c_double, _P, ctypes.c_size_t, _P, _P, _P]),
    "dit_dbcache_residual_diff_noalloc": (_I, [_P, _P, ctypes.c_int64, ctypes.c_double, _P, _P, _P]),
    "dit_clock_probe": (_I, [_P, ctypes.c_size_t, _I, _I, _P]),
    "dit_wall_clock_khz": (_I, [ctypes.POINTER(ctypes.c_int)]),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)


class DitAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use); raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python dit_joint_self_amd/build.py`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def lib_loaded() -> bool:
    return _lib is not None


def load_library(path: str) -> ctypes.CDLL:
    """A separate handle on another build of the library (for example the
    LDS-NaN debug build), with the same signatures; the wrappers above keep
    using the main library."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built")
    handle = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def _ptr(x) -> Optional[int]:
    """Device pointer of a validated tensor, or None."""
    if x is None:
        return None
    return x.data_ptr()


# ---------------------------------------------------------------- argument checks
#
# The C ABI sees pointers and sizes only.  Every wrapper below checks, before
# calling the library, what it cannot see: that each argument is a contiguous
# torch tensor of the right dtype and shape, that shapes agree across
# arguments, and that every tensor lives on one GPU.  Violations raise
# ValueError (TypeError for a non-tensor) and nothing is enqueued.

def _dt(name):
    import torch
    return getattr(torch, name)


def _tensor(t, name, dtypes, shape=None, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor (got {type(t).__name__})")
    allowed = tuple(_dt(d) for d in dtypes)
    if t.dtype not in allowed:
        raise ValueError(f"{name} must have dtype {' or '.join(dtypes)} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got shape {tuple(t.shape)})")
    if shape is not None and tuple(int(x) for x in t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _same_gpu(**named):
    """All given tensors (None skipped) on one GPU; returns that device."""
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU (got {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, other arguments on {dev}")
    return dev


def _tables(rope_cos, rope_sin, S, D):
    """Both None (no RoPE), or float32 [S, D/2] each."""
    if (rope_cos is None) != (rope_sin is None):
        raise ValueError("give both rope_cos and rope_sin, or neither")
    if rope_cos is not None:
        _tensor(rope_cos, "rope_cos", ["float32"], shape=(S, D // 2))
        _tensor(rope_sin, "rope_sin", ["float32"], shape=(S, D // 2))


def _workspace(ws, ws_bytes, name="workspace"):
    """A contiguous device buffer; returns the byte count passed to the library
    (at most the buffer's own size)."""
    import torch
    if not isinstance(ws, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor (got {type(ws).__name__})")
    if not ws.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = ws.numel() * ws.element_size()
    if ws_bytes is None:
        return have
    if int(ws_bytes) > have:
        raise ValueError(f"{name}_bytes = {int(ws_bytes)} exceeds the buffer's {have} bytes")
    return int(ws_bytes)


def _bhsd(t, name, dtypes):
    _tensor(t, name, dtypes, ndim=4)
    return tuple(int(x) for x in t.shape)


_F8 = ["uint8", "float8_e4m3fn"]


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int) -> None:
    if status != DIT_OK:
        raise DitAttnError(status, dit_last_error())


def dit_last_error() -> str:
    return lib().dit_last_error().decode()


def dit_abi_version() -> int:
    return lib().dit_abi_version()


def dit_rope_tables(pos, axes_dim: Sequence[int], theta: float, rope_cos=None, rope_sin=None, stream=None):
    """cos/sin tables [S, D/2] fp32 from int32 positions [S, n_axes] on the device.

    Allocates the outputs when not given; returns (rope_cos, rope_sin).
    """
    import torch
    _tensor(pos, "pos", ["int32"], ndim=2)
    S, n_axes = int(pos.shape[0]), int(pos.shape[1])
    if len(axes_dim) != n_axes:
        raise ValueError(f"axes_dim has {len(axes_dim)} entries, pos has {n_axes} axes")
    half = sum(int(a) for a in axes_dim) // 2
    if rope_cos is None:
        rope_cos = torch.empty((S, half), dtype=torch.float32, device=pos.device)
    if rope_sin is None:
        rope_sin = torch.empty((S, half), dtype=torch.float32, device=pos.device)
    _tensor(rope_cos, "rope_cos", ["float32"], shape=(S, half))
    _tensor(rope_sin, "rope_sin", ["float32"], shape=(S, half))
    _same_gpu(pos=pos, rope_cos=rope_cos, rope_sin=rope_sin)
    dims = (ctypes.c_int32 * len(axes_dim))(*[int(a) for a in axes_dim])
    _check(lib().dit_rope_tables(_ptr(pos), S, n_axes, dims, float(theta), _ptr(rope_cos), _ptr(rope_sin),
                                 _stream(stream)))
    return rope_cos, rope_sin


def dit_attn_forward(q, k, v, rope_cos=None, rope_sin=None, out=None, S_txt: int = 0, S_img: Optional[int] = None,
                     scale: Optional[float] = None, dtype: int = DIT_DTYPE_BF16, stream=None):
    """Joint self-attention with RoPE on Q/K: q, k, v bf16 [B, H, S, D] on the device.

    S_img defaults to S - S_txt; scale defaults to 1/sqrt(D).  Returns ``out``.
    """
    import torch
    B, H, S, D = shp = _bhsd(q, "q", ["bfloat16"])
    _tensor(k, "k", ["bfloat16"], shape=shp)
    _tensor(v, "v", ["bfloat16"], shape=shp)
    _tables(rope_cos, rope_sin, S, D)
    if S_img is None:
        S_img = S - S_txt
    if int(S_txt) < 0 or int(S_txt) + int(S_img) != S:
        raise ValueError(f"S_txt + S_img = {int(S_txt)} + {int(S_img)} does not match the sequence length {S}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _tensor(out, "out", ["bfloat16"], shape=shp)
    _same_gpu(q=q, k=k, v=v, rope_cos=rope_cos, rope_sin=rope_sin, out=out)
    _check(lib().dit_attn_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(rope_cos), _ptr(rope_sin), _ptr(out),
                                  B, H, S_txt, S_img, D, float(scale), int(dtype), _stream(stream)))
    return out


def dit_attn_workspace_bytes(B: int, H: int, S: int, D: int) -> int:
    return int(lib().dit_attn_workspace_bytes(B, H, S, D))


def dit_attn_prepare_k(k, rope_cos, rope_sin, workspace, workspace_bytes: Optional[int] = None, stream=None):
    """RoPE on K and its tile layout, into the caller's workspace (V is not prepared)."""
    B, H, S, D = _bhsd(k, "k", ["bfloat16"])
    _tables(rope_cos, rope_sin, S, D)
    workspace_bytes = _workspace(workspace, workspace_bytes)
    _same_gpu(k=k, rope_cos=rope_cos, rope_sin=rope_sin, workspace=workspace)
    _check(lib().dit_attn_prepare_k(_ptr(k), _ptr(rope_cos), _ptr(rope_sin), _ptr(workspace),
                                    int(workspace_bytes), B, H, S, D, _stream(stream)))


def dit_attn_core(q, v, rope_cos, rope_sin, workspace, out, scale: Optional[float] = None,
                  workspace_bytes: Optional[int] = None, stream=None):
    """Attention of q against the keys prepared in `workspace` and the values v."""
    B, H, S, D = shp = _bhsd(q, "q", ["bfloat16"])
    _tensor(v, "v", ["bfloat16"], shape=shp)
    _tables(rope_cos, rope_sin, S, D)
    _tensor(out, "out", ["bfloat16"], shape=shp)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    workspace_bytes = _workspace(workspace, workspace_bytes)
    _same_gpu(q=q, v=v, rope_cos=rope_cos, rope_sin=rope_sin, workspace=workspace, out=out)
    _check(lib().dit_attn_core(_ptr(q), _ptr(v), _ptr(rope_cos), _ptr(rope_sin), _ptr(workspace),
                               int(workspace_bytes), _ptr(out), B, H, S, D, float(scale), _stream(stream)))
    return out


def dit_attn_core_lse(q, v, rope_cos, rope_sin, workspace, out, lse=None, scale: Optional[float] = None,
                      workspace_bytes: Optional[int] = None, stream=None):
    """dit_attn_core plus the row log-sum-exp [B, H, S] fp32 (allocated when not given); returns (out, lse)."""
    import torch
    B, H, S, D = shp = _bhsd(q, "q", ["bfloat16"])
    _tensor(v, "v", ["bfloat16"], shape=shp)
    _tables(rope_cos, rope_sin, S, D)
    _tensor(out, "out", ["bfloat16"], shape=shp)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    workspace_bytes = _workspace(workspace, workspace_bytes)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    _tensor(lse, "lse", ["float32"], shape=(B, H, S))
    _same_gpu(q=q, v=v, rope_cos=rope_cos, rope_sin=rope_sin, workspace=workspace, out=out, lse=lse)
    _check(lib().dit_attn_core_lse(_ptr(q), _ptr(v), _ptr(rope_cos), _ptr(rope_sin), _ptr(workspace),
                                   int(workspace_bytes), _ptr(out), _ptr(lse), B, H, S, D, float(scale),
                                   _stream(stream)))
    return out, lse


def dit_attn_merge_lse(o_a, lse_a, o_b, lse_b, out=None, lse_out=None, stream=None):
    """Fold two partial results over disjoint key blocks; out / lse_out may be o_a / lse_a (in place)."""
    import torch
    B, H, S, D = shp = _bhsd(o_a, "o_a", ["bfloat16"])
    _tensor(o_b, "o_b", ["bfloat16"], shape=shp)
    _tensor(lse_a, "lse_a", ["float32"], shape=(B, H, S))
    _tensor(lse_b, "lse_b", ["float32"], shape=(B, H, S))
    if out is None:
        out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    _tensor(out, "out", ["bfloat16"], shape=shp)
    _tensor(lse_out, "lse_out", ["float32"], shape=(B, H, S))
    _same_gpu(o_a=o_a, lse_a=lse_a, o_b=o_b, lse_b=lse_b, out=out, lse_out=lse_out)
    _check(lib().dit_attn_merge_lse(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(out), _ptr(lse_out),
                                    B, H, S, D, _stream(stream)))
    return out, lse_out


# ---------------------------------------------------------------- MXFP4 linear layers

def mxfp4_scale_shape(rows: int, K: int):
    """Shape of the tiled E8M0 scale array the library uses for an MXFP4 [rows, K]
    operand: (ceil(rows / 32), ceil(K / 256), 256) bytes, tile (i, g) holding the
    scales of blocks 8g..8g+7 of rows 32i..32i+31, 8 bytes per row (see
    include/dit_attn.h)."""
    return (-(-rows // 32), -(-K // 256), 256)


def dit_mxfp4_scale_bytes(rows: int, K: int) -> int:
    return int(lib().dit_mxfp4_scale_bytes(int(rows), int(K)))


def mxfp4_scales_to_tiles(scales):
    """numpy uint8 [rows, K/32] (row-major scales) -> the tiled array of
    mxfp4_scale_shape (unused bytes zero).  A layout permutation only."""
    import numpy as np
    rows, nb = scales.shape
    nt, g, _ = mxfp4_scale_shape(rows, nb * 32)
    pad = np.zeros((nt * 32, g * 8), dtype=np.uint8)
    pad[:rows, :nb] = scales
    return np.ascontiguousarray(pad.reshape(nt, 32, g, 8).transpose(0, 2, 1, 3)).reshape(nt, g, 256)


def mxfp4_scales_from_tiles(tiles, rows: int, K: int):
    """The inverse of mxfp4_scales_to_tiles: tiled uint8 -> row-major [rows, K/32]."""
    import numpy as np
    nt, g, _ = mxfp4_scale_shape(rows, K)
    t = np.asarray(tiles).reshape(nt, g, 32, 8).transpose(0, 2, 1, 3).reshape(nt * 32, g * 8)
    return np.ascontiguousarray(t[:rows, :K // 32])


def dit_mxfp4_quantize(x, codes=None, scales=None, stream=None):
    """bf16 [rows, K] -> (codes uint8 [rows, K/2], scales uint8 in the tiled shape
    mxfp4_scale_shape(rows, K)) on the device."""
    import torch
    _tensor(x, "x", ["bfloat16"], ndim=2)
    rows, K = (int(s) for s in x.shape)
    if K % 32:
        raise ValueError(f"K = {K} must be a multiple of 32")
    if codes is None:
        codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(mxfp4_scale_shape(rows, K), dtype=torch.uint8, device=x.device)
    _tensor(codes, "codes", ["uint8"], shape=(rows, K // 2))
    _tensor(scales, "scales", ["uint8"], shape=mxfp4_scale_shape(rows, K))
    _same_gpu(x=x, codes=codes, scales=scales)
    _check(lib().dit_mxfp4_quantize(_ptr(x), _ptr(codes), _ptr(scales), rows, K, _stream(stream)))
    return codes, scales


def dit_mxfp4_gemm(a_codes, a_scales, w_codes, w_scales, out=None, stream=None):
    """out [M, N] bf16 = deq(A) deq(W)^T from MXFP4 codes [M, K/2], [N, K/2] and
    tiled scales (mxfp4_scale_shape(M, K), mxfp4_scale_shape(N, K))."""
    import torch
    _tensor(a_codes, "a_codes", ["uint8"], ndim=2)
    _tensor(w_codes, "w_codes", ["uint8"], ndim=2)
    M, N, K = int(a_codes.shape[0]), int(w_codes.shape[0]), 2 * int(a_codes.shape[1])
    if K % 32:
        raise ValueError(f"K = {K} must be a multiple of 32")
    _tensor(w_codes, "w_codes", ["uint8"], shape=(N, K // 2))
    _tensor(a_scales, "a_scales", ["uint8"], shape=mxfp4_scale_shape(M, K))
    _tensor(w_scales, "w_scales", ["uint8"], shape=mxfp4_scale_shape(N, K))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_codes.device)
    _tensor(out, "out", ["bfloat16"], shape=(M, N))
    _same_gpu(a_codes=a_codes, a_scales=a_scales, w_codes=w_codes, w_scales=w_scales, out=out)
    _check(lib().dit_mxfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales), _ptr(out), M, N, K,
                                _stream(stream)))
    return out


def dit_mxfp4_linear(x, w_codes, w_scales, out=None, stream=None):
    """x bf16 [M, K] times the MXFP4 weight [N, K]^T (codes [N, K/2], tiled scales
    mxfp4_scale_shape(N, K)): dynamic per-1x32 quantisation + A4W4 GEMM."""
    import torch
    _tensor(x, "x", ["bfloat16"], ndim=2)
    M, K = (int(s) for s in x.shape)
    if K % 32:
        raise ValueError(f"K = {K} must be a multiple of 32")
    _tensor(w_codes, "w_codes", ["uint8"], ndim=2)
    N = int(w_codes.shape[0])
    _tensor(w_codes, "w_codes", ["uint8"], shape=(N, K // 2))
    _tensor(w_scales, "w_scales", ["uint8"], shape=mxfp4_scale_shape(N, K))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _tensor(out, "out", ["bfloat16"], shape=(M, N))
    _same_gpu(x=x, w_codes=w_codes, w_scales=w_scales, out=out)
    _check(lib().dit_mxfp4_linear(_ptr(x), _ptr(w_codes), _ptr(w_scales), _ptr(out), M, N, K, _stream(stream)))
    return out


# ---------------------------------------------------------------- DBCache reuse decision

def dit_dbcache_workspace_bytes() -> int:
    return int(lib().dit_dbcache_workspace_bytes())


def dit_dbcache_residual_diff(prev, cur, threshold: float, ws=None, diff=None, reuse=None, stream=None):
    """Relative L1 difference of two bf16 residuals of the same size and the
    decision diff < threshold, both left on the device: (diff float64 [1],
    reuse int32 [1])."""
    import torch
    _tensor(prev, "prev", ["bfloat16"])
    _tensor(cur, "cur", ["bfloat16"])
    n = int(prev.numel())
    if int(cur.numel()) != n:
        raise ValueError("prev and cur must have the same number of elements")
    if ws is None:
        ws = torch.empty(dit_dbcache_workspace_bytes(), dtype=torch.uint8, device=prev.device)
    if diff is None:
        diff = torch.empty(1, dtype=torch.float64, device=prev.device)
    if reuse is None:
        reuse = torch.empty(1, dtype=torch.int32, device=prev.device)
    ws_bytes = _workspace(ws, None, "ws")
    _tensor(diff, "diff", ["float64"])
    _tensor(reuse, "reuse", ["int32"])
    if diff.numel() < 1 or reuse.numel() < 1:
        raise ValueError("diff and reuse must hold at least one element")
    _same_gpu(prev=prev, cur=cur, ws=ws, diff=diff, reuse=reuse)
    _check(lib().dit_dbcache_residual_diff(_ptr(prev), _ptr(cur), n, float(threshold), _ptr(ws), ws_bytes,
                                           _ptr(diff), _ptr(reuse), _stream(stream)))
    return diff, reuse


def dit_dbcache_residual_diff_noalloc(prev, cur, threshold: float, diff, reuse=None, stream=None):
    """dit_dbcache_residual_diff with the library's static scratch instead of a
    workspace: the library allocates nothing, so ``diff`` (float64, >= 1
    element) must be given, and ``reuse`` (int32) may be.  Calls that overlap on
    one GPU share the scratch and race."""
    _tensor(prev, "prev", ["bfloat16"])
    _tensor(cur, "cur", ["bfloat16"])
    n = int(prev.numel())
    if int(cur.numel()) != n:
        raise ValueError("prev and cur must have the same number of elements")
    _tensor(diff, "diff", ["float64"])
    if diff.numel() < 1:
        raise ValueError("diff must hold at least one element")
    if reuse is not None:
        _tensor(reuse, "reuse", ["int32"])
        if reuse.numel() < 1:
            raise ValueError("reuse must hold at least one element")
    _same_gpu(prev=prev, cur=cur, diff=diff, reuse=reuse)
    _check(lib().dit_dbcache_residual_diff_noalloc(_ptr(prev), _ptr(cur), n, float(threshold), _ptr(diff),
                                                   _ptr(reuse), _stream(stream)))
    return diff, reuse


# ---------------------------------------------------------------- clock probe

def dit_wall_clock_khz() -> int:
    khz = ctypes.c_int(0)
    _check(lib().dit_wall_clock_khz(ctypes.byref(khz)))
    return int(khz.value)


def dit_clock_probe(blocks: int = 512, iters: int = 20000, stream=None):
    """Shader clock under a bf16 MFMA load on every CU: (GHz, MFMA TFLOP/s of
    the probe).  The median over waves of shader cycles / constant-rate ticks,
    times the constant counter's rate."""
    import torch
    out = torch.zeros(blocks * 4 * 3, dtype=torch.int64, device="cuda")
    _check(lib().dit_clock_probe(_ptr(out), out.numel() * 8, blocks, iters, _stream(stream)))
    torch.cuda.synchronize()
    v = out.view(-1, 3).cpu().numpy().astype("float64")
    if (v[:, 2] != 0).any() or (v[:, 1] <= 0).any():
        raise RuntimeError("clock probe produced invalid counters")
    rate_hz = dit_wall_clock_khz() * 1e3
    ghz = float(sorted(v[:, 0] / v[:, 1])[len(v) // 2]) * rate_hz / 1e9
    seconds = float(v[:, 1].max()) / rate_hz
    tflops = blocks * 4 * iters * 4 * 2.0 * 32 * 32 * 16 / seconds / 1e12
    return ghz, tflops


# ---------------------------------------------------------------- fp8 (e4m3 codes + per-tensor scales)

def _shape8(t, name="q8"):
    """[B, H, S, D] of an e4m3 code tensor (uint8 or float8_e4m3fn)."""
    return _bhsd(t, name, _F8)


def dit_attn_workspace_bytes_fp8(B: int, H: int, S: int, D: int) -> int:
    return int(lib().dit_attn_workspace_bytes_fp8(B, H, S, D))


def dit_attn_prepare_kv_fp8(k8, v8, k_scale: float, v_scale: float, rope_cos, rope_sin, workspace,
                            workspace_bytes: Optional[int] = None, stream=None):
    B, H, S, D = shp = _shape8(k8, "k8")
    _tensor(v8, "v8", _F8, shape=shp)
    _tables(rope_cos, rope_sin, S, D)
    workspace_bytes = _workspace(workspace, workspace_bytes)
    _same_gpu(k8=k8, v8=v8, rope_cos=rope_cos, rope_sin=rope_sin, workspace=workspace)
    _check(lib().dit_attn_prepare_kv_fp8(_ptr(k8), _ptr(v8), float(k_scale), float(v_scale), _ptr(rope_cos),
                                         _ptr(rope_sin), _ptr(workspace), int(workspace_bytes), B, H, S, D,
                                         _stream(stream)))


def dit_attn_core_fp8(q8, q_scale: float, rope_cos, rope_sin, workspace, out, scale: Optional[float] = None,
                      workspace_bytes: Optional[int] = None, stream=None):
    B, H, S, D = shp = _shape8(q8)
    _tables(rope_cos, rope_sin, S, D)
    _tensor(out, "out", ["bfloat16"], shape=shp)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    workspace_bytes = _workspace(workspace, workspace_bytes)
    _same_gpu(q8=q8, rope_cos=rope_cos, rope_sin=rope_sin, workspace=workspace, out=out)
    _check(lib().dit_attn_core_fp8(_ptr(q8), float(q_scale), _ptr(rope_cos), _ptr(rope_sin), _ptr(workspace),
                                   int(workspace_bytes), _ptr(out), B, H, S, D, float(scale), _stream(stream)))
    return out


def dit_attn_forward_fp8(q8, k8, v8, q_scale: float, k_scale: float, v_scale: float, rope_cos=None, rope_sin=None,
                         out=None, S_txt: int = 0, S_img: Optional[int] = None, scale: Optional[float] = None,
                         stream=None):
    """Joint self-attention on e4m3 codes [B, H, S, D] with per-tensor scales; bf16 output."""
    import torch
    B, H, S, D = shp = _shape8(q8)
    _tensor(k8, "k8", _F8, shape=shp)
    _tensor(v8, "v8", _F8, shape=shp)
    _tables(rope_cos, rope_sin, S, D)
    if S_img is None:
        S_img = S - S_txt
    if int(S_txt) < 0 or int(S_txt) + int(S_img) != S:
        raise ValueError(f"S_txt + S_img = {int(S_txt)} + {int(S_img)} does not match the sequence length {S}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, S, D), dtype=torch.bfloat16, device=q8.device)
    _tensor(out, "out", ["bfloat16"], shape=shp)
    _same_gpu(q8=q8, k8=k8, v8=v8, rope_cos=rope_cos, rope_sin=rope_sin, out=out)
    _check(lib().dit_attn_forward_fp8(_ptr(q8), _ptr(k8), _ptr(v8), float(q_scale), float(k_scale), float(v_scale),
                                      _ptr(rope_cos), _ptr(rope_sin), _ptr(out), B, H, S_txt, S_img, D,
                                      float(scale), _stream(stream)))
    return out
