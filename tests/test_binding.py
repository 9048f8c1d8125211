"""The Python binding's own checks, on the CPU: every wrapper rejects what the
C ABI cannot see (dtype, contiguity, shape agreement, rope-table shape, the
device) with ValueError/TypeError before the library is called."""
import pytest
import torch

import dit_joint_self_amd as dj

BF = torch.bfloat16


def _qkv(S=8, H=2, D=128, dtype=BF):
    return [torch.zeros((1, H, S, D), dtype=dtype) for _ in range(3)]


def test_forward_rejects_wrong_dtype():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="dtype"):
        dj.dit_attn_forward(q.float(), k, v)
    with pytest.raises(ValueError, match="dtype"):
        dj.dit_attn_forward(q, k.half(), v)


def test_forward_rejects_non_contiguous_views():
    big = torch.zeros((1, 2, 16, 128), dtype=BF)
    view = big[:, :, ::2]                                 # strided rows (the qkv.chunk kind of view)
    assert view.shape == (1, 2, 8, 128) and not view.is_contiguous()
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="contiguous"):
        dj.dit_attn_forward(view, k, v)
    with pytest.raises(ValueError, match="contiguous"):
        dj.dit_attn_forward(q, view, v)


def test_forward_rejects_shape_disagreement():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="shape"):
        dj.dit_attn_forward(q, torch.zeros((1, 2, 9, 128), dtype=BF), v)
    with pytest.raises(ValueError, match="shape"):
        dj.dit_attn_forward(q, k, v, out=torch.zeros((1, 2, 8, 64), dtype=BF))
    with pytest.raises(ValueError, match="dimensions"):
        dj.dit_attn_forward(q[0], k, v)
    with pytest.raises(ValueError, match="S_txt"):
        dj.dit_attn_forward(q, k, v, S_txt=3, S_img=4)


def test_forward_rejects_bad_rope_tables():
    q, k, v = _qkv()
    good = torch.zeros((8, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="shape"):
        dj.dit_attn_forward(q, k, v, torch.zeros((7, 64)), good)   # tables built for fewer tokens
    with pytest.raises(ValueError, match="shape"):
        dj.dit_attn_forward(q, k, v, good, torch.zeros((8, 32)))   # axes not summing to 128
    with pytest.raises(ValueError, match="dtype"):
        dj.dit_attn_forward(q, k, v, good.double(), good.double())
    with pytest.raises(ValueError, match="both"):
        dj.dit_attn_forward(q, k, v, good, None)
    with pytest.raises(ValueError, match="contiguous"):
        dj.dit_attn_forward(q, k, v, torch.zeros((64, 8)).t(), good)


def test_forward_rejects_host_tensors():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="GPU"):
        dj.dit_attn_forward(q, k, v)


def test_split_entry_points_reject_bad_arguments():
    q, k, v = _qkv()
    ws = torch.zeros(dj.dit_attn_workspace_bytes(1, 2, 8, 128), dtype=torch.uint8)
    with pytest.raises(ValueError, match="shape"):
        dj.dit_attn_prepare_k(k, torch.zeros((7, 64)), torch.zeros((7, 64)), ws)
    with pytest.raises(ValueError, match="exceeds"):
        dj.dit_attn_prepare_k(k, None, None, ws, workspace_bytes=ws.numel() + 1)
    with pytest.raises(TypeError):
        dj.dit_attn_prepare_k(k, None, None, 0x1000)
    with pytest.raises(ValueError, match="shape"):
        dj.dit_attn_core(q, v, None, None, ws, torch.zeros((1, 2, 8, 64), dtype=BF))
    with pytest.raises(ValueError, match="shape"):
        dj.dit_attn_core(q, torch.zeros((1, 2, 16, 128), dtype=BF), None, None, ws, torch.empty_like(q))
    with pytest.raises(ValueError, match="shape"):
        dj.dit_attn_core_lse(q, v, None, None, ws, torch.empty_like(q), lse=torch.zeros((1, 2, 7)))
    with pytest.raises(ValueError, match="GPU"):
        dj.dit_attn_core(q, v, None, None, ws, torch.empty_like(q))


def test_merge_lse_rejects_bad_arguments():
    o, _, _ = _qkv()
    l = torch.zeros((1, 2, 8))
    with pytest.raises(ValueError, match="shape"):
        dj.dit_attn_merge_lse(o, l, o, torch.zeros((1, 2, 9)))
    with pytest.raises(ValueError, match="dtype"):
        dj.dit_attn_merge_lse(o, l.double(), o, l)


def test_fp8_entry_points_reject_bad_arguments():
    q8, k8, v8 = _qkv(dtype=torch.uint8)
    with pytest.raises(ValueError, match="dtype"):
        dj.dit_attn_forward_fp8(q8.to(BF), k8, v8, 1.0, 1.0, 1.0)
    with pytest.raises(ValueError, match="shape"):
        dj.dit_attn_forward_fp8(q8, k8[:, :1].contiguous(), v8, 1.0, 1.0, 1.0)
    with pytest.raises(ValueError, match="GPU"):
        dj.dit_attn_forward_fp8(q8, k8.view(torch.float8_e4m3fn), v8, 1.0, 1.0, 1.0)
    ws = torch.zeros(dj.dit_attn_workspace_bytes_fp8(1, 2, 8, 128), dtype=torch.uint8)
    with pytest.raises(ValueError, match="dtype"):
        dj.dit_attn_core_fp8(q8, 1.0, None, None, ws, torch.zeros((1, 2, 8, 128), dtype=torch.float32))


def test_mxfp4_and_dbcache_reject_bad_arguments():
    x = torch.zeros((4, 64), dtype=BF)
    with pytest.raises(ValueError, match="multiple of 32"):
        dj.dit_mxfp4_quantize(torch.zeros((4, 48), dtype=BF))
    with pytest.raises(ValueError, match="shape"):
        dj.dit_mxfp4_quantize(x, codes=torch.zeros((4, 31), dtype=torch.uint8))
    wc, wsc = torch.zeros((8, 32), dtype=torch.uint8), torch.zeros(dj.mxfp4_scale_shape(8, 64), dtype=torch.uint8)
    with pytest.raises(ValueError, match="shape"):
        dj.dit_mxfp4_linear(x, wc, torch.zeros((8, 3), dtype=torch.uint8))
    with pytest.raises(ValueError, match="shape"):   # row-major scales are not the library's layout
        dj.dit_mxfp4_linear(x, wc, torch.zeros((8, 2), dtype=torch.uint8))
    with pytest.raises(ValueError, match="dtype"):
        dj.dit_mxfp4_linear(x.float(), wc, wsc)
    with pytest.raises(ValueError, match="shape"):
        dj.dit_mxfp4_gemm(torch.zeros((4, 32), dtype=torch.uint8), torch.zeros((4, 1), dtype=torch.uint8), wc, wsc)
    with pytest.raises(ValueError, match="GPU"):
        dj.dit_mxfp4_linear(x, wc, wsc)
    p = torch.zeros(100, dtype=BF)
    with pytest.raises(ValueError, match="same number"):
        dj.dit_dbcache_residual_diff(p, torch.zeros(99, dtype=BF), 0.12)
    with pytest.raises(ValueError, match="dtype"):
        dj.dit_dbcache_residual_diff(p.float(), p.float(), 0.12)
    with pytest.raises(ValueError, match="dtype"):
        dj.dit_dbcache_residual_diff(p, p, 0.12, ws=torch.zeros(1 << 17, dtype=torch.uint8),
                                     diff=torch.zeros(1), reuse=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        dj.dit_dbcache_residual_diff(p, p, 0.12)


def test_rope_tables_reject_bad_arguments():
    pos = torch.zeros((8, 3), dtype=torch.int32)
    with pytest.raises(ValueError, match="dtype"):
        dj.dit_rope_tables(pos.long(), (16, 56, 56), 1e4)
    with pytest.raises(ValueError, match="axes"):
        dj.dit_rope_tables(pos, (64, 64), 1e4)
    with pytest.raises(ValueError, match="shape"):
        dj.dit_rope_tables(pos, (16, 56, 56), 1e4, rope_cos=torch.zeros((8, 32)))
    with pytest.raises(ValueError, match="GPU"):
        dj.dit_rope_tables(pos, (16, 56, 56), 1e4)


def test_mxfp4_scale_tiles_round_trip():
    """The tiled scale layout is a permutation: block b of row r sits at byte
    ((r // 32) * G + b // 8) * 256 + (r % 32) * 8 + b % 8, G = ceil(K / 256)."""
    import numpy as np
    rng = np.random.default_rng(5)
    for rows, K in [(1, 32), (33, 288), (64, 256), (70, 3072)]:
        s = rng.integers(0, 256, size=(rows, K // 32), dtype=np.uint8)
        t = dj.mxfp4_scales_to_tiles(s)
        assert t.shape == dj.mxfp4_scale_shape(rows, K)
        assert t.size == -(-rows // 32) * -(-K // 256) * 256
        flat, G = t.reshape(-1), -(-K // 256)
        for r, b in [(0, 0), (rows - 1, K // 32 - 1), (rows // 2, (K // 32) // 2)]:
            assert flat[((r // 32) * G + b // 8) * 256 + (r % 32) * 8 + b % 8] == s[r, b]
        assert np.array_equal(dj.mxfp4_scales_from_tiles(t, rows, K), s)
