"""The LDS-NaN debug build (libditattn_ldsnan.so: every attention kernel fills
its LDS buffers with NaN bytes before its first tile copy) against the normal
build, on shapes that exercise ragged key and query tails, single-tile
sequences, the key-range pieces and the merge.  A read of LDS that no tile
copy wrote (a missing wait, a copy placed in the wrong buffer, a padding chunk
used as data) turns outputs into NaN; correct kernels give outputs identical
bit for bit to the normal build."""
import ctypes
import math

import numpy as np
import pytest

import dit_workloads as W
from tests.gpu_inputs import to_device_bf16

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _debug_lib():
    import os
    import dit_joint_self_amd as dj
    if not os.path.exists(dj.DEBUG_LDS_NAN_LIB_PATH):
        pytest.fail("libditattn_ldsnan.so is not built (build() builds it)")
    return dj.load_library(dj.DEBUG_LDS_NAN_LIB_PATH)


SHAPES = [  # (H, S_txt, grid)
    (1, 1, (0, 0)), (2, 0, (1, 31)), (2, 1, (4, 8)), (3, 1, (8, 8)), (2, 12, (12, 24)),
    (37, 0, (30, 60)),          # 296 items: whole-range workgroups + key-range pieces + merge
]


def _w(H, S_txt, grid, seed):
    return W.Workload("ldsnan", B=1, H=H, D=128, S_txt=S_txt, grid=grid, axes_dim=(64, 64), theta=10000.0, seed=seed)


@pytest.mark.parametrize("H,S_txt,grid", SHAPES)
def test_bf16_debug_build_matches(H, S_txt, grid):
    torch = _torch()
    import dit_joint_self_amd as dj
    L = _debug_lib()
    w = _w(H, S_txt, grid, seed=600 + H)
    qb, kb, vb = W.make_bf16_inputs(w)
    q, k, v = to_device_bf16(qb), to_device_bf16(kb), to_device_bf16(vb)
    cos, sin = dj.dit_rope_tables(torch.from_numpy(W.positions(w)).to("cuda"), w.axes_dim, w.theta)
    want = dj.dit_attn_forward(q, k, v, cos, sin, S_txt=w.S_txt)
    got = torch.empty_like(q)
    st = L.dit_attn_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), cos.data_ptr(), sin.data_ptr(), got.data_ptr(),
                            w.B, w.H, w.S_txt, w.S_img, w.D, 1.0 / math.sqrt(w.D), 0,
                            torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert not torch.isnan(got.float()).any().item(), f"S={w.S}: NaN from LDS no copy wrote"
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"S={w.S}"


@pytest.mark.parametrize("H,S_txt,grid", SHAPES)
def test_fp8_debug_build_matches(H, S_txt, grid):
    torch = _torch()
    import dit_joint_self_amd as dj
    L = _debug_lib()
    w = _w(H, S_txt, grid, seed=700 + H)
    (q8, sq), (k8, sk), (v8, sv) = [W.fp8_e4m3_quantize(x) for x in W.draw_qkv_f32(w)]
    dev = lambda c: torch.from_numpy(np.ascontiguousarray(c)).to("cuda")
    q, k, v = dev(q8), dev(k8), dev(v8)
    cos, sin = dj.dit_rope_tables(torch.from_numpy(W.positions(w)).to("cuda"), w.axes_dim, w.theta)
    want = dj.dit_attn_forward_fp8(q, k, v, sq, sk, sv, cos, sin, S_txt=w.S_txt)
    got = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    st = L.dit_attn_forward_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), sq, sk, sv, cos.data_ptr(), sin.data_ptr(),
                                got.data_ptr(), w.B, w.H, w.S_txt, w.S_img, w.D, 1.0 / math.sqrt(w.D),
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert not torch.isnan(got.float()).any().item(), f"S={w.S}: NaN from LDS no copy wrote"
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"S={w.S}"
