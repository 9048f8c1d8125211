"""The C-ABI library without a GPU: it loads, exports what include/dit_attn.h
declares, and rejects bad arguments before touching HIP."""
import ctypes
import os
import re
import subprocess

import pytest

import dit_joint_self_amd as dj

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dj.LIB_PATH), reason="libditattn.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dit_[a-z0-9_]+)\s*\(", text)))


def _no_device():
    import torch
    return torch.cuda.device_count() == 0


def test_header_and_binding_agree():
    assert _declared_functions() == sorted(dj.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", dj.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (dit_[a-z0-9_]+)$", out, flags=re.M))
    for name in _declared_functions():
        assert name in exported, name
    lib = dj.lib()
    for name in dj.EXPORTED_SYMBOLS:
        assert getattr(lib, name) is not None
    assert dj.dit_abi_version() == 6


def _expected_workspace(B, H, S):
    """Tile stream (17 KiB of K' per 64-key tile per (batch, head), rounded up to 256 B)
    plus the key-range partials: items = B*H*ceil(S/256) query tiles; the r = items
    mod 256 items past the last full round of 256 CUs run split into the f key
    ranges (1 <= f <= min(8, ntiles)) that minimise ceil(r f / 256) * (1/f + 1/32)
    (rounds of pieces, each piece 1/f of an item plus a fixed 1/32), the smallest
    f on ties, when f >= 2; each range keeps 256 x 128 + 2 x 256 fp32 values; then
    256 bytes for the launch's piece counters."""
    from fractions import Fraction
    ntiles = -(-S // 64)
    tiles = (B * H * ntiles * 17408 + 255) // 256 * 256
    items = B * H * -(-S // 256)
    r = items % 256
    f = 1
    if r:
        cost = lambda g: -(-r * g // 256) * (Fraction(1, g) + Fraction(1, 32))
        f = min(range(1, min(8, ntiles) + 1), key=lambda g: (cost(g), g))
    part = r * f * (256 * 128 + 512) * 4 if (r and f >= 2) else 0
    return tiles + part + 256


def test_workspace_bytes():
    assert dj.dit_attn_workspace_bytes(1, 24, 16896, 128) == 24 * 264 * 17408 + 48 * 5 * 33280 * 4 + 256
    assert dj.dit_attn_workspace_bytes(1, 1, 1, 128) == 17408 + 256
    # The video share: 2980 items leave 164 after 11 rounds, split over 3 key ranges.
    assert dj.dit_attn_workspace_bytes(1, 10, 76112, 128) == 10 * 1190 * 17408 + 164 * 3 * 33280 * 4 + 256
    for B, H, S in [(1, 24, 16896), (2, 3, 65), (1, 1, 1), (1, 24, 3584), (1, 10, 76112), (1, 2, 320), (3, 7, 999),
                    (1, 1, 130000), (4, 13, 4000), (1, 200, 256)]:
        assert dj.dit_attn_workspace_bytes(B, H, S, 128) == _expected_workspace(B, H, S), (B, H, S)
    assert dj.dit_attn_workspace_bytes(1, 1, 0, 128) == 0
    assert dj.dit_attn_workspace_bytes(1, 1, 64, 64) == 0
    assert dj.dit_attn_workspace_bytes(1, 1, 2**21, 128) > 0
    assert dj.dit_attn_workspace_bytes(1, 1, 2**21 + 1, 128) == 0
    assert dj.dit_attn_workspace_bytes_fp8(1, 1, 2**21 + 1, 128) == 0


FAKE = 0x100000  # 16-byte aligned, never dereferenced: validation fails first


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, cos=None, sin=None, out=FAKE * 4, B=1, H=2, S_txt=3, S_img=5,
             D=128, scale=0.1, dtype=0, stream=None)
    a.update(kw)
    return dj.lib().dit_attn_forward(a["q"], a["k"], a["v"], a["cos"], a["sin"], a["out"], a["B"], a["H"],
                                     a["S_txt"], a["S_img"], a["D"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), dj.DIT_ERR_INVALID_ARG),
    (dict(out=None), dj.DIT_ERR_INVALID_ARG),
    (dict(cos=FAKE * 5), dj.DIT_ERR_INVALID_ARG),             # exactly one table
    (dict(sin=FAKE * 5), dj.DIT_ERR_INVALID_ARG),
    (dict(cos=FAKE * 5 + 4, sin=FAKE * 6), dj.DIT_ERR_INVALID_ARG),  # misaligned table
    (dict(B=0), dj.DIT_ERR_INVALID_ARG),
    (dict(H=-1), dj.DIT_ERR_INVALID_ARG),
    (dict(S_txt=-1), dj.DIT_ERR_INVALID_ARG),
    (dict(S_txt=0, S_img=0), dj.DIT_ERR_INVALID_ARG),
    (dict(S_txt=2**31 - 1, S_img=1), dj.DIT_ERR_INVALID_ARG),  # S overflows int
    (dict(D=64), dj.DIT_ERR_UNSUPPORTED),
    (dict(S_txt=2**21, S_img=1), dj.DIT_ERR_UNSUPPORTED),      # longer than the longest supported sequence
    (dict(D=0), dj.DIT_ERR_INVALID_ARG),
    (dict(dtype=1), dj.DIT_ERR_UNSUPPORTED),
    (dict(dtype=7), dj.DIT_ERR_INVALID_ARG),
    (dict(scale=float("nan")), dj.DIT_ERR_INVALID_ARG),
    (dict(scale=float("inf")), dj.DIT_ERR_INVALID_ARG),
    (dict(q=FAKE + 2), dj.DIT_ERR_INVALID_ARG),               # misaligned
    (dict(out=FAKE), dj.DIT_ERR_INVALID_ARG),                 # out aliases q
    (dict(out=FAKE * 2 + 256), dj.DIT_ERR_INVALID_ARG),       # out overlaps k
    (dict(B=70000, H=1), dj.DIT_ERR_INVALID_ARG),             # too many (b, h) for one launch
    (dict(B=1, H=60000, S_txt=2**20, S_img=0), dj.DIT_ERR_INVALID_ARG),
])
def test_forward_rejects_bad_arguments(kw, status):
    assert _fwd(**kw) == status
    assert dj.dit_last_error() != ""


def test_split_entry_points_reject_bad_arguments():
    L = dj.lib()
    need = dj.dit_attn_workspace_bytes(1, 2, 8, 128)
    ws = 0x10000000
    V = FAKE * 7
    assert L.dit_attn_prepare_k(FAKE, None, None, ws, need - 1, 1, 2, 8, 128, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_prepare_k(FAKE, None, None, ws + 16, need, 1, 2, 8, 128, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_prepare_k(FAKE, None, None, FAKE, need, 1, 2, 8, 128, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_prepare_k(None, None, None, ws, need, 1, 2, 8, 128, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_prepare_k(FAKE, None, None, ws, need, 1, 2, 8, 96, None) == dj.DIT_ERR_UNSUPPORTED
    assert L.dit_attn_core(FAKE, V, None, None, ws, need, ws, 1, 2, 8, 128, 0.1, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_core(FAKE, V, FAKE * 2, None, ws, need, FAKE * 3, 1, 2, 8, 128, 0.1, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_core(FAKE, V, None, None, ws, need, FAKE * 3, 1, 2, 8, 128, float("nan"), None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_core(FAKE, V, None, None, ws, need - 1, FAKE * 3, 1, 2, 8, 128, 0.1, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_core(FAKE, None, None, None, ws, need, FAKE * 3, 1, 2, 8, 128, 0.1, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_core(FAKE, V + 8, None, None, ws, need, FAKE * 3, 1, 2, 8, 128, 0.1, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_core(FAKE, FAKE * 3 + 64, None, None, ws, need, FAKE * 3, 1, 2, 8, 128, 0.1, None) == dj.DIT_ERR_INVALID_ARG
    # core writes key-range partials into its workspace: q, v and the tables must lie outside it
    assert L.dit_attn_core(ws + 256, V, None, None, ws, need, FAKE * 3, 1, 2, 8, 128, 0.1, None) == dj.DIT_ERR_INVALID_ARG
    assert "overlaps the workspace" in dj.dit_last_error()
    assert L.dit_attn_core(FAKE, ws + 256, None, None, ws, need, FAKE * 3, 1, 2, 8, 128, 0.1, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_core(FAKE, V, ws + 512, FAKE * 5, ws, need, FAKE * 3, 1, 2, 8, 128, 0.1, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_core(FAKE, V, FAKE * 5, FAKE * 3 + 64, ws, need, FAKE * 3, 1, 2, 8, 128, 0.1, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_prepare_k(FAKE, ws + 512, FAKE * 5, ws, need, 1, 2, 8, 128, None) == dj.DIT_ERR_INVALID_ARG
    assert _fwd(cos=FAKE * 4 + 256, sin=FAKE * 6) == dj.DIT_ERR_INVALID_ARG      # a table inside out
    if _no_device():                                                             # tables apart: valid
        assert L.dit_attn_core(FAKE, V, FAKE * 5, FAKE * 6, ws, need, FAKE * 3, 1, 2, 8, 128, 0.1, None) == dj.DIT_ERR_NO_DEVICE
        assert L.dit_attn_prepare_k(FAKE, FAKE * 5, FAKE * 6, ws, need, 1, 2, 8, 128, None) == dj.DIT_ERR_NO_DEVICE


def test_rope_tables_reject_bad_arguments():
    L = dj.lib()
    dims = lambda *d: (ctypes.c_int32 * len(d))(*d)
    assert L.dit_rope_tables(None, 4, 2, dims(64, 64), 1e4, FAKE, FAKE * 2, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_rope_tables(FAKE, 0, 2, dims(64, 64), 1e4, FAKE, FAKE * 2, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_rope_tables(FAKE, 4, 0, dims(64, 64), 1e4, FAKE, FAKE * 2, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_rope_tables(FAKE, 4, 5, dims(2, 2, 2, 2, 2), 1e4, FAKE, FAKE * 2, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_rope_tables(FAKE, 4, 2, dims(63, 65), 1e4, FAKE, FAKE * 2, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_rope_tables(FAKE, 4, 2, dims(64, 64), 0.0, FAKE, FAKE * 2, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_rope_tables(FAKE, 4, 2, dims(64, 64), 1e4, FAKE + 4, FAKE * 2, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_rope_tables(FAKE, 4, 2, dims(64, 64), 1e4, FAKE, FAKE + 64, None) == dj.DIT_ERR_INVALID_ARG


@pytest.mark.skipif(not _no_device(), reason="a GPU is visible")
def test_valid_call_without_device_reports_no_device():
    assert _fwd() == dj.DIT_ERR_NO_DEVICE
    assert "device" in dj.dit_last_error()
    dims = (ctypes.c_int32 * 2)(64, 64)
    assert dj.lib().dit_rope_tables(FAKE, 4, 2, dims, 1e4, FAKE, FAKE * 2, None) == dj.DIT_ERR_NO_DEVICE


def test_binding_raises_on_error_status():
    with pytest.raises(dj.DitAttnError) as ei:
        dj._check(dj.DIT_ERR_UNSUPPORTED)
    assert "DIT_ERR_UNSUPPORTED" in str(ei.value)


def test_fp8_entry_points_reject_bad_arguments():
    L = dj.lib()
    # fp8 workspace: 256-byte header + 19 KiB tiles, the same split partials as bf16, the pool counters.
    # header, one 64-key tile, the launch's pool counters
    assert dj.dit_attn_workspace_bytes_fp8(1, 1, 1, 128) == 256 + 19456 + 256
    assert dj.dit_attn_workspace_bytes_fp8(1, 1, 64, 64) == 0
    F = L.dit_attn_forward_fp8
    ok = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, sq=0.1, sk=0.1, sv=0.1, out=FAKE * 4)
    def call(**kw):
        a = dict(ok); a.update(kw)
        return F(a["q"], a["k"], a["v"], a["sq"], a["sk"], a["sv"], None, None, a["out"], 1, 2, 3, 5, 128, 0.1, None)
    assert call(q=None) == dj.DIT_ERR_INVALID_ARG
    assert call(sq=0.0) == dj.DIT_ERR_INVALID_ARG
    assert call(sk=float("nan")) == dj.DIT_ERR_INVALID_ARG
    assert call(sv=-1.0) == dj.DIT_ERR_INVALID_ARG
    assert call(q=FAKE + 8) == dj.DIT_ERR_INVALID_ARG
    assert call(out=FAKE * 3) == dj.DIT_ERR_INVALID_ARG
    need = dj.dit_attn_workspace_bytes_fp8(1, 2, 8, 128)
    ws = 0x10000000
    assert L.dit_attn_prepare_kv_fp8(FAKE, FAKE * 2, 0.1, 0.1, None, None, ws, need - 1, 1, 2, 8, 128, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_prepare_kv_fp8(FAKE, FAKE * 2, 0.0, 0.1, None, None, ws, need, 1, 2, 8, 128, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_core_fp8(FAKE, 0.1, None, None, ws, need, FAKE * 3, 1, 2, 8, 96, 0.1, None) == dj.DIT_ERR_UNSUPPORTED
    assert L.dit_attn_core_fp8(FAKE, float("inf"), None, None, ws, need, FAKE * 3, 1, 2, 8, 128, 0.1, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_attn_core_fp8(ws + 1024, 0.1, None, None, ws, need, FAKE * 3, 1, 2, 8, 128, 0.1, None) == dj.DIT_ERR_INVALID_ARG
    if _no_device():                                  # a negative softmax scale is valid (either sign)
        assert L.dit_attn_core_fp8(FAKE, 0.1, None, None, ws, need, FAKE * 3, 1, 2, 8, 128, -0.1, None) == dj.DIT_ERR_NO_DEVICE
        assert F(FAKE, FAKE * 2, FAKE * 3, 0.1, 0.1, 0.1, None, None, FAKE * 4, 1, 2, 3, 5, 128, -0.1, None) == dj.DIT_ERR_NO_DEVICE
    if _no_device():
        assert call() == dj.DIT_ERR_NO_DEVICE


def test_lse_entry_points_reject_bad_arguments():
    L = dj.lib()
    need = dj.dit_attn_workspace_bytes(1, 2, 8, 128)
    ws = 0x10000000
    lse = 0x20000000
    core = lambda **kw: L.dit_attn_core_lse(kw.get("q", FAKE), FAKE * 7, None, None, ws, need, kw.get("out", FAKE * 3),
                                            kw.get("lse", lse), 1, 2, 8, 128, 0.1, None)
    assert core(lse=None) == dj.DIT_ERR_INVALID_ARG
    assert core(lse=lse + 2) == dj.DIT_ERR_INVALID_ARG                 # misaligned
    assert core(lse=FAKE * 3 + 64) == dj.DIT_ERR_INVALID_ARG           # inside out
    assert core(lse=ws + 128) == dj.DIT_ERR_INVALID_ARG                # inside the workspace
    assert core(q=None) == dj.DIT_ERR_INVALID_ARG
    tb, lb = 2 * 8 * 128 * 2, 2 * 8 * 4
    oa, ob, o = 0x30000000, 0x40000000, 0x50000000
    la, lb_, lo = 0x60000000, 0x70000000, 0x80000000
    merge = lambda **kw: L.dit_attn_merge_lse(kw.get("oa", oa), kw.get("la", la), kw.get("ob", ob), kw.get("lb", lb_),
                                              kw.get("o", o), kw.get("lo", lo), 1, 2, 8, kw.get("D", 128), None)
    assert merge(oa=None) == dj.DIT_ERR_INVALID_ARG
    assert merge(lo=None) == dj.DIT_ERR_INVALID_ARG
    assert merge(D=64) == dj.DIT_ERR_UNSUPPORTED
    assert merge(o=oa + 16) == dj.DIT_ERR_INVALID_ARG                  # partial overlap with o_a
    assert merge(lo=la + 4) == dj.DIT_ERR_INVALID_ARG                  # partial overlap with lse_a
    assert merge(o=la) == dj.DIT_ERR_INVALID_ARG                       # out over an lse input
    assert merge(lo=ob + 64) == dj.DIT_ERR_INVALID_ARG                 # lse_out inside o_b
    assert merge(o=oa + 8) == dj.DIT_ERR_INVALID_ARG                   # misaligned
    assert merge(la=la + 1) == dj.DIT_ERR_INVALID_ARG
    if _no_device():                                                   # exact in-place folding is valid
        assert merge(o=oa, lo=la) == dj.DIT_ERR_NO_DEVICE
        assert merge(o=ob, lo=lb_) == dj.DIT_ERR_NO_DEVICE
        assert core() == dj.DIT_ERR_NO_DEVICE


def test_mxfp4_entry_points_reject_bad_arguments():
    L = dj.lib()
    x, c, s, o = 0x30000000, 0x40000000, 0x50000000, 0x60000000
    # tiled scales: ceil(rows / 32) x ceil(K / 256) tiles of 256 bytes
    assert L.dit_mxfp4_scale_bytes(16896, 3072) == 528 * 12 * 256
    assert L.dit_mxfp4_scale_bytes(33, 288) == 2 * 2 * 256
    assert L.dit_mxfp4_scale_bytes(1, 32) == 256
    assert L.dit_mxfp4_scale_bytes(0, 64) == 0 and L.dit_mxfp4_scale_bytes(4, 48) == 0
    q = L.dit_mxfp4_quantize
    assert q(None, c, s, 4, 64, None) == dj.DIT_ERR_INVALID_ARG
    assert q(x, c, s, 0, 64, None) == dj.DIT_ERR_INVALID_ARG
    assert q(x, c, s, 4, 48, None) == dj.DIT_ERR_INVALID_ARG              # K not a multiple of 32
    assert q(x + 8, c, s, 4, 64, None) == dj.DIT_ERR_INVALID_ARG          # x misaligned
    assert q(x, x + 64, s, 4, 64, None) == dj.DIT_ERR_INVALID_ARG         # codes inside x
    assert q(x, c, c + 8, 4, 64, None) == dj.DIT_ERR_INVALID_ARG          # scales inside codes
    assert q(x, c, s, 2 ** 20, 2 ** 12, None) == dj.DIT_ERR_UNSUPPORTED   # rows * K / 2 >= 2^31
    g = lambda **kw: L.dit_mxfp4_gemm(kw.get("ac", c), kw.get("as_", s), kw.get("wc", c + 2 ** 24),
                                      kw.get("ws", s + 2 ** 24), kw.get("o", o), kw.get("M", 8),
                                      kw.get("N", 16), kw.get("K", 256), None)
    assert g(ac=None) == dj.DIT_ERR_INVALID_ARG
    assert g(K=192) == dj.DIT_ERR_INVALID_ARG                             # K not a multiple of 128
    assert g(N=18) == dj.DIT_ERR_INVALID_ARG                              # N not a multiple of 4
    assert g(ac=c + 8) == dj.DIT_ERR_INVALID_ARG                          # codes misaligned
    assert g(ws=s + 2 ** 24 + 2) == dj.DIT_ERR_INVALID_ARG                # scales misaligned
    assert g(o=o + 4) == dj.DIT_ERR_INVALID_ARG                           # out misaligned
    assert g(o=c) == dj.DIT_ERR_INVALID_ARG                               # out over the A codes
    assert g(M=2 ** 20, K=2 ** 12) == dj.DIT_ERR_UNSUPPORTED
    lin = L.dit_mxfp4_linear
    assert lin(None, c, s, o, 8, 16, 256, None) == dj.DIT_ERR_INVALID_ARG
    assert lin(x, c, s, x, 8, 16, 256, None) == dj.DIT_ERR_INVALID_ARG    # out over x
    assert lin(x, c, s, o, 8, 16, 100, None) == dj.DIT_ERR_INVALID_ARG
    if _no_device():
        assert q(x, c, s, 4, 64, None) == dj.DIT_ERR_NO_DEVICE
        assert g() == dj.DIT_ERR_NO_DEVICE
        assert lin(x, c, s, o, 8, 16, 256, None) == dj.DIT_ERR_NO_DEVICE


def test_dbcache_entry_point_rejects_bad_arguments():
    L = dj.lib()
    need = L.dit_dbcache_workspace_bytes()
    assert need == 8192 * 16
    p, c, w, d, r = 0x30000000, 0x40000000, 0x50000000, 0x60000000, 0x60000040
    f = lambda **kw: L.dit_dbcache_residual_diff(kw.get("p", p), kw.get("c", c), kw.get("n", 1000), 0.12,
                                                 kw.get("w", w), kw.get("wb", need), kw.get("d", d),
                                                 kw.get("r", r), None)
    assert f(p=None) == dj.DIT_ERR_INVALID_ARG
    assert f(c=None) == dj.DIT_ERR_INVALID_ARG
    assert f(w=None) == dj.DIT_ERR_INVALID_ARG
    assert f(d=None) == dj.DIT_ERR_INVALID_ARG
    assert f(n=-1) == dj.DIT_ERR_INVALID_ARG
    assert f(n=2 ** 40 + 1) == dj.DIT_ERR_UNSUPPORTED
    assert f(wb=need - 16) == dj.DIT_ERR_INVALID_ARG                      # workspace too small
    assert f(c=c + 2) == dj.DIT_ERR_INVALID_ARG                           # misaligned input
    assert f(d=d + 4) == dj.DIT_ERR_INVALID_ARG                           # misaligned diff
    assert f(w=p + 1024) == dj.DIT_ERR_INVALID_ARG                        # workspace inside prev
    assert f(d=c + 16) == dj.DIT_ERR_INVALID_ARG                          # diff inside cur
    assert f(r=d + 4) == dj.DIT_ERR_INVALID_ARG                           # reuse over diff
    if _no_device():
        assert f() == dj.DIT_ERR_NO_DEVICE
        assert f(n=0, r=None) == dj.DIT_ERR_NO_DEVICE                     # empty residuals are valid
        assert f(n=0, p=None, c=None) == dj.DIT_ERR_NO_DEVICE             # ... also as NULL pointers
    # the allocation-free variant: the same checks, minus the workspace
    na = lambda **kw: L.dit_dbcache_residual_diff_noalloc(kw.get("p", p), kw.get("c", c), kw.get("n", 1000), 0.12,
                                                          kw.get("d", d), kw.get("r", r), None)
    assert na(p=None) == dj.DIT_ERR_INVALID_ARG
    assert na(d=None) == dj.DIT_ERR_INVALID_ARG
    assert na(n=-1) == dj.DIT_ERR_INVALID_ARG
    assert na(n=2 ** 40 + 1) == dj.DIT_ERR_UNSUPPORTED
    assert na(c=c + 2) == dj.DIT_ERR_INVALID_ARG                          # misaligned input
    assert na(d=d + 4) == dj.DIT_ERR_INVALID_ARG                          # misaligned diff
    assert na(d=c + 16) == dj.DIT_ERR_INVALID_ARG                         # diff inside cur
    assert na(r=d + 4) == dj.DIT_ERR_INVALID_ARG                          # reuse over diff
    if _no_device():
        assert na() == dj.DIT_ERR_NO_DEVICE
        assert na(n=0, p=None, c=None, r=None) == dj.DIT_ERR_NO_DEVICE


def test_clock_probe_rejects_bad_arguments():
    L = dj.lib()
    out = 0x30000000
    assert L.dit_clock_probe(None, 4096, 8, 10, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_clock_probe(out, 4096, 0, 10, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_clock_probe(out, 4096, 8, 0, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_clock_probe(out, 4096, 8, 2 ** 24 + 1, None) == dj.DIT_ERR_INVALID_ARG
    assert L.dit_clock_probe(out, 8 * 4 * 24 - 1, 8, 10, None) == dj.DIT_ERR_INVALID_ARG   # out too small
    assert L.dit_clock_probe(out + 4, 4096, 8, 10, None) == dj.DIT_ERR_INVALID_ARG         # misaligned
    assert L.dit_wall_clock_khz(None) == dj.DIT_ERR_INVALID_ARG
    if _no_device():
        assert L.dit_clock_probe(out, 4096, 8, 10, None) == dj.DIT_ERR_NO_DEVICE
