"""The attention entry points with a caller-owned workspace allocate nothing
and clear nothing, so a caller can capture them in a HIP graph.  Each test
captures prepare + core once, then replays the graph several times with new
inputs copied into the captured buffers and with eager library work between
the replays, and checks every replay against the eager call on the same
inputs, bit for bit (the kernels are deterministic)."""
import numpy as np
import pytest

import dit_workloads as W
from tests.gpu_inputs import to_device_bf16

pytestmark = pytest.mark.gpu

# 336 (head, query-tile) items: a whole-range round plus key-range splits and
# their merge, so every kernel of the call is in the graph.
SHAPE = dict(B=1, H=24, D=128, S_txt=512, grid=(1, 48, 64), axes_dim=(16, 56, 56), theta=10000.0)


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _dj():
    import dit_joint_self_amd as dj
    return dj


def _workload(seed):
    return W.Workload("graph", seed=seed, **SHAPE)


def _tables(w):
    torch = _torch()
    pos = torch.from_numpy(W.positions(w)).to("cuda")
    return _dj().dit_rope_tables(pos, w.axes_dim, w.theta)


def _capture(fn):
    torch = _torch()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    return g


def test_bf16_prepare_core_lse_graph_replays():
    torch = _torch()
    dj = _dj()
    w0 = _workload(41)
    cos, sin = _tables(w0)
    draws = [W.make_bf16_inputs(_workload(41 + i)) for i in range(3)]
    q, k, v = (to_device_bf16(x) for x in draws[0])
    nbytes = dj.dit_attn_workspace_bytes(w0.B, w0.H, w0.S, w0.D)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    out2 = torch.empty_like(q)
    lse = torch.empty((w0.B, w0.H, w0.S), dtype=torch.float32, device="cuda")

    def call():
        dj.dit_attn_prepare_k(k, cos, sin, ws)
        dj.dit_attn_core(q, v, cos, sin, ws, out)
        dj.dit_attn_core_lse(q, v, cos, sin, ws, out2, lse)

    call()                                   # eager once before capture (device checks cached)
    torch.cuda.synchronize()
    g = _capture(call)
    for rep, (qb, kb, vb) in enumerate(draws + draws[::-1]):
        qe, ke, ve = (to_device_bf16(x) for x in (qb, kb, vb))
        # eager reference on separate buffers (also the eager work between replays)
        ws_e = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        want = torch.empty_like(qe)
        want2 = torch.empty_like(qe)
        want_lse = torch.empty_like(lse)
        dj.dit_attn_prepare_k(ke, cos, sin, ws_e)
        dj.dit_attn_core(qe, ve, cos, sin, ws_e, want)
        dj.dit_attn_core_lse(qe, ve, cos, sin, ws_e, want2, want_lse)
        torch.cuda.synchronize()
        q.copy_(qe)
        k.copy_(ke)
        v.copy_(ve)
        out.zero_()
        out2.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph bf16] replay {rep}", flush=True)
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), rep
        assert torch.equal(out2.view(torch.int16), want2.view(torch.int16)), rep
        assert torch.equal(lse, want_lse), rep


def test_fp8_prepare_core_graph_replays():
    torch = _torch()
    dj = _dj()
    w0 = _workload(51)
    cos, sin = _tables(w0)

    def draw(seed):
        (q8, sq), (k8, sk), (v8, sv) = [W.fp8_e4m3_quantize(x) for x in W.draw_qkv_f32(_workload(seed))]
        return [torch.from_numpy(np.ascontiguousarray(c)).to("cuda") for c in (q8, k8, v8)], (sq, sk, sv)

    draws = [draw(51 + i) for i in range(3)]
    (q, k, v), scales0 = draws[0]
    q, k, v = q.clone(), k.clone(), v.clone()
    nbytes = dj.dit_attn_workspace_bytes_fp8(w0.B, w0.H, w0.S, w0.D)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    # the per-tensor scales are captured as launch arguments: keep them fixed
    sq, sk, sv = scales0

    def call():
        dj.dit_attn_prepare_kv_fp8(k, v, sk, sv, cos, sin, ws)
        dj.dit_attn_core_fp8(q, sq, cos, sin, ws, out)

    call()
    torch.cuda.synchronize()
    g = _capture(call)
    for rep, ((qe, ke, ve), _) in enumerate(draws + draws[::-1]):
        ws_e = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        want = torch.empty_like(out)
        dj.dit_attn_prepare_kv_fp8(ke, ve, sk, sv, cos, sin, ws_e)
        dj.dit_attn_core_fp8(qe, sq, cos, sin, ws_e, want)
        torch.cuda.synchronize()
        q.copy_(qe)
        k.copy_(ke)
        v.copy_(ve)
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph fp8] replay {rep}", flush=True)
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), rep
