"""The allocation-free DBCache entry point (static device scratch) against the
workspace entry point, through the C ABI: identical difference and decision,
bit for bit, on two calls in a row, the second with a smaller input (so the
scratch holds the first call's partials when the second one starts)."""
import numpy as np
import pytest

import dit_workloads as W

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _dev(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


@pytest.mark.parametrize("first,second", [("flux2048_residual", "residual_ragged"),
                                          ("flux1024x768_residual", "residual_ragged")])
def test_noalloc_equals_workspace_entry_point(first, second):
    torch = _torch()
    import dit_joint_self_amd as dj
    ws = torch.empty(dj.dit_dbcache_workspace_bytes(), dtype=torch.uint8, device="cuda")
    for name in (first, second):
        rw = W.RESIDUAL_WORKLOADS[name]
        pb, cb = W.make_residual_inputs(rw)
        prev, cur = _dev(torch, pb), _dev(torch, cb)
        d_ws = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
        r_ws = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        d_na = torch.full((1,), -2.0, dtype=torch.float64, device="cuda")
        r_na = torch.full((1,), -2, dtype=torch.int32, device="cuda")
        for thr in (0.12, 0.2):
            dj.dit_dbcache_residual_diff(prev, cur, thr, ws=ws, diff=d_ws, reuse=r_ws)
            dj.dit_dbcache_residual_diff_noalloc(prev, cur, thr, d_na, r_na)
            torch.cuda.synchronize()
            a, b = float(d_ws.item()), float(d_na.item())
            print(f"[noalloc] {name} n={rw.n} thr={thr}: workspace {a!r} static {b!r} reuse {int(r_ws.item())}/"
                  f"{int(r_na.item())}", flush=True)
            assert np.float64(a).tobytes() == np.float64(b).tobytes(), (name, a, b)
            assert int(r_ws.item()) == int(r_na.item()) == (1 if a < thr else 0)


def test_noalloc_without_reuse_output_and_empty_input():
    torch = _torch()
    import dit_joint_self_amd as dj
    rw = W.RESIDUAL_WORKLOADS["residual_ragged"]
    pb, cb = W.make_residual_inputs(rw)
    prev, cur = _dev(torch, pb), _dev(torch, cb)
    d_na = torch.zeros(1, dtype=torch.float64, device="cuda")
    d_ws, _ = dj.dit_dbcache_residual_diff(prev, cur, 0.12)
    dj.dit_dbcache_residual_diff_noalloc(prev, cur, 0.12, d_na, None)
    torch.cuda.synchronize()
    assert np.float64(d_ws.item()).tobytes() == np.float64(d_na.item()).tobytes()
    e = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    r = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    dj.dit_dbcache_residual_diff_noalloc(e, e, 0.12, d_na, r)
    torch.cuda.synchronize()
    assert np.isinf(d_na.item()) and d_na.item() > 0 and int(r.item()) == 0
