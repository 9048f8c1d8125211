"""DBCache reuse decision on the GPU (through the C ABI) against the float64
oracle (oracle.dbcache).

Gate on the difference: each |cur - prev| is one fp32 rounding of exact bf16
values, and the kernel adds 8 positive terms in fp32 before folding them into
fp64 sums, so each sum carries a relative error of at most 9 u (u = 2^-24)
plus the fp64 part (n 2^-53, below 2^-22 for every size here). The ratio then
lies within 2 x (9 u + 2^-22) < 2^-19 of the exact one, relatively. The
decision is a comparison of the kernel's own fp64 difference with the
threshold, so it must agree exactly with `diff < threshold` on the returned
value, and with the oracle's decision wherever the oracle's difference is
farther than the gate from the threshold.
"""
import math

import numpy as np
import pytest

import dit_workloads as W
from oracle.dbcache import residual_diff

pytestmark = pytest.mark.gpu

REL_GATE = 2.0 ** -19


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _dj():
    import dit_joint_self_amd as dj
    return dj


def _dev(bits):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def _run(prev_bits, cur_bits, threshold):
    torch = _torch()
    diff, reuse = _dj().dit_dbcache_residual_diff(_dev(prev_bits), _dev(cur_bits), threshold)
    torch.cuda.synchronize()
    return float(diff.cpu().numpy()[0]), int(reuse.cpu().numpy()[0])


def _check(prev_bits, cur_bits, threshold, tag):
    got, reuse = _run(prev_bits, cur_bits, threshold)
    want = residual_diff(W.bf16_bits_to_f32(prev_bits), W.bf16_bits_to_f32(cur_bits))
    print(f"[dbcache parity] {tag}: n {prev_bits.size}, gpu {got!r}, oracle {want!r}", flush=True)
    if math.isinf(want):
        assert math.isinf(got) and got > 0 and reuse == 0, tag
        return got
    assert abs(got - want) <= REL_GATE * want, tag
    assert reuse == (1 if got < threshold else 0), tag
    if abs(want - threshold) > REL_GATE * want:
        assert reuse == (1 if want < threshold else 0), tag
    return got


def _pair(n, rel, seed):
    rng = np.random.default_rng(seed)
    p = rng.standard_normal(n, dtype=np.float32) * np.exp(rng.standard_normal(n, dtype=np.float32))
    c = p + np.float32(rel) * rng.standard_normal(n, dtype=np.float32)
    return W.bf16_round_bits(p), W.bf16_round_bits(c)


# sizes: one element, below / at / past one 8-element chunk, several blocks
# with ragged tails, more chunks than one pass of the largest grid (8192 blocks
# x 256 threads, one chunk each) with a ragged tail
@pytest.mark.parametrize("n", [1, 7, 8, 9, 1000, 8 * 1024 * 5 + 3, 2048 * 256 * 8 * 4 + 8 * 777 + 5])
def test_random_sizes(n):
    p, c = _pair(n, 0.1, n)
    _check(p, c, 0.12, f"n={n}")


@pytest.mark.parametrize("name", ["residual_ragged", "flux1024x768_residual"])
def test_workloads(name):
    p, c = W.make_residual_inputs(W.RESIDUAL_WORKLOADS[name])
    d = _check(p, c, 0.12, name)
    assert abs(d - W.RESIDUAL_WORKLOADS[name].rel_change) < 0.02 * W.RESIDUAL_WORKLOADS[name].rel_change


def test_full_size():
    """The 16896 x 3072 residual of the 2048x2048 sequence, in the launch the
    benchmark times, against the oracle over every element."""
    w = W.RESIDUAL_WORKLOADS["flux2048_residual"]
    p, c = W.make_residual_inputs(w)
    _check(p, c, 0.12, w.name)


def test_special_cases():
    torch = _torch()
    dj = _dj()
    p, c = _pair(4099, 0.3, 7)
    # cur == prev: exactly 0, reused for any positive threshold
    assert _run(p, p, 1e-300) == (0.0, 1)
    # cur = 2 prev (exact in bf16): |cur - prev| = |prev| term by term, so num and den are the same sums
    two = W.bf16_round_bits(2.0 * W.bf16_bits_to_f32(p))
    assert _run(p, two, 1.0) == (1.0, 0)
    assert _run(p, two, 1.0000001) == (1.0, 1)
    # cur = 0: the difference is exactly 1
    assert _run(p, np.zeros_like(p), 0.12) == (1.0, 0)
    # previous residual all zero: +inf, never reused
    d, r = _run(np.zeros_like(p), c, 1e300)
    assert math.isinf(d) and d > 0 and r == 0
    # empty residuals: +inf, no reuse
    e = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    diff, reuse = dj.dit_dbcache_residual_diff(e, e, 0.12)
    torch.cuda.synchronize()
    assert math.isinf(float(diff.item())) and int(reuse.item()) == 0
    # NaN in the current residual: NaN difference, no reuse
    nan = c.copy()
    nan[100] = 0x7FC0
    d, r = _run(p, nan, 1e300)
    assert math.isnan(d) and r == 0
    # negative zero and subnormal bf16 values count like their magnitudes
    tiny = W.bf16_round_bits(np.array([1e-40, -1e-40, -0.0, 0.0, 3e-39, -2e-39, 1.0, -1.0, 5e-41], np.float32))
    _check(tiny, W.bf16_round_bits(np.zeros(9, np.float32)), 0.5, "subnormal prev")
    _check(tiny, tiny[::-1].copy(), 0.5, "subnormal both")


def test_threshold_straddle_and_reuse_pointer_optional():
    torch = _torch()
    dj = _dj()
    p, c = _pair(123457, 0.1, 11)
    got, _ = _run(p, c, 0.12)
    assert _run(p, c, got * (1 + 1e-9))[1] == 1
    assert _run(p, c, got * (1 - 1e-9))[1] == 0
    assert _run(p, c, got)[1] == 0                      # strict comparison
    ws = torch.empty(dj.dit_dbcache_workspace_bytes(), dtype=torch.uint8, device="cuda")
    diff = torch.empty(1, dtype=torch.float64, device="cuda")
    pd, cd = _dev(p), _dev(c)
    st = dj.lib().dit_dbcache_residual_diff(pd.data_ptr(), cd.data_ptr(), p.size, 0.12, ws.data_ptr(),
                                            ws.numel(), diff.data_ptr(), None,
                                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == dj.DIT_OK and float(diff.item()) == got


def test_deterministic():
    p, c = _pair(3_000_001, 0.1, 12)
    a = _run(p, c, 0.12)
    assert all(_run(p, c, 0.12) == a for _ in range(3))


def test_graph_replays_match_eager():
    """Both launches captured in a graph: each replay, with new residuals
    copied in and eager work between replays, equals the eager call."""
    torch = _torch()
    dj = _dj()
    n = 1_000_003
    pairs = [_pair(n, r, 20 + i) for i, r in enumerate([0.05, 0.2, 0.11, 0.13])]
    prev, cur = _dev(pairs[0][0]), _dev(pairs[0][1])
    ws = torch.empty(dj.dit_dbcache_workspace_bytes(), dtype=torch.uint8, device="cuda")
    diff = torch.empty(1, dtype=torch.float64, device="cuda")
    reuse = torch.empty(1, dtype=torch.int32, device="cuda")
    dj.dit_dbcache_residual_diff(prev, cur, 0.12, ws=ws, diff=diff, reuse=reuse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            dj.dit_dbcache_residual_diff(prev, cur, 0.12, ws=ws, diff=diff, reuse=reuse)
    torch.cuda.synchronize()
    for pb, cb in pairs + pairs[::-1]:
        prev.copy_(_dev(pb))
        cur.copy_(_dev(cb))
        want = _run(pb, cb, 0.12)
        diff.fill_(-1.0)
        reuse.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert (float(diff.item()), int(reuse.item())) == want
