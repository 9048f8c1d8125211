"""Benchmark: joint self-attention TFLOP/s on one MI355X.

One step = one whole pass of the path over one batch of synthetic input:
RoPE on K + its tile layout (dit_attn_prepare_k) and the attention kernel
with RoPE on Q fused into its prologue (dit_attn_core), i.e. the work of
dit_attn_forward.  RoPE tables are built once per resolution (outside the
step), as a DiT reuses them across all blocks and denoising steps.

Prints one JSON line.  `value` is attention TFLOP/s (4 B H S^2 D flop per
step) over the timed steps; `roofline` prices the attention kernel alone
against the dense bf16 MFMA peak; `cpu_baseline` times the float64 oracle on
a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

import dit_workloads as W

METRIC = "attention TFLOP/s and % of bf16 MFMA peak at S=16896,H=24,D=128 (1 GPU)"

# HBM bytes per kernel launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by a
# plain-copy calibration), keyed by the hash of the sources of the kernel they were taken on
# and by workload; reported as roofline.traffic only while those sources are unchanged.
BF16_SOURCES = ["dit_joint_self_amd/csrc/attn_core.hip", "dit_joint_self_amd/csrc/attn_common.h",
                "dit_joint_self_amd/csrc/gfx950.h", "dit_joint_self_amd/csrc/tile_layout.h",
                "dit_joint_self_amd/csrc/bf16_util.h"]
# (the fp8 call's merge kernel lives in attn_core.hip)
FP8_SOURCES = ["dit_joint_self_amd/csrc/attn_core_fp8.hip", "dit_joint_self_amd/csrc/attn_core.hip",
               "dit_joint_self_amd/csrc/attn_common.h",
               "dit_joint_self_amd/csrc/gfx950.h", "dit_joint_self_amd/csrc/tile_layout.h",
               "dit_joint_self_amd/csrc/bf16_util.h", "dit_joint_self_amd/csrc/fp8_util.h"]
KERNEL_SOURCES = BF16_SOURCES
MEASURED_TRAFFIC = {
    # dit_attn_core (attn_core_kernel + attn_merge_kernel), hash over BF16_SOURCES
    ("fa548de7e9f15bb5", "flux2048"): {"read_bytes": 1051.6e6, "write_bytes": 135.8e6,
                                       "profile": "profiles/attn_core_flux2048.md"},
    # dit_attn_core_fp8 (attn_core_fp8_kernel + attn_merge_kernel), hash over FP8_SOURCES
    ("65b1ca7361f29fcd", "flux2048_fp8"): {"read_bytes": 707.0e6, "write_bytes": 135.8e6,
                                           "profile": "profiles/attn_core_fp8_flux2048.md"},
    # mxfp4_gemm_kernel alone (hash over MXFP4_SOURCES)
    ("3f50413424c15d89", "flux2048_qkv"): {"read_bytes": 547.2e6, "write_bytes": 349.2e6,
                                           "profile": "profiles/mxfp4_gemm_flux2048_qkv.md"},
    # residual_diff_partials + residual_diff_finish (hash over RESIDUAL_SOURCES)
    ("ab5d6a5aa3060f98", "flux2048_residual"): {"read_bytes": 207.80e6, "write_bytes": 0.26e6,
                                                "profile": "profiles/dbcache_residual_diff_flux2048.md"},
}


MXFP4_SOURCES = ["dit_joint_self_amd/csrc/mxfp4.hip", "dit_joint_self_amd/csrc/gfx950.h",
                 "dit_joint_self_amd/csrc/bf16_util.h"]
RESIDUAL_SOURCES = ["dit_joint_self_amd/csrc/dbcache.hip", "dit_joint_self_amd/csrc/gfx950.h"]


def kernel_sources_hash(files=None) -> str:
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for f in files or KERNEL_SOURCES:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]
BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz, dense
FP8_PEAK_TFLOPS = 5033.2    # 256 CU x 8192 flop/clk x 2.4 GHz, dense
FP4_PEAK_TFLOPS = 10066.3   # 256 CU x 16384 flop/clk x 2.4 GHz, dense
HBM_PEAK_GBS = 8000.0


def clock_record(torch, dj, kernel_tflops, step_tflops, flop_per_clk_per_cu):
    """Peak recomputed from the device's CU count and the shader clock that a
    bf16 MFMA load on every CU runs at (the clock probe, right after the timed
    steps), and the two rates priced against it."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ghz, probe_tflops = dj.dit_clock_probe(blocks=2 * cus, iters=20000)
    peak = cus * flop_per_clk_per_cu * ghz * 1e9 / 1e12
    return {"probe_GHz": ghz, "cus": cus, "peak_at_probe_clock_TFLOPs": peak,
            "probe_mfma_TFLOPs": probe_tflops,
            "pct_of_peak_at_probe_clock": 100.0 * step_tflops / peak,
            "kernel_frac_at_probe_clock": kernel_tflops / peak}


def _traffic(files, workload):
    """Measured HBM bytes per launch while the kernel sources match the ones profiled, else None."""
    meas = MEASURED_TRAFFIC.get((kernel_sources_hash(files), workload))
    return None if meas is None else meas["read_bytes"] + meas["write_bytes"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="flux2048",
                    choices=list(W.WORKLOADS) + list(W.LINEAR_WORKLOADS) + list(W.RESIDUAL_WORKLOADS),
                    help="an attention workload, or an MXFP4 linear-layer shape (quantise + A4W4 GEMM)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="time budget of the oracle sample")
    ap.add_argument("--prewarm-s", type=float, default=0.5,
                    help="seconds of untimed back-to-back steps before the warmup steps (clock ramp-up)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-library-baseline", action="store_true",
                    help="skip timing the library's own kernel on the same shape (PyTorch SDPA / _scaled_mm)")
    ap.add_argument("--single-config", action="store_true",
                    help="time only --workload (by default an attention run also times every other attention "
                         "workload and reports them under `configs`)")
    ap.add_argument("--ring", type=int, default=1,
                    help="time one rank's share of a ring of this many ranks (bf16 workloads): its query shard "
                         "against every key/value block, folded with the LSE merge")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of attention, time a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def copy_calibration(args, torch):
    """A plain device-to-device copy of known size, run under the same counters
    as the attention kernel so FETCH_SIZE / WRITE_SIZE can be scaled to bytes."""
    n = args.copy_mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({"copy_bytes": n, "read_bytes": n, "write_bytes": n, "ms": ms,
                      "GBps_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}), flush=True)


def ws_bytes_tiles(w, fp8):
    """Bytes of prepared tiles the attention kernel streams: 64-key K' tiles of
    17408 B (bf16; V is read as it is) or K'/V^T tiles of 19456 B (fp8, plus its
    256 B scale header) per (b, h)."""
    tiles = w.B * w.H * ((w.S + 63) // 64)
    return tiles * 19456 + 256 if fp8 else tiles * 17408


def bf16_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def host_info():
    """CPU model, usable host cores and the BLAS thread count numpy runs its
    products with (the oracle's matrix products are its multi-threaded part)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas_threads, blas = 1, "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            blas_threads = max(int(p.get("num_threads", 1)) for p in libs)
            blas = ",".join(sorted({str(p.get("internal_api", "?")) for p in libs}))
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass
    return {"cpu_model": model, "host_cpus": len(os.sched_getaffinity(0)), "blas_threads": blas_threads,
            "blas": blas}


def cpu_baseline(w, f64_head, budget_s, gpu_rows=None):
    """The float64 oracle as it stands, on the first query rows of successive
    heads until the time budget is spent; TFLOP/s at 4 * rows * S * D flop.
    ``f64_head(h)`` returns the head's (q, k, v) as float64 [1, 1, S, D].
    ``gpu_rows(h, rows)`` returns the timed GPU output of those rows of head h
    ([1, 1, R, D], float64): every oracle row computed for the timing, in every
    head reached, is compared with it (max and mean |diff|, outside the timed
    oracle time)."""
    from oracle import joint_attention, rope_angles
    info = host_info()
    ang = rope_angles(W.positions(w), w.axes_dim, w.theta)
    rows_per_head = min(w.S, 8192)
    rows = np.arange(rows_per_head)
    t0 = time.perf_counter()
    done_rows = 0
    heads = 0
    dmax, dsum, dn, osum = 0.0, 0.0, 0, 0.0
    for h in range(w.H):
        q, k, v = f64_head(h)
        ref = joint_attention(q, k, v, ang, rows=rows)
        if gpu_rows is not None:
            tc = time.perf_counter()
            d = np.abs(gpu_rows(h, rows) - ref)
            dmax = max(dmax, float(d.max()))
            dsum += float(d.sum())
            osum += float(np.abs(ref).sum())
            dn += d.size
            t0 += time.perf_counter() - tc  # the comparison is not oracle time
        done_rows += rows_per_head
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 4.0 * done_rows * w.S * w.D
    rec = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(info["blas_threads"]), "kind": "oracle",
           "sample": f"{w.name}: first {rows_per_head} query rows x {heads} of {w.H} heads vs all {w.S} keys, "
                     f"float64 numpy (incl. RoPE of the head's K), {dt:.1f} s; cores = numpy's BLAS threads "
                     f"(the products), the softmax passes run on one",
           **info}
    if gpu_rows is not None:
        rec["sample_parity"] = {"compared": f"all {done_rows} rows x {w.D} dims computed ({heads} heads)",
                                "max_abs": dmax, "mean_abs": dsum / max(dn, 1),
                                "rel_mean": dsum / max(osum, 1e-300)}
    return rec


def ring_bench(args, w, torch, dj):
    """One rank of a P-way ring on one GPU: the rank holds query shard 0 (S/P rows)
    and receives the P key/value blocks of S/P tokens in ring order; for each
    block it prepares the tiles (the block's own RoPE tables), runs attention
    with the row LSE and folds the result into its running output in place."""
    P = args.ring
    if w.dtype != "bf16" or w.S % P:
        print(f"--ring {P} needs a bf16 workload whose S is a multiple of {P}", file=sys.stderr)
        sys.exit(2)
    n = w.S // P
    stream = torch.cuda.current_stream()
    qb, kb, vb = W.make_bf16_inputs(w)
    q, k, v = bf16_dev(qb, torch), bf16_dev(kb, torch), bf16_dev(vb, torch)
    pos = W.positions(w)
    tabs = [dj.dit_rope_tables(torch.from_numpy(np.ascontiguousarray(pos[b * n:(b + 1) * n])).to("cuda"),
                               w.axes_dim, w.theta) for b in range(P)]
    qs = q[:, :, :n].contiguous()
    kbk = [k[:, :, b * n:(b + 1) * n].contiguous() for b in range(P)]
    vbk = [v[:, :, b * n:(b + 1) * n].contiguous() for b in range(P)]
    ws_bytes = dj.dit_attn_workspace_bytes(w.B, w.H, n, w.D)
    ws = [torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") for _ in range(P)]
    outs = [torch.empty_like(qs) for _ in range(P)]
    lses = [torch.empty((w.B, w.H, n), dtype=torch.float32, device="cuda") for _ in range(P)]
    scale = 1.0 / math.sqrt(w.D)

    def step(ev):
        for b in range(P):
            ev.append(torch.cuda.Event(enable_timing=True)); ev[-1].record(stream)
            dj.dit_attn_prepare_k(kbk[b], tabs[b][0], tabs[b][1], ws[b], ws_bytes, stream=stream)
            ev.append(torch.cuda.Event(enable_timing=True)); ev[-1].record(stream)
            dj.dit_attn_core_lse(qs, vbk[b], tabs[0][0], tabs[0][1], ws[b], outs[b], lses[b], scale=scale,
                                 workspace_bytes=ws_bytes, stream=stream)
            ev.append(torch.cuda.Event(enable_timing=True)); ev[-1].record(stream)
            if b > 0:
                dj.dit_attn_merge_lse(outs[0], lses[0], outs[b], lses[b], out=outs[0], lse_out=lses[0],
                                      stream=stream)
            ev.append(torch.cuda.Event(enable_timing=True)); ev[-1].record(stream)

    prewarm(torch, lambda: step([]), args.prewarm_s)
    for _ in range(args.warmup):
        step([])
    torch.cuda.synchronize()
    K = args.steps
    evs = [[] for _ in range(K)]
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    prep = [sum(e[4 * b].elapsed_time(e[4 * b + 1]) for b in range(P)) for e in evs]
    core = [sum(e[4 * b + 1].elapsed_time(e[4 * b + 2]) for b in range(P)) for e in evs]
    merge = [sum(e[4 * b + 2].elapsed_time(e[4 * b + 3]) for b in range(1, P)) for e in evs]
    steps_ms = [e[0].elapsed_time(e[-1]) for e in evs]
    step_ms = evs[0][0].elapsed_time(evs[-1][-1]) / K

    flops = 4.0 * w.B * w.H * n * w.S * w.D
    core_avg = float(np.mean(core))
    achieved = flops / (core_avg * 1e-3) / 1e12
    rows_all = w.B * w.H * n
    merge_bytes = rows_all * (2 * w.D * 2 + 8 + w.D * 2 + 4)
    merge_avg = float(np.mean(merge)) / max(P - 1, 1)
    rec = {
        "metric": METRIC,
        "value": flops / (step_ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "ms_per_step_median": float(np.median(steps_ms)),
        "ms_per_step_min": float(np.min(steps_ms)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name} ring of {P}: one rank ({n} query rows x {P} key/value blocks of {n})",
                   "B": w.B, "H": w.H, "S": w.S, "D": w.D, "ranks_in_ring": P, "non_causal": True},
        "pct_of_peak": 100.0 * flops / (step_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "roofline": {"bound": "mfma", "kernel": "dit_attn_core_lse: attn_core_kernel + attn_merge_kernel",
                     "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None, "avg_ms": core_avg / P},
        "stages_ms": {"prepare_kv_all_blocks": float(np.mean(prep)), "attn_core_lse_all_blocks": core_avg,
                      "merge_all": float(np.mean(merge))},
        "merge": {"bound": "hbm", "avg_ms": merge_avg, "algorithmic_bytes": merge_bytes,
                  "achieved_GBps": merge_bytes / (merge_avg * 1e-3) / 1e9 if P > 1 else None,
                  "peak_GBps": HBM_PEAK_GBS},
    }
    print(json.dumps(rec), flush=True)


def gemm_bench(args, lw, torch, dj):
    """MXFP4 linear layer: one step = dit_mxfp4_linear on bf16 activations
    [M, K] with a weight [N, K] quantised beforehand (the activation quantiser
    and the A4W4 GEMM, the two kernels of the layer); the GEMM is also timed
    alone for the roofline."""
    xb, wb = W.make_linear_inputs(lw)
    x, w = bf16_dev(xb, torch), bf16_dev(wb, torch)
    stream = torch.cuda.current_stream()
    wc, ws = dj.dit_mxfp4_quantize(w, stream=stream)
    ac, as_ = dj.dit_mxfp4_quantize(x, stream=stream)
    out = torch.empty((lw.M, lw.N), dtype=torch.bfloat16, device="cuda")
    step = lambda: dj.dit_mxfp4_linear(x, wc, ws, out=out, stream=stream)
    gemm = lambda: dj.dit_mxfp4_gemm(ac, as_, wc, ws, out=out, stream=stream)
    quant = lambda: dj.dit_mxfp4_quantize(x, ac, as_, stream=stream)

    def timed(fn, K):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in ev]

    prewarm(torch, lambda: (step(), gemm(), quant()), args.prewarm_s)
    for _ in range(args.warmup):
        step(); gemm(); quant()
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / K
    gemm_ms = timed(gemm, K)
    quant_ms = timed(quant, K)
    g_avg, q_avg = float(np.mean(gemm_ms)), float(np.mean(quant_ms))
    flops = lw.flops
    gemm_bytes = lw.M * lw.K // 2 + lw.M * lw.K // 32 + lw.N * lw.K // 2 + lw.N * lw.K // 32 + 2 * lw.M * lw.N
    quant_bytes = 2 * lw.M * lw.K + lw.M * lw.K // 2 + lw.M * lw.K // 32
    rec = {
        "metric": "MXFP4 linear-layer TFLOP/s (dynamic 1x32 activation quantisation + A4W4 GEMM), 1 GPU",
        "value": flops / (step_ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 (e2m1 + e8m0 per 32), bf16 in/out",
        "data": "synthetic",
        "config": {"workload": lw.name, "M": lw.M, "N": lw.N, "K": lw.K, "note": lw.note},
        "pct_of_peak": 100.0 * flops / (step_ms * 1e-3) / 1e12 / FP4_PEAK_TFLOPS,
        "roofline": {"bound": "mfma", "kernel": "mxfp4_gemm_kernel", "achieved": flops / (g_avg * 1e-3) / 1e12,
                     "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / (g_avg * 1e-3) / 1e12 / FP4_PEAK_TFLOPS, "traffic": _traffic(MXFP4_SOURCES, lw.name),
                     "algorithmic_bytes": gemm_bytes, "avg_ms": g_avg},
        "stages_ms": {"mxfp4_quantize": q_avg, "mxfp4_gemm": g_avg,
                      "quantize_GBps": quant_bytes / (q_avg * 1e-3) / 1e9},
    }
    if not args.no_library_baseline:
        rec["library_baseline"] = library_gemm(lw, torch, K, ac, wc, g_avg)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        from oracle.mx import mx_linear, mxfp4_quantize
        w_c, w_s = mxfp4_quantize(W.bf16_bits_to_f32(wb).astype(np.float64))
        xf = W.bf16_bits_to_f32(xb).astype(np.float64)
        rows = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds and rows < lw.M:
            a_c, a_s = mxfp4_quantize(xf[rows:rows + 64])
            ref = mx_linear(a_c, a_s, w_c, w_s)
            if rows == 0:
                tc = time.perf_counter()
                got = out[:64].float().cpu().numpy().astype(np.float64)
                parity = float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))
                t0 += time.perf_counter() - tc
            rows += 64
        dt = time.perf_counter() - t0
        info = host_info()
        rec["cpu_baseline"] = {"value": 2.0 * rows * lw.N * lw.K / dt / 1e12, "unit": "TFLOP/s",
                               "cores": int(info["blas_threads"]), "kind": "oracle",
                               "sample": f"{lw.name}: quantise + float64 product of the first {rows} of {lw.M} rows "
                                         f"(weight quantised beforehand), {dt:.1f} s",
                               **info, "sample_parity_max_rel": parity}
    print(json.dumps(rec), flush=True)


def residual_bench(args, rw, torch, dj):
    """DBCache reuse decision: one step = dit_dbcache_residual_diff over two
    bf16 residuals of one step pair (the partial-sum kernel and the one-block
    finish).  HBM bound: the algorithmic bytes are the two residuals, read once."""
    pb, cb = W.make_residual_inputs(rw)
    prev, cur = bf16_dev(pb, torch), bf16_dev(cb, torch)
    stream = torch.cuda.current_stream()
    ws = torch.empty(dj.dit_dbcache_workspace_bytes(), dtype=torch.uint8, device="cuda")
    diff = torch.empty(1, dtype=torch.float64, device="cuda")
    reuse = torch.empty(1, dtype=torch.int32, device="cuda")
    step = lambda: dj.dit_dbcache_residual_diff(prev, cur, 0.12, ws=ws, diff=diff, reuse=reuse, stream=stream)
    prewarm(torch, step, args.prewarm_s)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    nbytes = 4.0 * rw.n
    gbs = nbytes / (step_ms * 1e-3) / 1e9
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    rec = {
        "metric": "DBCache residual-difference GB/s (relative L1 distance of two bf16 residuals + decision), 1 GPU",
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, fp32/fp64 sums",
        "data": "synthetic",
        "config": {"workload": rw.name, "tokens": rw.tokens, "hidden": rw.hidden, "n": rw.n, "note": rw.note},
        "decision": {"diff": float(diff.item()), "reuse": int(reuse.item()), "threshold": 0.12},
        "roofline": {"bound": "hbm", "kernel": "residual_diff_partials + residual_diff_finish (one call)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": _traffic(RESIDUAL_SOURCES, rw.name), "algorithmic_bytes": nbytes, "avg_ms": call_ms},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        from oracle.dbcache import residual_diff
        rows, chunk = 0, 512
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds and rows < rw.tokens:
            residual_diff(W.bf16_bits_to_f32(pb[rows:rows + chunk]), W.bf16_bits_to_f32(cb[rows:rows + chunk]))
            rows += chunk
        dt = time.perf_counter() - t0
        rows = min(rows, rw.tokens)
        rec["cpu_baseline"] = {"value": 4.0 * rows * rw.hidden / dt / 1e9, "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{rw.name}: the float64 difference over the first {rows} of {rw.tokens} "
                                         f"tokens in chunks of {chunk}, {dt:.1f} s (numpy element-wise passes: "
                                         f"one thread)",
                               **host_info()}
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library runs on one GPU (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import dit_joint_self_amd as dj

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_mib:
        copy_calibration(args, torch)
        return
    if args.workload in W.LINEAR_WORKLOADS:
        gemm_bench(args, W.LINEAR_WORKLOADS[args.workload], torch, dj)
        return
    if args.workload in W.RESIDUAL_WORKLOADS:
        residual_bench(args, W.RESIDUAL_WORKLOADS[args.workload], torch, dj)
        return
    w = W.get(args.workload)
    if args.ring > 1:
        ring_bench(args, w, torch, dj)
        return
    print(f"[bench] workload {w.name}: B={w.B} H={w.H} S={w.S} D={w.D} {w.dtype}", file=sys.stderr, flush=True)
    run = AttentionRun(w, torch, dj)
    timing = run.time_steps(args.steps, args.warmup, args.prewarm_s)
    fwd_ms = run.time_forward(args.steps)
    fp8, flops, peak = run.fp8, w.flops, run.peak
    step_ms, core_avg, prep_avg = timing["step_ms"], timing["core_ms"], timing["prep_ms"]
    src_hash = kernel_sources_hash(FP8_SOURCES if fp8 else BF16_SOURCES)
    meas = MEASURED_TRAFFIC.get((src_hash, w.name))
    traffic = None if meas is None else meas["read_bytes"] + meas["write_bytes"]
    achieved = flops / (core_avg * 1e-3) / 1e12
    tensor_bytes = w.B * w.H * w.S * w.D * (1 if fp8 else 2)
    # read Q, the prepared tiles and the two tables; write the bf16 output
    tables = 2 * w.S * (w.D // 2) * 4
    # core: read Q, the prepared tiles (bf16: K' only, plus V as it is) and the two tables; write the bf16 output
    core_bytes = (tensor_bytes + ws_bytes_tiles(w, fp8) + (0 if fp8 else tensor_bytes) + tables
                  + w.B * w.H * w.S * w.D * 2)
    # preparation: read K (fp8: and V) and the tables; write the prepared tiles
    prep_bytes = (2 if fp8 else 1) * tensor_bytes + tables + ws_bytes_tiles(w, fp8)
    rec = {
        "metric": METRIC,
        "value": flops / (step_ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "ms_per_step_median": timing["step_median_ms"],
        "ms_per_step_min": timing["step_min_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S_txt": w.S_txt, "S_img": w.S_img, "S": w.S,
                   "D": w.D, "rope_axes": list(w.axes_dim), "non_causal": True},
        "pct_of_peak": 100.0 * flops / (step_ms * 1e-3) / 1e12 / peak,
        "roofline": {"bound": "mfma",
                     "kernel": ("dit_attn_core_fp8: attn_core_fp8_kernel" if fp8 else "dit_attn_core: attn_core_kernel")
                               + " (whole-range workgroups and key-range pieces, one launch) + attn_merge_kernel",
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     "frac_timing": "HIP events on the launch stream around each dit_attn_core call, mean over the "
                                    "timed steps (a rocprofv3 kernel trace of the same command is in profiles/)",
                     "traffic": traffic, "traffic_unit": "HBM bytes per dit_attn_core call (read + write)",
                     "hbm_GBps": None if traffic is None else traffic / (core_avg * 1e-3) / 1e9,
                     "algorithmic_bytes": core_bytes, "avg_ms": core_avg, "kernel_sources": src_hash},
        "stages_ms": {"prepare_kv": prep_avg, "attn_core": core_avg,
                      "prepare_kv_GBps": prep_bytes / (prep_avg * 1e-3) / 1e9,
                      "prepare_kv_algorithmic_bytes": prep_bytes},
        "forward_ms": fwd_ms,
        "wall_s": timing["wall_s"],
        "prewarm": {"seconds": args.prewarm_s, "steps": run.prewarm_steps,
                    "why": "untimed steps before the warmup steps: the shader clock ramps up over the first tens of "
                           "ms of sustained load after an idle spell (first calls up to 20% slower)"},
        "clock": clock_record(torch, dj, achieved, flops / (step_ms * 1e-3) / 1e12, 8192 if fp8 else 4096),
    }
    out_host = run.out.cpu()
    f64_head = run.f64_head
    run.release()
    if not args.no_library_baseline:
        rec["library_baseline"] = library_attention(w, torch, args.steps, core_avg)
    if not args.single_config:
        rec["configs"] = other_configs(w, args, torch, dj)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)

        def gpu_rows(h, rows):
            bits = out_host[:, h:h + 1, torch.from_numpy(rows)].view(torch.int16).numpy().view(np.uint16)
            return W.bf16_bits_to_f32(bits).astype(np.float64)

        rec["cpu_baseline"] = cpu_baseline(w, f64_head, args.cpu_seconds, gpu_rows)
    print(json.dumps(rec), flush=True)


def prewarm(torch, step, seconds):
    """Run `step` back to back until `seconds` of wall time have passed
    (synchronising every few steps so the queue stays short); returns the
    number of steps run.  Brings the GPU from its idle clock to the clock it
    holds under sustained load before anything is timed."""
    n = 0
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(4):
            step()
        n += 4
        torch.cuda.synchronize()
    return n


class AttentionRun:
    """Device inputs, RoPE tables, workspace and output of one attention
    workload, with the two stages of a step (prepare_kv, core) as closures."""

    def __init__(self, w, torch, dj):
        self.w, self.torch, self.dj = w, torch, dj
        self.fp8 = w.dtype == "fp8_e4m3"
        pos = torch.from_numpy(W.positions(w)).to("cuda")
        cos, sin = dj.dit_rope_tables(pos, w.axes_dim, w.theta)
        scale = 1.0 / math.sqrt(w.D)
        stream = self.stream = torch.cuda.current_stream()
        if self.fp8:
            (q8, sq), (k8, sk), (v8, sv) = [W.fp8_e4m3_quantize(x) for x in W.draw_qkv_f32(w)]
            q, k, v = (torch.from_numpy(np.ascontiguousarray(c)).to("cuda") for c in (q8, k8, v8))
            self.out = out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
            ws_bytes = dj.dit_attn_workspace_bytes_fp8(w.B, w.H, w.S, w.D)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
            self.prep = lambda: dj.dit_attn_prepare_kv_fp8(k, v, sk, sv, cos, sin, ws, ws_bytes, stream=stream)
            self.core = lambda: dj.dit_attn_core_fp8(q, sq, cos, sin, ws, out, scale=scale, workspace_bytes=ws_bytes,
                                                     stream=stream)
            self.forward = lambda: dj.dit_attn_forward_fp8(q, k, v, sq, sk, sv, cos, sin, out=out, S_txt=w.S_txt,
                                                           scale=scale)

            def f64_head(h):  # the oracle's dequantisation, for the CPU baseline leg only
                from oracle.fp8 import dequantize
                return tuple(dequantize(c[:, h:h + 1], s_) for c, s_ in ((q8, sq), (k8, sk), (v8, sv)))
            self.f64_head = f64_head
            self.peak = FP8_PEAK_TFLOPS
        else:
            qb, kb, vb = W.make_bf16_inputs(w)
            q, k, v = bf16_dev(qb, torch), bf16_dev(kb, torch), bf16_dev(vb, torch)
            self.out = out = torch.empty_like(q)
            ws_bytes = dj.dit_attn_workspace_bytes(w.B, w.H, w.S, w.D)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
            self.prep = lambda: dj.dit_attn_prepare_k(k, cos, sin, ws, ws_bytes, stream=stream)
            self.core = lambda: dj.dit_attn_core(q, v, cos, sin, ws, out, scale=scale, workspace_bytes=ws_bytes,
                                                 stream=stream)
            self.forward = lambda: dj.dit_attn_forward(q, k, v, cos, sin, out=out, S_txt=w.S_txt, scale=scale)
            self.f64_head = lambda h: tuple(W.bf16_bits_to_f32(b[:, h:h + 1]).astype(np.float64) for b in (qb, kb, vb))
            self.peak = BF16_PEAK_TFLOPS

    def time_steps(self, K, warmup, prewarm_s=0.0):
        """Steps back to back for `prewarm_s` seconds (untimed: the shader clock
        ramps up over the first tens of milliseconds of sustained load after an
        idle spell), then `warmup` untimed steps, then K steps; each stage
        bracketed by HIP events on the launch stream."""
        torch, stream = self.torch, self.stream
        self.prewarm_steps = prewarm(torch, lambda: (self.prep(), self.core()), prewarm_s)
        for _ in range(warmup):
            self.prep()
            self.core()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
        t0 = time.perf_counter()
        for i in range(K):
            ev[i][0].record(stream)
            self.prep()
            ev[i][1].record(stream)
            self.core()
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        steps_ms = [ev[i][0].elapsed_time(ev[i][2]) for i in range(K)]
        return {"step_ms": ev[0][0].elapsed_time(ev[K - 1][2]) / K,
                "step_median_ms": float(np.median(steps_ms)), "step_min_ms": float(np.min(steps_ms)),
                "prep_ms": float(np.mean([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)])),
                "core_ms": float(np.mean([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)])),
                "wall_s": wall}

    def time_forward(self, K):
        """The allocating entry point itself (workspace from the stream pool), for reference."""
        torch = self.torch
        for _ in range(2):
            self.forward()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(K):
            self.forward()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    def release(self):
        self.prep = self.core = self.forward = None
        self.out = None
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def _event_ms(torch, fn, K, prewarm_s=0.3):
    """Mean ms of fn over K back-to-back calls between HIP events (after a
    short clock warm-up)."""
    fn()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + prewarm_s
    while time.perf_counter() < t_end:
        fn()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / K


def library_attention(w, torch, K, core_ms):
    """PyTorch's own fused attention on the same shape, for comparison:
    scaled_dot_product_attention restricted to its FLASH_ATTENTION backend
    (AOTriton on ROCm), bf16 Q, K, V of [B, H, S, D] drawn at random, no RoPE
    (the library has none), non-causal, scale 1/sqrt(D).  Timing only; bf16
    workloads up to 20000 tokens (the library call takes seconds beyond)."""
    if w.dtype != "bf16" or w.S > 20000:
        return None
    try:
        import torch.nn.functional as F
        from torch.nn.attention import SDPBackend, sdpa_kernel
        g = torch.Generator(device="cuda").manual_seed(0)
        q, k, v = (torch.randn((w.B, w.H, w.S, w.D), device="cuda", dtype=torch.bfloat16, generator=g)
                   for _ in range(3))
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            ms = _event_ms(torch, lambda: F.scaled_dot_product_attention(q, k, v, scale=1.0 / math.sqrt(w.D)), K)
        del q, k, v
    except Exception as ex:  # a library without this backend: report, do not fail the bench
        return {"error": f"{type(ex).__name__}: {str(ex)[:200]}"}
    tf = w.flops / (ms * 1e-3) / 1e12
    return {"what": "torch.nn.functional.scaled_dot_product_attention, FLASH_ATTENTION backend, same B/H/S/D in "
                    "bf16, no RoPE, timing only",
            "torch": torch.__version__, "ms": ms, "TFLOPs": tf, "frac": tf / BF16_PEAK_TFLOPS,
            "attn_core_speedup": ms / core_ms}


def library_gemm(lw, torch, K, ac, wc, gemm_ms):
    """The library's MXFP4 GEMM on the same shape, for comparison: torch._scaled_mm
    on the same E2M1 codes viewed as float4_e2m1fn_x2 with E8M0 scales of
    [rows, K/32] (hipBLASLt on ROCm), bf16 output.  Timing only (the scales are
    all 2^0: their layout is the library's, not this one's)."""
    try:
        a4 = ac.view(torch.float4_e2m1fn_x2)
        w4 = wc.view(torch.float4_e2m1fn_x2)
        sa = torch.full((lw.M, lw.K // 32), 127, dtype=torch.uint8, device="cuda").view(torch.float8_e8m0fnu)
        sw = torch.full((lw.N, lw.K // 32), 127, dtype=torch.uint8, device="cuda").view(torch.float8_e8m0fnu)
        ms = _event_ms(torch, lambda: torch._scaled_mm(a4, w4.t(), sa, sw, out_dtype=torch.bfloat16), K)
    except Exception as ex:
        return {"error": f"{type(ex).__name__}: {str(ex)[:200]}"}
    tf = lw.flops / (ms * 1e-3) / 1e12
    return {"what": "torch._scaled_mm on MXFP4 operands (float4_e2m1fn_x2 codes, e8m0 scales per 1x32), same "
                    "M/N/K, bf16 out, timing only", "torch": torch.__version__, "ms": ms, "TFLOPs": tf,
            "frac": tf / FP4_PEAK_TFLOPS, "gemm_speedup": ms / gemm_ms}


def other_configs(headline, args, torch, dj):
    """Every other attention workload timed the same way in the same run (at
    least 10 steps for the long video share): step and kernel time, TFLOP/s and
    the fraction of the dense MFMA peak of the workload's dtype."""
    res = {}
    for name, w in W.WORKLOADS.items():
        if name == headline.name:
            continue
        print(f"[bench] also timing {name}", file=sys.stderr, flush=True)
        run = AttentionRun(w, torch, dj)
        K = max(10, args.steps // 5) if w.S > 50000 else args.steps
        t = run.time_steps(K, args.warmup, args.prewarm_s)
        run.release()
        res[name] = {"B": w.B, "H": w.H, "S": w.S, "dtype": w.dtype, "steps": K,
                     "step_ms": t["step_ms"], "step_median_ms": t["step_median_ms"], "prepare_kv_ms": t["prep_ms"],
                     "kernel_ms": t["core_ms"], "value": w.flops / (t["step_ms"] * 1e-3) / 1e12,
                     "kernel_TFLOPs": w.flops / (t["core_ms"] * 1e-3) / 1e12,
                     "pct_of_peak": 100.0 * w.flops / (t["step_ms"] * 1e-3) / 1e12 / run.peak,
                     "kernel_frac": w.flops / (t["core_ms"] * 1e-3) / 1e12 / run.peak, "peak": run.peak}
    return res


if __name__ == "__main__":
    main()
