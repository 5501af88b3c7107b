#!/usr/bin/env python3
"""Benchmark of the fused MoE grouped GEMM layer on one MI355X.

One step = the whole hot path on one batch: build the routing schedule on the
device, the fused forward (gather on load, weighted atomic scatter-combine),
and the fused backward (dX with the routing-weight gradient, and dW).

Workload of the headline line (seeded, synthetic, resident in HBM before
timing): T=4096 tokens, K=N=2048, E=8 experts, top-2 routing drawn uniformly,
routing weights U[0,1), x, dY ~ N(0,1), W ~ N(0,1/K), bf16 storage with fp32
accumulation.

Metric: useful TFLOP/s = (2SKN forward + 4SKN backward + 2SN routing-weight
gradient) / step time, S = T*top_k; padding is never counted.  The roofline
object is the dominant kernel's useful TFLOP/s (from HIP events on the
kernels' own stream) against the bf16 matrix-core peak, with its measured HBM
bytes per launch (profiles/traffic_counters.json) while the kernel sources
match the counters.

More objects ride on the same line: "config3" (Zipf-skewed T=8192 K=4096
N=1408 E=64 top-4 step, with its own roofline), "config4" (the weight
gradient alone on S=65536 Dirichlet-sized groups, against the larger of its
matrix-core and HBM bounds), "decode" (masked decode forward, HBM GB/s),
"fp8" (the 8-bit forwards on the headline shape and on the masked decode),
"gated_ffn" (gated expert FFN forward and backward on the balanced step of the
page's worked example) and "cpu_baseline" (the float64 oracle on the host's
cores, a bounded number of steps).

--only LINE runs one of the extra lines by itself (for profiling one
workload's kernels).  Prints ONE JSON line.  --gpus above 1 is not supported
(this path runs on one GPU) and exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("useful TFLOP/s (2·S·K·N) + % bf16 MFMA peak, fused MoE fwd/bwd; "
          "decode HBM GB/s")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA (published)


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=400,
                   help="untimed steps first (also brings the GPU clocks to their loaded state)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-config3", action="store_true", help="skip the Zipf-skewed fwd+bwd line")
    p.add_argument("--no-config4", action="store_true", help="skip the dW stress line")
    p.add_argument("--no-fp8", action="store_true", help="skip the 8-bit forward lines")
    p.add_argument("--no-gated", action="store_true",
                   help="skip the gated expert FFN line (its inputs take ~10 s to draw)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum host time spent on the oracle sample")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 256 MiB device copy (calibrates HBM byte counters)")
    p.add_argument("--only", choices=("config3", "config4", "decode", "fp8", "gated"),
                   help="run only this line, with --steps / --warmup as given (for profiling "
                        "one workload's kernels); prints {\"only\": name, name: object}")
    return p.parse_args()


def _calib_copy(torch, dev) -> None:
    """A plain device copy of known size (256 MiB) for the HBM byte counters."""
    src = torch.empty(64 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_baseline(r, flops_step: float, min_seconds: float) -> dict:
    """The CPU oracle, untuned, on the host cores: one full step (forward and
    backward) of the same workload."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max((d.get("num_threads", 1) for d in info), default=1)
        blas = ",".join(sorted({f"{d.get('internal_api')} {d.get('version')}" for d in info}))
    except Exception:  # pragma: no cover
        threads, blas = os.cpu_count() or 1, "unknown"
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.moe_forward(r.x.values, r.W.values, r.expert_ids, r.topk_weights, r.E)
        O.moe_backward(r.dY.values, r.x.values, r.W.values, r.expert_ids, r.topk_weights, r.E)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(reps * flops_step / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} full steps (forward + backward, float64) of the same workload",
            "seconds": round(dt, 3), "host_cpu": platform.processor() or platform.machine(),
            "blas": blas}


def _traffic(kernel_family: str, workload: str = "config2"):
    """HBM bytes per launch of a kernel family on a workload from the committed
    counter summary (FETCH_SIZE and WRITE_SIZE runs, scaled by a plain copy's
    reading), or None when there is none or the kernels changed since it was
    taken."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    from moe_variable_size_amd.counters import source_digest
    if rec.get("source_sha256") != source_digest():
        return None
    k = rec.get("workloads", {}).get(workload, {}).get("kernels", {}).get(kernel_family)
    return None if k is None else k.get("hbm_bytes_per_launch")


def _timed_steps(torch, api, step, steps: int, warmup: int, families) -> tuple:
    """Wall time per step over `steps` steps after `warmup`, then the library's
    per-launch HIP-event durations (us) of each kernel family over as many
    steps again."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    api.moe_timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    api.moe_timing_enable(False)
    kt = {}
    for f in families:
        tot, n = api.moe_timing_read(f)
        kt[f] = round(tot * 1e3 / max(n, 1), 3) if n else None
    return ms_step, kt


def useful_rows(counts) -> dict:
    """Fraction of the computed tile rows that are real rows, per tile height
    ("Grouped GEMM for MoE, in depth" -- "Worked example: tile counts under
    skew")."""
    c = np.asarray(counts, dtype=np.int64)
    out = {}
    for bm in (64, 128, 256):
        blocks = int((-(-c // bm)).sum())
        out[f"bm{bm}"] = round(float(c.sum()) / (blocks * bm), 4) if blocks else None
    return out


def config3_line(torch, api, WL, dev, steps: int, warmup: int) -> dict:
    """Zipf-skewed fused layer, forward + backward (T=8192, E=64, top-4,
    K=4096, N=1408; 4 empty experts): useful TFLOP/s of each grouped kernel
    against the bf16 matrix-core peak."""
    r = WL.config3()
    T, K, N, E, k = r.T, r.K, r.N, r.E, r.k
    S = T * k

    def to_dev(t):
        return torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x, W, dY = to_dev(r.x), to_dev(r.W), to_dev(r.dY)
    ids = torch.from_numpy(r.expert_ids).to(dev)
    w = torch.from_numpy(r.topk_weights).to(dev)
    ws = torch.empty(api.moe_schedule_workspace_bytes(T, k, E), dtype=torch.uint8, device=dev)
    y = torch.empty((T, N), dtype=torch.float32, device=dev)
    dX = torch.empty((T, K), dtype=torch.float32, device=dev)
    dW = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
    dT = torch.empty((T, k), dtype=torch.float32, device=dev)

    def step():
        sch = api.moe_build_schedule(ids, w, E, workspace=ws)
        api.moe_fused_fwd(x, W, sch, y=y)
        api.moe_fused_bwd(dY, x, W, sch, out_dX=dX, out_dW=dW, out_dtopk=dT)

    ms_step, kt = _timed_steps(torch, api, step, steps, warmup,
                               ("build_schedule", "fill_zero", "fused_fwd", "bwd_dx", "bwd_dw"))
    gemm = 2.0 * S * K * N
    tf = {f: round((gemm + (2.0 * S * N if f == "bwd_dx" else 0.0)) / (kt[f] * 1e-6) / 1e12, 2)
          for f in ("fused_fwd", "bwd_dx", "bwd_dw")}
    step_tf = (3 * gemm + 2.0 * S * N) / (ms_step * 1e-3) / 1e12
    dom = max(("fused_fwd", "bwd_dx", "bwd_dw"), key=lambda f: kt[f])
    counts = np.bincount(r.expert_ids.ravel(), minlength=E)
    del x, W, dY, dX, dW, y
    return {"workload": f"{r.name} fwd+bwd step (schedule + fused fwd + dX/d_topk + dW)",
            "T": T, "K": K, "N": N, "E": E, "top_k": k, "S": S,
            "max_expert_rows": int(counts.max()), "empty_experts": int((counts == 0).sum()),
            "step_ms": round(ms_step, 4), "tflops": round(step_tf, 2),
            "pct_bf16_peak": round(100.0 * step_tf / PEAK_BF16_TFLOPS, 2),
            "kernels_us": kt, "kernels_tflops": tf,
            "schedule_share": round(kt["build_schedule"] * 1e-3 / ms_step, 4),
            "useful_rows": useful_rows(counts),
            "roofline": {"bound": "mfma", "kernel": dom, "achieved": tf[dom],
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf[dom] / PEAK_BF16_TFLOPS, 4),
                         "traffic": _traffic(dom, "config3")}}


def config4_line(torch, api, WL, dev, steps: int, warmup: int) -> dict:
    """Weight-gradient stress (E=128, K=2048, N=768, 65536 grouped rows,
    Dirichlet(0.3) group sizes): dW = per-group dY^T X, useful TFLOP/s and
    HBM GB/s of the algorithmic bytes (X, dY read once, dW written once)
    against both rooflines."""
    g = WL.config4()
    r = WL.grouped_as_routed(g)

    def to_dev(t):
        return torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16).to(dev)

    X, dY = to_dev(r.x), to_dev(r.dY)
    ids = torch.from_numpy(r.expert_ids).to(dev)
    ws = torch.empty(api.moe_schedule_workspace_bytes(r.T, 1, g.E), dtype=torch.uint8, device=dev)
    dW = torch.empty((g.E, g.N, g.K), dtype=torch.bfloat16, device=dev)

    def step():
        sch = api.moe_build_schedule(ids, None, g.E, workspace=ws)
        api.moe_fused_bwd(dY, X, None, sch, dx=False, dtopk=False, N=g.N, out_dW=dW)

    ms_step, kt = _timed_steps(torch, api, step, steps, warmup, ("build_schedule", "bwd_dw"))
    flops = 2.0 * g.M * g.K * g.N
    nbytes = g.M * g.K * 2 + g.M * g.N * 2 + g.E * g.N * g.K * 2
    us = kt["bwd_dw"]
    tf = flops / (us * 1e-6) / 1e12
    gbs = nbytes / (us * 1e-6) / 1e9
    bound_us = max(flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)) * 1e6
    sizes = np.asarray(g.group_sizes)
    del X, dY, dW
    return {"workload": f"{g.name} weight gradient (schedule + dW)",
            "S": g.M, "K": g.K, "N": g.N, "E": g.E, "seed": g.seed,
            "max_group_rows": int(sizes.max()), "empty_groups": int((sizes == 0).sum()),
            "groups_over_4096": int((sizes > 4096).sum()),
            "step_ms": round(ms_step, 4), "kernels_us": kt,
            "dw_tflops": round(tf, 2), "dw_hbm_GBps": round(gbs, 1), "bytes_per_launch": nbytes,
            "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "roofline": {"bound": "hbm" if nbytes / (PEAK_HBM_GBS * 1e9) > flops / (PEAK_BF16_TFLOPS * 1e12)
                         else "mfma", "bound_us": round(bound_us, 2),
                         "frac": round(bound_us / us, 4),
                         "traffic": _traffic("bwd_dw_unweighted", "config4")},
            "schedule_share": round(kt["build_schedule"] * 1e-3 / ms_step, 4)}


def decode_line(torch, api, WL, dev, steps: int, warmup: int) -> dict:
    """Masked fixed-capacity decode (E=64, capacity 64, T=128 top-8, K=7168,
    N=2048): the forward streams every active expert's weights once.  Reported
    as HBM GB/s of the algorithmic bytes (weights of active experts + x + y)."""
    r = WL.config5()
    T, K, N, E, k, cap = r.T, r.K, r.N, r.E, r.k, r.capacity

    def to_dev(t):
        return torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x, W = to_dev(r.x), to_dev(r.W)
    ids = torch.from_numpy(r.expert_ids).to(dev)
    w = torch.from_numpy(r.topk_weights).to(dev)
    lay = api.MOE_LAYOUT_MASKED
    ws = torch.empty(api.moe_schedule_workspace_bytes(T, k, E, lay, cap), dtype=torch.uint8,
                     device=dev)
    y = torch.empty((T, N), dtype=torch.float32, device=dev)

    def step():
        sch = api.moe_build_schedule(ids, w, E, layout=lay, capacity=cap, workspace=ws)
        api.moe_fused_fwd(x, W, sch, y=y)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    api.moe_timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    api.moe_timing_enable(False)
    tot, n = api.moe_timing_read("fused_fwd")
    fwd_us = tot * 1e3 / max(n, 1)
    active = int(np.count_nonzero(np.bincount(r.expert_ids.ravel(), minlength=E)))
    nbytes = active * N * K * 2 + T * K * 2 + T * N * 4
    gbs = nbytes / (fwd_us * 1e-6) / 1e9
    return {"workload": f"{r.name} forward (masked layout)", "active_experts": active,
            "bytes_per_launch": nbytes, "fwd_us": round(fwd_us, 3),
            "hbm_GBps": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "step_ms": round(ms_step, 4),
            "step_GBps": round(nbytes / (ms_step * 1e-3) / 1e9, 1)}


def gated_line(torch, api, WL, dev, steps: int, warmup: int) -> dict:
    """Gated expert FFN forward and backward on the balanced step of the page's
    worked example (T=8192, hidden 4096, F=2048, E=64 with 256 rows each,
    top-2): gate+up as one grouped GEMM with silu(gate)*up in its epilogue,
    the down projection with the weighted scatter-combine, and the backward
    (dW_down, dh/dgu/d routing weight, dX, dW_gu).  Useful FLOPs: forward
    2*S*K*2F + 2*S*F*N, backward twice that.  Kernel times per launch (the
    backward's two dX-kernel launches and two dW launches average together)."""
    g = WL.gated_page_example()

    def to_dev(t):
        return torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x, Wgu, Wd = to_dev(g.x), to_dev(g.W_gu), to_dev(g.W_down)
    ids = torch.from_numpy(g.expert_ids).to(dev)
    w = torch.from_numpy(g.topk_weights).to(dev)
    S = g.T * g.k
    ws = torch.empty(api.moe_schedule_workspace_bytes(g.T, g.k, g.E), dtype=torch.uint8, device=dev)
    h = torch.empty((S, g.F), dtype=torch.bfloat16, device=dev)
    y = torch.empty((g.T, g.N), dtype=torch.float32, device=dev)

    gu = torch.empty((S, 2 * g.F), dtype=torch.float32, device=dev)
    rng = np.random.default_rng(g.seed + 1)
    dY = torch.from_numpy(rng.standard_normal((g.T, g.N), dtype=np.float32)).to(torch.bfloat16).to(dev)

    def step():
        sch = api.moe_build_schedule(ids, w, g.E, workspace=ws)
        api.moe_gated_ffn_fwd(x, Wgu, Wd, sch, h=h, y=y, gu=gu)
        api.moe_gated_ffn_bwd(dY, x, Wgu, Wd, sch, gu, h)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    api.moe_timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    api.moe_timing_enable(False)
    kt = {}
    for f in ("build_schedule", "gated_up", "fill_zero", "gated_down", "gated_bwd_dw_down",
              "gated_bwd_dh", "gated_bwd_dx", "gated_bwd_dw_gu"):
        tot, n = api.moe_timing_read(f)
        kt[f] = round(tot * 1e3 / max(n, 1), 3)
    fl_up = 2.0 * S * g.K * 2 * g.F
    fl_dn = 2.0 * S * g.F * g.N
    # backward: dh and dW_down (2 S N F each), dX and dW_gu (2 S 2F K each)
    fl_bwd = 2 * fl_dn + 2 * fl_up
    up_tf = fl_up / (kt["gated_up"] * 1e-6) / 1e12
    del x, Wgu, Wd, h, y, gu, dY
    return {"workload": f"{g.name} forward + backward (schedule, gated up saving gate/up, zero y, "
                        "down; dW_down, dh/dgu/d_topk, dX, dW_gu)",
            "T": g.T, "K": g.K, "F": g.F, "N": g.N, "E": g.E, "top_k": g.k,
            "step_ms": round(ms_step, 4),
            "tflops": round((fl_up + fl_dn + fl_bwd) / (ms_step * 1e-3) / 1e12, 2),
            "kernels_us": kt,
            "gated_up_tflops": round(up_tf, 2),
            "gated_down_tflops": round(fl_dn / (kt["gated_down"] * 1e-6) / 1e12, 2),
            "roofline": {"bound": "mfma", "kernel": "gated_up", "achieved": round(up_tf, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(up_tf / PEAK_BF16_TFLOPS, 4)}}


def fp8_line(torch, api, WL, dev, steps: int, warmup: int) -> dict:
    """8-bit (E4M3) forward with per-token and per-expert-channel scales on the
    config-2 shape (useful TFLOP/s against the 8-bit dense peak) and on the
    config-5 masked decode (HBM GB/s of the algorithmic bytes: 1-byte weights
    of the active experts + x codes + y)."""
    out = {}
    for name, r, lay in (("fwd", WL.config2(with_dy=False), api.MOE_LAYOUT_CONTIGUOUS),
                         ("decode", WL.config5(), api.MOE_LAYOUT_MASKED)):
        f = WL.fp8_routed(r)

        def u8(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        xq, sx, Wq, sw = u8(f.xq), u8(f.x_scale), u8(f.Wq), u8(f.w_scale)
        ids, w = u8(f.expert_ids), u8(f.topk_weights)
        ws = torch.empty(api.moe_schedule_workspace_bytes(f.T, f.k, f.E, lay, r.capacity),
                         dtype=torch.uint8, device=dev)
        y = torch.empty((f.T, f.N), dtype=torch.float32, device=dev)

        def step():
            sch = api.moe_build_schedule(ids, w, f.E, layout=lay, capacity=r.capacity, workspace=ws)
            api.moe_fused_fwd_fp8(xq, sx, Wq, sw, sch, y=y)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / steps
        api.moe_timing_enable(True)
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        api.moe_timing_enable(False)
        tot, n = api.moe_timing_read("fused_fwd_fp8")
        us = tot * 1e3 / max(n, 1)
        S = f.T * f.k
        if name == "fwd":
            tf = 2.0 * S * f.K * f.N / (us * 1e-6) / 1e12
            out[name] = {"workload": f"{f.name} forward (schedule + zero y + fp8 forward)",
                         "fwd_us": round(us, 3), "tflops": round(tf, 2),
                         "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                         "step_ms": round(ms_step, 4)}
        else:
            active = int(np.count_nonzero(np.bincount(f.expert_ids.ravel(), minlength=f.E)))
            nbytes = active * f.N * f.K + f.T * f.K + f.T * f.N * 4
            gbs = nbytes / (us * 1e-6) / 1e9
            out[name] = {"workload": f"{f.name} forward (masked layout)",
                         "bytes_per_launch": nbytes, "fwd_us": round(us, 3),
                         "hbm_GBps": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                         "step_ms": round(ms_step, 4)}
        del xq, Wq, y
    # per-32-element block scales (E8M0), same shapes
    for name, r, lay in (("fwd_mx", WL.config2(with_dy=False), api.MOE_LAYOUT_CONTIGUOUS),
                         ("decode_mx", WL.config5(), api.MOE_LAYOUT_MASKED)):
        f = WL.mx_routed(r)

        def u8(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        xq, xs, Wq, wsc = u8(f.xq), u8(f.x_bs), u8(f.Wq), u8(f.w_bs)
        ids, w = u8(f.expert_ids), u8(f.topk_weights)
        ws = torch.empty(api.moe_schedule_workspace_bytes(f.T, f.k, f.E, lay, r.capacity),
                         dtype=torch.uint8, device=dev)
        y = torch.empty((f.T, f.N), dtype=torch.float32, device=dev)

        def step_mx():
            sch = api.moe_build_schedule(ids, w, f.E, layout=lay, capacity=r.capacity, workspace=ws)
            api.moe_fused_fwd_mx(xq, xs, Wq, wsc, sch, y=y)

        for _ in range(warmup):
            step_mx()
        torch.cuda.synchronize()
        api.moe_timing_enable(True)
        for _ in range(steps):
            step_mx()
        torch.cuda.synchronize()
        api.moe_timing_enable(False)
        tot, n = api.moe_timing_read("fused_fwd_mx")
        us = tot * 1e3 / max(n, 1)
        S = f.T * f.k
        if name == "fwd_mx":
            tf = 2.0 * S * f.K * f.N / (us * 1e-6) / 1e12
            out[name] = {"workload": f"{f.name} forward (block scales per 32 elements)",
                         "fwd_us": round(us, 3), "tflops": round(tf, 2),
                         "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)}
        else:
            active = int(np.count_nonzero(np.bincount(f.expert_ids.ravel(), minlength=f.E)))
            nbytes = active * f.N * (f.K + f.K // 32) + f.T * (f.K + f.K // 32) + f.T * f.N * 4
            gbs = nbytes / (us * 1e-6) / 1e9
            out[name] = {"workload": f"{f.name} forward (masked layout, block scales)",
                         "bytes_per_launch": nbytes, "fwd_us": round(us, 3),
                         "hbm_GBps": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        del xq, Wq, y
    return out


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {a.gpus} is not supported (the library "
              "runs the single-GPU path; expert shards across GPUs are not built)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from moe_variable_size_amd import api
    from moe_variable_size_amd import workloads as WL

    dev = torch.device("cuda:0")
    if a.only:
        lines = {"config3": config3_line, "config4": config4_line, "decode": decode_line,
                 "fp8": fp8_line, "gated": gated_line}
        obj = lines[a.only](torch, api, WL, dev, a.steps, a.warmup)
        if a.calib_copy:
            _calib_copy(torch, dev)
        print(json.dumps({"only": a.only, a.only: obj}), flush=True)
        return

    r = WL.config2()
    T, K, N, E, k = r.T, r.K, r.N, r.E, r.k
    S = T * k

    def to_dev(t):
        return torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x, W, dY = to_dev(r.x), to_dev(r.W), to_dev(r.dY)
    ids = torch.from_numpy(r.expert_ids).to(dev)
    w = torch.from_numpy(r.topk_weights).to(dev)
    ws = torch.empty(api.moe_schedule_workspace_bytes(T, k, E), dtype=torch.uint8, device=dev)
    y = torch.empty((T, N), dtype=torch.float32, device=dev)
    dX = torch.empty((T, K), dtype=torch.float32, device=dev)
    dW = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
    dT = torch.empty((T, k), dtype=torch.float32, device=dev)

    def step():
        sch = api.moe_build_schedule(ids, w, E, workspace=ws)
        api.moe_fused_fwd(x, W, sch, y=y)
        api.moe_fused_bwd(dY, x, W, sch, out_dX=dX, out_dW=dW, out_dtopk=dT)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps, synchronised on both sides
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / a.steps

    # per-kernel durations: HIP events recorded by the library on each launch's
    # own stream, over a second run of the same steps
    api.moe_timing_enable(True)
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    api.moe_timing_enable(False)
    fams = ["build_schedule", "fill_zero", "fused_fwd", "bwd_dx", "bwd_dw"]
    kt = {}
    for f in fams:
        tot, n = api.moe_timing_read(f)
        kt[f] = {"avg_us": round(tot * 1e3 / max(n, 1), 3), "launches": n}

    if a.calib_copy:
        _calib_copy(torch, dev)

    gemm = 2.0 * S * K * N
    flops_step = 3 * gemm + 2.0 * S * N
    value = flops_step / (ms_step * 1e-3) / 1e12
    # dominant kernel = the grouped GEMM family with the largest time per launch
    dom = max(["fused_fwd", "bwd_dx", "bwd_dw"], key=lambda f: kt[f]["avg_us"])
    dom_flops = gemm + (2.0 * S * N if dom == "bwd_dx" else 0.0)
    achieved = dom_flops / (kt[dom]["avg_us"] * 1e-6) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy PCG64; bf16 storage, fp32 accumulation)",
        "config": {"workload": f"{r.name} fwd+bwd step (schedule + fused fwd + dX/d_topk + dW)",
                   "T": T, "K": K, "N": N, "E": E, "top_k": k, "S": S,
                   "routing": "2 distinct experts per token, uniform; weights U[0,1)"},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "kernels_us": kt,
        "pct_bf16_peak_fwd": round(100.0 * gemm / (kt["fused_fwd"]["avg_us"] * 1e-6) / 1e12
                                   / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(gemm / (kt["fused_fwd"]["avg_us"] * 1e-6) / 1e12, 2),
        "bwd_tflops": round((2 * gemm + 2.0 * S * N)
                            / ((kt["bwd_dx"]["avg_us"] + kt["bwd_dw"]["avg_us"]) * 1e-6) / 1e12, 2),
    }
    tr = _traffic(dom)
    if tr is not None:
        out["roofline"]["traffic"] = tr
    out["schedule_share"] = round(kt["build_schedule"]["avg_us"] * 1e-3 / ms_step, 4)
    out["useful_rows"] = useful_rows(np.bincount(r.expert_ids.ravel(), minlength=E))
    del x, W, dY, y, dX, dW, dT
    if not a.no_config3:
        out["config3"] = config3_line(torch, api, WL, dev, min(a.steps, 50), min(a.warmup, 20))
    if not a.no_config4:
        out["config4"] = config4_line(torch, api, WL, dev, min(a.steps, 100), min(a.warmup, 20))
    if not a.no_decode:
        out["decode"] = decode_line(torch, api, WL, dev, a.steps, a.warmup)
    if not a.no_fp8:
        out["fp8"] = fp8_line(torch, api, WL, dev, min(a.steps, 100), min(a.warmup, 50))
    if not a.no_gated:
        out["gated_ffn"] = gated_line(torch, api, WL, dev, min(a.steps, 50), min(a.warmup, 20))
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(r, flops_step, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
