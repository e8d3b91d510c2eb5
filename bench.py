#!/usr/bin/env python3
"""Throughput of the routed MoE expert step (permute + grouped SwiGLU expert + unpermute) on one MI355X.

Metric: useful TFLOP/s = 6 * sum_e M_e * d * h / t, where t is the wall time of
one whole step (moe_permute, grouped_swiglu_expert, moe_unpermute) on one
stream with inputs resident in HBM; also reported as a share of the dense bf16
MFMA peak. The useful-FLOP convention (two FLOPs per multiply-add, three
projections of d x h per gated expert, nothing for the activation, routing or
permutations) is the grouped-expert essay's; the timing protocol (warm-up
steps, then a fixed number of queued steps) follows the OLMo report's Fig 38.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config zipf64]
Prints one JSON line. Extra measurements ride along in the same line:
per-stage times, the padded-BMM and per-expert-loop variants (vendor BLAS
through torch, same inputs), the roofline of the dominant kernel and the CPU
oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "useful TFLOP/s (6·ΣM_e·d·h) grouped SwiGLU expert fwd; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
GEMM_SRC = os.path.join(ROOT, "ragged_grouped_gemm_histogram_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_up_swiglu_zipf64_traffic.json")


def roofline_attainable(intensity: float, bandwidth: float, peak: float) -> float:
    """Attainable throughput = min(peak, intensity * bandwidth) (the essay's roofline lab)."""
    return min(peak, intensity * bandwidth)


def useful_flops(M: int, d: int, h: int) -> int:
    return 6 * M * d * h


def algorithmic_bytes(T, k, M, d, h, nonempty, fused=True):
    """Bytes each stage must move at minimum (bf16 = 2 B, int32/fp32 = 4 B); see the design doc.

    fused: the permute writes index maps only and the gate/up GEMM reads each token row of X once at minimum;
    otherwise the permute also copies rows into x_perm, which the GEMM reads back.
    """
    S = T * k
    permute = 4 * S * 3 + (0 if fused else 2 * T * d + 2 * M * d)  # ids + perm + inv (+ read X, write x_perm)
    gemm1 = (2 * T * d if fused else 2 * M * d) + nonempty * 2 * (2 * h) * d + 2 * M * h
    gemm2 = 2 * M * h + nonempty * 2 * h * d + 2 * M * d
    unpermute = 2 * M * d + 8 * S + 2 * T * d
    return {"permute": permute, "gemm_up_swiglu": gemm1, "gemm_down": gemm2, "unpermute": unpermute}


def file_sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def cpu_baseline(wl, tokens: int):
    """Time the oracle (as it stands) on the first `tokens` tokens of the workload."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # threadpoolctl missing: report the process affinity
        threads = len(os.sched_getaffinity(0))
    sl = slice(0, tokens)
    t0 = time.perf_counter()
    r = oracle.moe_expert_forward(wl.x[sl], wl.expert_ids[sl], wl.routing_w[sl], wl.w_ug, wl.w_down)
    dt = time.perf_counter() - t0
    M = int(r.offsets[-1])
    return {"value": useful_flops(M, wl.d, wl.h) / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": dt,
            "sample": f"first {tokens} of {wl.T} tokens of {wl.name} ({M} routed rows, all {wl.E} experts' weights), "
                      f"float64 oracle, 1 run", "host_cpus": len(os.sched_getaffinity(0)),
            "numpy": np.__version__}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="zipf64", choices=["toy", "edge", "qwen3_30b", "zipf64", "square"])
    ap.add_argument("--no-variants", action="store_true", help="skip the padded-BMM and per-expert-loop variants")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="tokens in the oracle sample (0: all T tokens)")
    ap.add_argument("--unfused", action="store_true",
                    help="copy rows into x_perm in moe_permute instead of gathering them inside the gate/up GEMM")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain device copy of known size (HBM counter calibration)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}, WORLD_SIZE={world}): the expert step here "
              "has no collectives; an expert-parallel layer would run this same step per GPU on its own experts.",
              file=sys.stderr)
        return 2

    import torch

    import ragged_grouped_gemm_histogram_amd as moe
    from workloads import WORKLOADS, make_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = make_workload(args.config)
    T, k, E, d, h = wl.T, wl.k, wl.E, wl.d, wl.h
    S = T * k

    def bf(a):
        import numpy as np

        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    x, w_ug, w_down = bf(wl.x), bf(wl.w_ug), bf(wl.w_down)
    ids = torch.from_numpy(wl.expert_ids).to(dev)
    rw = torch.from_numpy(wl.routing_w).to(dev)
    fused = not args.unfused
    x_perm = None if fused else torch.empty((S, d), dtype=torch.bfloat16, device=dev)
    h_buf = torch.empty((S, h), dtype=torch.bfloat16, device=dev)
    y_perm = torch.empty((S, d), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    perm = torch.empty((S,), dtype=torch.int32, device=dev)
    inv = torch.empty((T, k), dtype=torch.int32, device=dev)
    ws = torch.empty((max(moe.permute_workspace_bytes(T, k, E), 4),), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        p = moe.moe_permute(x, ids, E, x_perm=x_perm, counts=counts, offsets=offsets, perm=perm, inv_map=inv,
                            workspace=ws, gather=not fused)
        if ev is not None:
            ev[1].record()
        if fused:
            moe.moe_gemm_up_swiglu_gather(x, p.perm, p.offsets, w_ug, k, h_buf=h_buf)
        else:
            moe.moe_gemm_up_swiglu(p.x_perm, p.offsets, w_ug, h_buf=h_buf)
        if ev is not None:
            ev[2].record()
        moe.moe_gemm_down(h_buf, p.offsets, w_down, y_perm=y_perm)
        if ev is not None:
            ev[3].record()
        moe.moe_unpermute(y_perm, p.inv_map, rw, y=y)
        if ev is not None:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: exactly K steps, events bracket every stage on the launch stream.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    M = int(offsets[-1].item())
    nonempty = int((counts > 0).sum().item())
    ms_per_step = elapsed * 1e3 / args.steps
    flops = useful_flops(M, d, h)
    value = flops / (ms_per_step * 1e-3) / 1e12
    names = ["permute", "gemm_up_swiglu", "gemm_down", "unpermute"]
    stage_ms = {n: sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / args.steps for j, n in enumerate(names)}
    algo = algorithmic_bytes(T, k, M, d, h, nonempty, fused)
    gemm1_flops = 2 * M * d * (2 * h)
    gemm2_flops = 2 * M * h * d
    stages = {
        "permute": {"ms": stage_ms["permute"], "GB/s": algo["permute"] / stage_ms["permute"] / 1e6},
        "gemm_up_swiglu": {"ms": stage_ms["gemm_up_swiglu"],
                           "TFLOP/s": gemm1_flops / stage_ms["gemm_up_swiglu"] / 1e9},
        "gemm_down": {"ms": stage_ms["gemm_down"], "TFLOP/s": gemm2_flops / stage_ms["gemm_down"] / 1e9},
        "unpermute": {"ms": stage_ms["unpermute"], "GB/s": algo["unpermute"] / stage_ms["unpermute"] / 1e6},
    }

    # Roofline of the dominant kernel: the gate/up projection with fused SwiGLU (two thirds of the FLOPs).
    g1_ms = stage_ms["gemm_up_swiglu"]
    achieved = gemm1_flops / (g1_ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if (tr.get("gemm_src_sha") == file_sha(GEMM_SRC) and tr.get("workload") == wl.name
                and tr.get("fused_gather", False) == fused):
            traffic = tr.get("bytes_per_launch")
    roofline = {"bound": "mfma", "kernel": "grouped_gemm_pipe_kernel<gate/up + SwiGLU" + (", fused gather>" if fused else ">"),
                "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": traffic, "algorithmic_bytes": algo["gemm_up_swiglu"], "flops_per_launch": gemm1_flops,
                "avg_launch_ms": g1_ms}

    variants = None
    if not args.no_variants:
        xp = x_perm if x_perm is not None else torch.empty((S, d), dtype=torch.bfloat16, device=dev)
        variants = run_variants(torch, moe, x, ids, rw, w_ug, w_down, wl, counts, offsets, xp, inv, y_perm, ws,
                                steps=max(3, min(args.steps, 10)))

    if args.calib_copy:
        src = torch.full((256 << 20,), 7, dtype=torch.uint8, device=dev)  # written first: a real read stream
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        tokens = args.cpu_tokens or T
        cpu = cpu_baseline(wl, min(tokens, T))

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "k": k, "E": E, "d": d, "h": h, "M": M, "nonempty_experts": nonempty,
                   "seed": WORKLOADS[wl.name][0], "parallelism": "single GPU",
                   "gather": "fused into the gate/up GEMM" if fused else "x_perm copy in moe_permute"},
        "pct_of_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "useful_gflop": flops / 1e9,
        "stages": stages,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "variants": variants,
    }
    print(json.dumps(out))
    return 0


def run_variants(torch, moe, x, ids, rw, w_ug, w_down, wl, counts, offsets, x_perm, inv, y_perm, ws, steps):
    """Padded BMM at capacity factor 1.25 and the per-expert launch loop (vendor BLAS through torch)."""
    import torch.nn.functional as F

    T, k, E, d, h = wl.T, wl.k, wl.E, wl.d, wl.h
    dev = x.device
    M = int(offsets[-1].item())
    C = math.ceil(1.25 * M / E)
    cnt = counts.cpu().tolist()
    kept_rows = sum(min(c, C) for c in cnt)
    # torch.bmm wants the right operand materialised: convert the weight layout once, before timing.
    w_ug_t = w_ug.transpose(1, 2).contiguous()  # [E, d, 2h]
    flat_ids = ids.reshape(-1).long()
    valid = (flat_ids >= 0) & (flat_ids < E)

    def bmm_step():
        # dispatch: stable order by expert, rank inside the expert, keep ranks < C
        key = torch.where(valid, flat_ids, torch.full_like(flat_ids, E))
        order = torch.sort(key, stable=True).indices
        sorted_key = key[order]
        starts = torch.searchsorted(sorted_key, torch.arange(E + 1, device=dev))
        rank = torch.arange(order.numel(), device=dev) - starts[sorted_key.clamp(max=E)]
        keep = (sorted_key < E) & (rank < C)
        slot = order[keep]
        e_of = sorted_key[keep]
        r_of = rank[keep]
        padded = torch.zeros((E, C, d), dtype=torch.bfloat16, device=dev)
        padded[e_of, r_of] = x[slot // k]
        u = torch.bmm(padded, w_ug_t)  # [E, C, 2h]
        hh = F.silu(u[..., :h]) * u[..., h:]
        out = torch.bmm(hh.contiguous(), w_down)  # [E, C, d]
        yy = torch.zeros((T * k, d), dtype=torch.float32, device=dev)
        yy[slot] = out[e_of, r_of].float() * rw.reshape(-1)[slot, None]
        return yy.view(T, k, d).sum(1).to(torch.bfloat16)

    def loop_step():
        p = moe.moe_permute(x, ids, E, x_perm=x_perm, counts=counts, offsets=offsets, inv_map=inv, workspace=ws)
        offs = p.offsets.cpu().tolist()  # the host needs the counts: device-to-host wait
        for e in range(E):
            lo, hi = offs[e], offs[e + 1]
            if hi == lo:
                continue
            u = F.linear(p.x_perm[lo:hi], w_ug[e])
            y_perm[lo:hi] = (F.silu(u[:, :h]) * u[:, h:]) @ w_down[e]
        return moe.moe_unpermute(y_perm, p.inv_map, rw)

    res = {}
    for name, fn in (("padded_bmm_c1.25", bmm_step), ("per_expert_loop", loop_step)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        useful = useful_flops(kept_rows if name.startswith("padded") else M, d, h)
        entry = {"ms_per_step": ms, "useful_TFLOP/s": useful / (ms * 1e-3) / 1e12, "timing": "host wall clock, synced"}
        if name.startswith("padded"):
            entry.update({"capacity_C": C, "rows_executed": E * C, "rows_dropped": M - kept_rows,
                          "padding_fraction_executed": 1 - kept_rows / (E * C)})
        res[name] = entry
    return res


if __name__ == "__main__":
    sys.exit(main())
