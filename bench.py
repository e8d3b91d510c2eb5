#!/usr/bin/env python3
"""Throughput of the routed MoE expert step (permute + grouped SwiGLU expert + unpermute) on one MI355X.

Metric: useful TFLOP/s = 6 * sum_e M_e * d * h / t, where t is the wall time of
one whole step (moe_permute, the grouped SwiGLU expert, moe_unpermute) on one
stream with inputs resident in HBM; also reported as a share of the dense bf16
MFMA peak. The useful-FLOP convention (two FLOPs per multiply-add, three
projections of d x h per gated expert, nothing for the activation, routing or
permutations) is the grouped-expert essay's; the timing protocol (warm-up
steps, then a fixed number of queued steps) follows the OLMo report's Fig 38.
The step is timed twice: K eager steps with HIP events around every stage (the
per-stage times and the roofline come from these), then K replays of the same
step captured once in a HIP graph, which is the headline unless --eager.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config zipf64]
Prints one JSON line. Extra measurements ride along in the same line:
per-stage times, the padded-BMM and per-expert-loop variants (vendor BLAS
through torch, same inputs), the roofline of the dominant kernel, the CPU
oracle timed on a bounded sample of the same workload, and the GPU clock and
socket power read during a steady back-to-back loop after the timed region
(the OLMo report ties its largest-shape results to the clock under power limits).
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
    """Bytes each stage must move at minimum (bf16 = 2 B, int32/fp32 = 4 B).

    fused: the permute writes index maps only and the gate/up GEMM reads each token row of X once at minimum;
    otherwise the permute also copies rows into x_perm, which the GEMM reads back.
    """
    S = T * k
    permute = 4 * S * 3 + (0 if fused else 2 * T * d + 2 * M * d)  # ids + perm + inv (+ read X, write x_perm)
    gemm1 = (2 * T * d if fused else 2 * M * d) + nonempty * 2 * (2 * h) * d + 2 * M * h
    gemm2 = 2 * M * h + nonempty * 2 * h * d + 2 * M * d
    unpermute = 2 * M * d + 8 * S + 2 * T * d
    return {"permute": permute, "gemm_up_swiglu": gemm1, "gemm_down": gemm2, "unpermute": unpermute}


def entropy_deficit(counts) -> float:
    """Eq 18 of the OLMo report (Sec 9.6): I_H = 1 - H(p) / log N_local with p_e = M_e / M, 0 log 0 = 0;
    N_local counts every local expert, empty ones included; one expert, or no rows, gives 0."""
    n = len(counts)
    M = sum(int(c) for c in counts)
    if n <= 1 or M == 0:
        return 0.0
    H = -sum((c / M) * math.log(c / M) for c in counts if c > 0)
    return 1.0 - H / math.log(n)


def capacity_eq16(c: float, mbar: float, ranks: int) -> int:
    """Eq 16: C = M_E * 8 * ceil(floor(c * Mbar / M_E) / 8), the eight-row-aligned capacity per EP rank."""
    from fractions import Fraction

    inner = math.floor(Fraction(str(c)) * Fraction(mbar).limit_denominator(1 << 20) / ranks)
    return ranks * 8 * math.ceil(Fraction(inner, 8))


def histogram_stats(counts, tile_rows: int) -> dict:
    """Load statistics of one routing (OLMo report Sec 9.2 and 9.6): I_H (Eq 18); the padded BMM's capacity
    C = ceil(1.25 * M / E) (Fig 35 and the Fig 38 footnote), its padding fraction Eq 14 over the rows it
    executes, E*C, counting only the rows that fit (rows past C are dropped), and the rows it drops; Eq 16's
    capacity at c = 1.25 for one rank (this step runs without expert parallelism); the grouped GEMM's own
    waste, the share of its row-tile slots that hold no row at the tile height it runs."""
    counts = [int(c) for c in counts]
    E, M = len(counts), sum(counts)
    C = math.ceil(1.25 * M / E) if E else 0
    kept = sum(min(c, C) for c in counts)
    slots = sum(-(-c // tile_rows) * tile_rows for c in counts)
    return {"I_H_eq18": entropy_deficit(counts), "M": M, "E": E, "nonempty_experts": sum(c > 0 for c in counts),
            "max_rows": max(counts) if counts else 0, "min_nonempty_rows": min([c for c in counts if c > 0] or [0]),
            "bmm_capacity_C": C, "rho_pad_eq14_at_C": (1 - kept / (E * C)) if E * C else 0.0,
            "rho_pad_eq14_unclipped": (1 - M / (E * C)) if E * C else 0.0, "bmm_rows_dropped": M - kept,
            "capacity_eq16_c1.25_one_rank": capacity_eq16(1.25, M / E, 1) if E else 0,
            "grouped_tile_rows": tile_rows, "grouped_tile_padding": (1 - M / slots) if slots else 0.0}


def gemm_tile_rows(M_cap: int, E: int, N_tiles: int, cus: int = 256, down: bool = False) -> int:
    """Row-tile height the grouped GEMM launch picks (256 when the mean block has >= 384 rows, or for the down
    projection 192 to 256 rows, and its 256-row tiles can occupy every CU, else 128); the rule the library
    applies on the host."""
    tall = M_cap >= 384 * E or (down and 192 * E <= M_cap <= 256 * E)
    return 256 if (tall and (M_cap // 256 + E) * N_tiles >= cus) else 128


class StepRun:
    """Device buffers of one workload and its step: moe_permute (index maps only, or with the x_perm copy),
    the gate/up GEMM with SwiGLU (gathering A rows through perm when fused), the down GEMM, moe_unpermute."""

    def __init__(self, torch, moe, wl, dev, fused: bool):
        import numpy as np

        def bf(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        T, k, E, d, h = wl.T, wl.k, wl.E, wl.d, wl.h
        S = T * k
        self.wl, self.fused, self.moe = wl, fused, moe
        self.x, self.w_ug, self.w_down = bf(wl.x), bf(wl.w_ug), bf(wl.w_down)
        self.ids = torch.from_numpy(wl.expert_ids).to(dev)
        self.rw = torch.from_numpy(wl.routing_w).to(dev)
        self.x_perm = None if fused else torch.empty((S, d), dtype=torch.bfloat16, device=dev)
        self.h_buf = torch.empty((S, h), dtype=torch.bfloat16, device=dev)
        self.y_perm = torch.empty((S, d), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
        self.counts = torch.empty((E,), dtype=torch.int32, device=dev)
        self.offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        self.perm = torch.empty((S,), dtype=torch.int32, device=dev)
        self.inv = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.ws = torch.empty((max(moe.permute_workspace_bytes(T, k, E), 4),), dtype=torch.uint8, device=dev)

    def step(self, ev=None):
        moe, wl = self.moe, self.wl
        if ev is not None:
            ev[0].record()
        p = moe.moe_permute(self.x, self.ids, wl.E, x_perm=self.x_perm, counts=self.counts, offsets=self.offsets,
                            perm=self.perm, inv_map=self.inv, workspace=self.ws, gather=not self.fused)
        if ev is not None:
            ev[1].record()
        if self.fused:
            moe.moe_gemm_up_swiglu_gather(self.x, p.perm, p.offsets, self.w_ug, wl.k, h_buf=self.h_buf)
        else:
            moe.moe_gemm_up_swiglu(p.x_perm, p.offsets, self.w_ug, h_buf=self.h_buf)
        if ev is not None:
            ev[2].record()
        moe.moe_gemm_down(self.h_buf, p.offsets, self.w_down, y_perm=self.y_perm)
        if ev is not None:
            ev[3].record()
        moe.moe_unpermute(self.y_perm, p.inv_map, self.rw, y=self.y)
        if ev is not None:
            ev[4].record()

    def stage_calls(self) -> dict:
        """Each stage of the step on its own, reading the buffers an earlier step left (idempotent)."""
        moe, wl = self.moe, self.wl

        def permute():
            moe.moe_permute(self.x, self.ids, wl.E, x_perm=self.x_perm, counts=self.counts, offsets=self.offsets,
                            perm=self.perm, inv_map=self.inv, workspace=self.ws, gather=not self.fused)

        def gemm_up():
            if self.fused:
                moe.moe_gemm_up_swiglu_gather(self.x, self.perm, self.offsets, self.w_ug, wl.k, h_buf=self.h_buf)
            else:
                moe.moe_gemm_up_swiglu(self.x_perm, self.offsets, self.w_ug, h_buf=self.h_buf)

        return {"permute": permute, "gemm_up_swiglu": gemm_up,
                "gemm_down": lambda: moe.moe_gemm_down(self.h_buf, self.offsets, self.w_down, y_perm=self.y_perm),
                "unpermute": lambda: moe.moe_unpermute(self.y_perm, self.inv, self.rw, y=self.y)}


STAGES = ["permute", "gemm_up_swiglu", "gemm_down", "unpermute"]


def time_step(torch, step, steps: int, warmup: int, graph: bool = True) -> dict:
    """K eager steps with HIP events around every stage (per-stage times, each step's span on the stream), then,
    unless graph is False, the same step captured once in a HIP graph and K replays, wall-clock timed. The
    library allocates, synchronises and copies nothing, so its calls capture as they are; the kernels are the
    same, the host launch gaps between them are gone."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps
    graph_ms, graph_note, replay = None, None, None
    if graph:
        try:
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    step()
            torch.cuda.current_stream().wait_stream(side)
            for _ in range(warmup):
                g.replay()
            torch.cuda.synchronize()
            tg = time.perf_counter()
            for _ in range(steps):
                g.replay()
            torch.cuda.synchronize()
            graph_ms = (time.perf_counter() - tg) * 1e3 / steps
            replay = g.replay
        except Exception as exc:  # capture unavailable: the eager time stays the headline
            graph_note = f"graph capture failed ({type(exc).__name__}: {exc}); eager launches reported"
            torch.cuda.synchronize()
    stage_ms = {n: sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / steps for j, n in enumerate(STAGES)}
    step_ev = sorted(ev[0].elapsed_time(ev[4]) for ev in events)  # each step's own span on the stream
    step_events = {"mean_ms": sum(step_ev) / len(step_ev), "median_ms": step_ev[len(step_ev) // 2],
                   "min_ms": step_ev[0], "max_ms": step_ev[-1]}
    return {"eager_ms": eager_ms, "graph_ms": graph_ms, "graph_note": graph_note, "replay": replay,
            "stage_ms": stage_ms, "step_events": step_events}


def time_stages_graph(torch, calls: dict, reps: int = 10, rounds: int = 5) -> dict | None:
    """Each stage alone, `reps` back-to-back launches captured in one HIP graph, replayed `rounds` times between
    HIP events: the per-launch time without host launch gaps (the eager stage times include them, which for the
    ~10 us permute is a third of its time). Median over the rounds, ms per launch."""
    out = {}
    try:
        for name, fn in calls.items():
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    for _ in range(reps):
                        fn()
            torch.cuda.current_stream().wait_stream(side)
            g.replay()
            torch.cuda.synchronize()
            times = []
            for _ in range(rounds):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) / reps)
            out[name] = sorted(times)[len(times) // 2]
            del g
    except Exception:  # capture unavailable: the eager stage times stand alone
        torch.cuda.synchronize()
        return None
    return out


def stage_table(stage_ms: dict, algo: dict, M: int, d: int, h: int) -> dict:
    """Per-stage mean time with its rate: GB/s of algorithmic bytes for the HBM-bound permutations, TFLOP/s for
    the GEMMs (plus their algorithmic-byte rate, the bound of weight-streaming shapes)."""
    gemm1_flops, gemm2_flops = 2 * M * d * (2 * h), 2 * M * h * d

    def rate(b, ms):
        return b / ms / 1e6 if ms > 0 else None

    return {
        "permute": {"ms": stage_ms["permute"], "GB/s": rate(algo["permute"], stage_ms["permute"])},
        "gemm_up_swiglu": {"ms": stage_ms["gemm_up_swiglu"],
                           "TFLOP/s": gemm1_flops / stage_ms["gemm_up_swiglu"] / 1e9,
                           "algorithmic_GB/s": rate(algo["gemm_up_swiglu"], stage_ms["gemm_up_swiglu"])},
        "gemm_down": {"ms": stage_ms["gemm_down"], "TFLOP/s": gemm2_flops / stage_ms["gemm_down"] / 1e9,
                      "algorithmic_GB/s": rate(algo["gemm_down"], stage_ms["gemm_down"])},
        "unpermute": {"ms": stage_ms["unpermute"], "GB/s": rate(algo["unpermute"], stage_ms["unpermute"])},
    }


def measure_config(torch, moe, name: str, dev, steps: int, warmup: int, fused: bool = True) -> dict:
    """One named workload's step, timed as the headline is (graph replays; stages from eager events), with the
    load statistics of its routing. A parity-test configuration, reported beside the headline."""
    from workloads import WORKLOADS, make_workload

    wl = make_workload(name)
    run = StepRun(torch, moe, wl, dev, fused)
    tm = time_step(torch, run.step, steps, warmup)
    sg = time_stages_graph(torch, run.stage_calls()) if tm["graph_ms"] is not None else None
    cnt = run.counts.cpu().tolist()
    M = sum(cnt)
    nonempty = sum(c > 0 for c in cnt)
    ms = tm["graph_ms"] if tm["graph_ms"] is not None else tm["eager_ms"]
    flops = useful_flops(M, wl.d, wl.h)
    algo = algorithmic_bytes(wl.T, wl.k, M, wl.d, wl.h, nonempty, fused)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    t1 = gemm_tile_rows(wl.T * wl.k, wl.E, -(-wl.h // 128), cus)
    t2 = gemm_tile_rows(wl.T * wl.k, wl.E, -(-wl.d // 256), cus, down=True)
    out = {"workload": name, "seed": WORKLOADS[name][0], "T": wl.T, "k": wl.k, "E": wl.E, "d": wl.d, "h": wl.h,
           "M": M, "ms_per_step": ms, "timing": "graph replays" if tm["graph_ms"] is not None else "eager",
           "eager_ms_per_step": tm["eager_ms"], "useful_TFLOP/s": flops / (ms * 1e-3) / 1e12,
           "pct_of_peak": 100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "step_events": tm["step_events"], "stages": stage_table(tm["stage_ms"], algo, M, wl.d, wl.h),
           "stages_graph_ms": sg,
           "histogram": histogram_stats(cnt, t1), "down_tile_rows": t2}
    del run
    torch.cuda.empty_cache()
    return out


def file_sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def cpu_baseline(wl, tokens: int, min_seconds: float = 10.0, precision: str = "f32", max_runs: int = 5):
    """Time the oracle (as it stands) on the first `tokens` tokens of the workload: its per-expert loop in
    float32 (the form the method states), or float64 on request."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # threadpoolctl missing: report the process affinity
        threads = len(os.sched_getaffinity(0))
    sl = slice(0, tokens)
    # whole runs until about 10 s of host work (at most 5 runs); the rate is the mean over them
    runs, total = 0, 0.0
    while runs < max_runs and (runs == 0 or total < min_seconds):
        t0 = time.perf_counter()
        r = oracle.moe_expert_forward(wl.x[sl], wl.expert_ids[sl], wl.routing_w[sl], wl.w_ug, wl.w_down,
                                      precision=precision)
        total += time.perf_counter() - t0
        runs += 1
    dt = total / runs
    M = int(r.offsets[-1])
    return {"value": useful_flops(M, wl.d, wl.h) / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": total, "runs": runs,
            "sample": f"first {tokens} of {wl.T} tokens of {wl.name} ({M} routed rows, all {wl.E} experts' weights), "
                      f"{'float32' if precision == 'f32' else 'float64'} oracle (per-expert loop), mean of {runs} "
                      f"runs ({total:.1f} s)", "host_cpus": len(os.sched_getaffinity(0)),
            "numpy": np.__version__, "precision": precision}


def summarize_telemetry(samples, t0: float, t1: float, settle: float = 0.25):
    """Clock and power over the steady part of a back-to-back loop.

    samples: (time, per-XCD gfx clocks in MHz, socket power in W, gfx activity in %) tuples; entries that the
    driver reports as unavailable (anything not a number) are skipped. The first `settle` fraction of the loop
    (clock ramp) is left out.
    """
    lo = t0 + settle * (t1 - t0)
    steady = [s for s in samples if lo <= s[0] <= t1]

    def nums(vals):
        return [float(v) for v in vals if isinstance(v, (int, float)) and not isinstance(v, bool) and v > 0]

    clk = [sum(c) / len(c) for c in (nums(s[1] or []) for s in steady) if c]
    pwr = nums([s[2] for s in steady])
    act = nums([s[3] for s in steady])

    def stats(v):
        if not v:
            return None
        v = sorted(v)
        return {"median": v[len(v) // 2], "min": v[0], "max": v[-1]}

    distinct = len({(tuple(nums(s[1] or [])), s[2], s[3]) for s in steady})
    return {"samples": len(steady), "distinct_readings": distinct, "gfx_clock_mhz": stats(clk),
            "socket_power_w": stats(pwr), "gfx_activity_pct": stats(act)}


def energy_average_power(e0, e1, host_seconds: float):
    """Average power from two energy-counter readings (accumulator, microjoules per count, timestamp).

    The timestamp's unit is not fixed across library versions: it is taken as the power of ten that makes the
    counter's interval closest to the host's. Returns (watts, seconds) or (None, None).
    """
    try:
        de = (e1["energy_accumulator"] - e0["energy_accumulator"]) * float(e0["counter_resolution"]) * 1e-6
        dts = e1["timestamp"] - e0["timestamp"]
    except (KeyError, TypeError):
        return None, None
    if de <= 0 or dts <= 0 or host_seconds <= 0:
        return None, None
    unit = min((1e9, 1e8, 1e6, 1e3), key=lambda u: abs(math.log(dts / u / host_seconds)))
    secs = dts / unit
    return de / secs, secs


def steady_telemetry(torch, run_step, ms_per_step: float, seconds: float = 3.0, interval_s: float = 0.02):
    """GPU clock and socket power read through amdsmi (read-only queries) while the step runs back to back.

    The loop is separate from the timed region. Returns {"error": ...} when the library or the device is not
    reachable; the benchmark line is printed either way.
    """
    import threading

    try:
        import amdsmi
    except Exception as exc:  # the python bindings are not installed
        return {"error": f"amdsmi not importable ({type(exc).__name__})"}
    try:
        amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
    except Exception as exc:
        return {"error": f"amdsmi_init failed ({type(exc).__name__}: {exc})"}
    try:
        props = torch.cuda.get_device_properties(torch.cuda.current_device())
        want = (props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
        handles = amdsmi.amdsmi_get_processor_handles()
        handle = None
        for hd in handles:
            dom, bus, rest = amdsmi.amdsmi_get_gpu_device_bdf(hd).split(":")
            if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                handle = hd
                break
        if handle is None:
            return {"error": f"no amdsmi device at PCI {want[0]:04x}:{want[1]:02x}:{want[2]:02x} "
                             f"({len(handles)} visible)"}
        n = max(1, int(seconds * 1e3 / max(ms_per_step, 1e-3)))
        samples, done = [], threading.Event()

        def sampler():
            while not done.is_set():
                try:
                    m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                    clks = m.get("current_gfxclks")
                    samples.append((time.perf_counter(), clks if isinstance(clks, list) else [],
                                    m.get("current_socket_power"), m.get("average_gfx_activity")))
                except Exception:  # one failed read drops one sample
                    pass
                time.sleep(interval_s)

        def energy():
            try:
                return amdsmi.amdsmi_get_energy_count(handle)
            except Exception:  # no energy counter on this device or library
                return None

        torch.cuda.synchronize()
        th = threading.Thread(target=sampler, daemon=True)
        th.start()
        t0 = time.perf_counter()
        for _ in range(n // 4):  # settle: the clock and the counters' windows fill with the loop
            run_step()
        torch.cuda.synchronize()
        e0, te0 = energy(), time.perf_counter()
        for _ in range(n - n // 4):
            run_step()
        torch.cuda.synchronize()
        e1, t1 = energy(), time.perf_counter()
        done.set()
        th.join()
        out = summarize_telemetry(samples, t0, t1)
        watts, secs = energy_average_power(e0, e1, t1 - te0) if e0 and e1 else (None, None)
        out["energy_average_power_w"] = watts
        out["energy_interval_s"] = secs
        out.update({"steps": n, "seconds": t1 - t0, "source": "amdsmi gpu_metrics (current_gfxclks averaged over "
                    "XCDs, current_socket_power) sampled every 20 ms over the last three quarters of a back-to-back "
                    "loop (the driver refreshes the table less often: distinct_readings counts the fresh ones), and "
                    "the energy counter's average over the same three quarters"})
        try:
            cap = amdsmi.amdsmi_get_power_info(handle).get("power_limit")  # microwatts
            out["power_limit_w"] = cap / 1e6 if isinstance(cap, (int, float)) and cap > 0 else None
        except Exception:
            out["power_limit_w"] = None
        return out
    except Exception as exc:
        return {"error": f"{type(exc).__name__}: {exc}"}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="zipf64", choices=["toy", "edge", "qwen3_30b", "zipf64", "square", "zipf64_top8"])
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other named workloads (reported under 'configs' beside the headline)")
    ap.add_argument("--no-variants", action="store_true", help="skip the padded-BMM and per-expert-loop variants")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="tokens in the oracle sample (0: all T tokens)")
    ap.add_argument("--unfused", action="store_true",
                    help="copy rows into x_perm in moe_permute instead of gathering them inside the gate/up GEMM")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain device copy of known size (HBM counter calibration)")
    ap.add_argument("--no-telemetry", action="store_true",
                    help="skip the clock and power readings taken during a steady loop after the timed region")
    ap.add_argument("--eager", action="store_true",
                    help="report eager launches as the headline instead of replays of the step captured in a HIP graph")
    ap.add_argument("--sweep", choices=SWEEPS,
                    help="instead of the step, run one sweep and print its own JSON line: histogram (Fig 40), "
                         "capacity (Fig 38) or decomposition (Fig 39) of one grouped projection, or the step's "
                         "backward kernels (Eq 15)")
    ap.add_argument("--sweep-samples", type=int, default=20, help="timed samples per sweep point")
    ap.add_argument("--sweep-warmup", type=int, default=10, help="warm-up samples per sweep point")
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
    if args.sweep:
        print(json.dumps(SWEEPS[args.sweep](torch, moe, dev, args.sweep_warmup, args.sweep_samples)))
        return 0
    fused = not args.unfused
    wl = make_workload(args.config)
    T, k, E, d, h = wl.T, wl.k, wl.E, wl.d, wl.h
    S = T * k
    run = StepRun(torch, moe, wl, dev, fused)
    x, ids, rw, w_ug, w_down = run.x, run.ids, run.rw, run.w_ug, run.w_down
    x_perm, y_perm, counts, offsets, inv, ws = run.x_perm, run.y_perm, run.counts, run.offsets, run.inv, run.ws
    tm = time_step(torch, run.step, args.steps, args.warmup, graph=not args.eager)
    eager_ms, graph_ms, graph_note, replay = tm["eager_ms"], tm["graph_ms"], tm["graph_note"], tm["replay"]
    stages_graph = time_stages_graph(torch, run.stage_calls()) if graph_ms is not None else None
    stage_ms, step_events = tm["stage_ms"], tm["step_events"]

    M = int(offsets[-1].item())
    nonempty = int((counts > 0).sum().item())
    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    # Clock and power during about 1.5 s of the headline step back to back (after the timed region).
    telemetry = None if args.no_telemetry else steady_telemetry(torch, replay or run.step, ms_per_step)
    flops = useful_flops(M, d, h)
    value = flops / (ms_per_step * 1e-3) / 1e12
    algo = algorithmic_bytes(T, k, M, d, h, nonempty, fused)
    gemm1_flops = 2 * M * d * (2 * h)
    stages = stage_table(stage_ms, algo, M, d, h)

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
        tokens = min(args.cpu_tokens or T, T)
        cpu = cpu_baseline(wl, tokens)  # the float32 per-expert loop, about 10 s of host work
        # the same oracle in float64, one run, for reference
        f64 = cpu_baseline(wl, tokens, min_seconds=0.0, precision="f64", max_runs=1)
        cpu["f64_oracle"] = {key: f64[key] for key in ("value", "unit", "cores", "seconds", "runs", "sample")}

    # Load statistics of the headline routing, and the other named workloads timed the same way.
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    hist = histogram_stats(counts.cpu().tolist(), gemm_tile_rows(S, E, -(-h // 128), cus))
    configs = None
    if not args.no_configs:
        configs = {}
        for name in [n for n in WORKLOADS if n != wl.name]:
            _progress(f"config {name}")
            try:
                configs[name] = measure_config(torch, moe, name, dev, steps=args.steps, warmup=args.warmup,
                                               fused=fused)
            except Exception as exc:  # one failed configuration is reported, not fatal to the headline
                configs[name] = {"error": f"{type(exc).__name__}: {exc}"}

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
        "timing": "replays of the step captured in a HIP graph" if graph_ms is not None else "eager launches",
        "eager_ms_per_step": eager_ms,
        "graph_note": graph_note,
        "step_events": step_events,
        "useful_gflop": flops / 1e9,
        "stages": stages,
        # each stage alone in graph replays (no host launch gaps), ms per launch
        "stages_graph_ms": stages_graph,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "histogram": hist,
        "variants": variants,
        "telemetry": telemetry,
        "configs": configs,
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


# --------------------------------------------------------------------------
# Single-projection sweeps (OLMo report Sec 9.6): one grouped projection
# Y[rows_e] = A[rows_e] @ W[e] (moe_gemm_down), 16 local experts unless stated.
# --------------------------------------------------------------------------


def _progress(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class QueuedTimer:
    """Fig 38's protocol: warm-up and timed samples are all queued behind a device-side gate (a
    spin kernel of fixed length) and released together, so host launch gaps never reach the GPU;
    each timed sample is bracketed by HIP events on the launch stream."""

    def __init__(self, torch):
        self.torch = torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        a.record()
        torch.cuda._sleep(2_000_000)
        b.record()
        torch.cuda.synchronize()
        self.cycles_per_ms = 2_000_000 / max(a.elapsed_time(b), 1e-3)
        self.gate_overruns = 0

    def __call__(self, fn, warmup: int, samples: int, gate_ms: float = 30.0):
        torch = self.torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
        gate_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        torch.cuda._sleep(int(gate_ms * self.cycles_per_ms))
        gate_end.record()
        for _ in range(warmup):
            fn()
        for a, b in evs:
            a.record()
            fn()
            b.record()
        queued_ms = (time.perf_counter() - t0) * 1e3
        torch.cuda.synchronize()
        if queued_ms > gate_ms:  # the gate opened before the host finished queuing
            self.gate_overruns += 1
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        return {"mean_ms": sum(ts) / len(ts), "median_ms": ts[len(ts) // 2], "min_ms": ts[0]}


def _offsets_dev(torch, counts, dev):
    import numpy as np

    offs = np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))]).astype(np.int32)
    return torch.from_numpy(offs).to(dev)


def sweep_histogram(torch, moe, dev, warmup, samples):
    """Fig 40: fixed rows and FLOPs, 100 load histograms spanning Eq 18's imbalance range.

    Each histogram is timed under four fixed expert-index orders; conditions run in a seeded
    random order, and a balanced control is timed before the first and after every ten
    conditions. A condition's relative throughput is the mean of its two bracketing controls'
    times over its own time; a histogram's value is the mean over its four orders."""
    import numpy as np
    from scipy.stats import spearmanr

    from workloads import SWEEP, balanced_counts, dirichlet_histograms, expert_orders, projection_inputs

    E, M, dim = SWEEP["E"], SWEEP["M"], SWEEP["dim"]
    a, w = projection_inputs(M, dim, dim, E, seed=40, device=dev)
    y = torch.empty((M, dim), dtype=torch.bfloat16, device=dev)
    hists = dirichlet_histograms()
    orders = expert_orders(E, 4)
    conds = []
    for hi, hrec in enumerate(hists):
        for oi, order in enumerate(orders):
            per_expert = np.empty(E, dtype=np.int64)
            per_expert[order] = hrec["counts"]  # expert order[i] gets the i-th count
            conds.append((hi, oi, _offsets_dev(torch, per_expert, dev)))
    rng = np.random.default_rng(42)
    conds = [conds[i] for i in rng.permutation(len(conds))]
    bal = _offsets_dev(torch, balanced_counts(E, M), dev)
    timer = QueuedTimer(torch)

    def run(offs):
        return timer(lambda: moe.moe_gemm_down(a, offs, w, y_perm=y), warmup, samples)["mean_ms"]

    controls = [run(bal)]
    times = []
    for i, (hi, oi, offs) in enumerate(conds):
        times.append(run(offs))
        if (i + 1) % 10 == 0 or i + 1 == len(conds):
            controls.append(run(bal))
            _progress(f"histogram sweep: {i + 1}/{len(conds)} conditions, control {controls[-1]:.3f} ms")
    rel = np.zeros((len(hists), len(orders)))
    ms = np.zeros((len(hists), len(orders)))
    for i, (hi, oi, _) in enumerate(conds):
        c = 0.5 * (controls[i // 10] + controls[i // 10 + 1])
        rel[hi, oi] = c / times[i]
        ms[hi, oi] = times[i]
    rel_h = rel.mean(axis=1)
    imb = np.array([h["imbalance"] for h in hists])
    rho = float(spearmanr(imb, rel_h).statistic)
    boot = []
    brng = np.random.default_rng(43)
    for _ in range(2000):
        idx = brng.integers(0, len(hists), len(hists))
        boot.append(spearmanr(imb[idx], rel_h[idx]).statistic)
    lo, hi_ = np.nanpercentile(boot, [2.5, 97.5])
    flops = 2 * M * dim * dim
    bal_ms = float(np.mean(controls))
    bins = sorted({h["bin"] for h in hists})
    medians = [{"bin": b, "imbalance_median": float(np.median(imb[[h["bin"] == b for h in hists]])),
                "rel_median": float(np.median(rel_h[[h["bin"] == b for h in hists]]))} for b in bins]
    return {
        "metric": "grouped projection throughput relative to balanced load vs imbalance I_H (Eq 18)",
        "sweep": "histogram", "unit": "ratio", "data": "synthetic", "dtype": "bf16",
        "config": {"workload": "histogram sweep", "E": E, "M": M, "d": dim, "h": dim, "align": SWEEP["align"],
                   "min_rows": SWEEP["min_rows"], "histograms": len(hists), "orders": len(orders),
                   "warmup": warmup, "samples": samples, "kernel": "moe_gemm_down"},
        "balanced_ms": bal_ms, "balanced_TFLOP/s": flops / bal_ms / 1e9,
        "controls_ms_min_max": [float(min(controls)), float(max(controls))],
        "spearman_rho": rho, "bootstrap_95": [float(lo), float(hi_)],
        "bin_medians": medians, "gate_overruns": timer.gate_overruns,
        "histograms": [{"imbalance": float(imb[i]), "alpha": float(hists[i]["alpha"]),
                        "counts_sorted": sorted(hists[i]["counts"].tolist(), reverse=True),
                        "rel": float(rel_h[i]), "rel_by_order": [float(v) for v in rel[i]],
                        "ms": float(ms[i].mean())} for i in range(len(hists))],
    }


def sweep_capacity(torch, moe, dev, warmup, samples):
    """Fig 38: exact-row grouped projection vs a batched GEMM padded to 1.25x the mean load, across
    total routed rows M with balanced routing (M/16 rows per expert); kernel time only, the padded
    operand built before timing. Useful FLOPs count valid rows only, 2*M*d*h."""
    from workloads import balanced_counts, projection_inputs

    E, dim = 16, 4096
    Ms = [64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536, 98304, 131072]
    a, w = projection_inputs(max(Ms), dim, dim, E, seed=38, device=dev)
    y = torch.empty((max(Ms), dim), dtype=torch.bfloat16, device=dev)
    timer = QueuedTimer(torch)
    points = []
    for M in Ms:
        counts = balanced_counts(E, M)
        offs = _offsets_dev(torch, counts, dev)
        C = math.ceil(1.25 * M / E)
        pad = torch.zeros((E, C, dim), dtype=torch.bfloat16, device=dev)
        lo = 0
        for e in range(E):
            pad[e, :counts[e]] = a[lo:lo + counts[e]]
            lo += int(counts[e])
        out = torch.empty((E, C, dim), dtype=torch.bfloat16, device=dev)
        am = a[:M]
        ym = y[:M]
        g = timer(lambda: moe.moe_gemm_down(am, offs, w, y_perm=ym), warmup, samples)
        b = timer(lambda: torch.bmm(pad, w, out=out), warmup, samples)
        flops = 2 * M * dim * dim
        points.append({"M": M, "rows_per_expert": M // E, "C": C,
                       "grouped_ms": g["mean_ms"], "bmm_ms": b["mean_ms"],
                       "grouped_TFLOP/s": flops / g["mean_ms"] / 1e9, "bmm_useful_TFLOP/s": flops / b["mean_ms"] / 1e9,
                       "bmm_padded_TFLOP/s": 2 * E * C * dim * dim / b["mean_ms"] / 1e9,
                       "bmm_over_grouped_time": b["mean_ms"] / g["mean_ms"],
                       "grouped_median_ms": g["median_ms"], "bmm_median_ms": b["median_ms"]})
        del pad, out
        _progress(f"capacity sweep: M={M} grouped {g['mean_ms']:.4f} ms, bmm {b['mean_ms']:.4f} ms")
    cross = next((p["M"] for p in points if p["bmm_over_grouped_time"] > 1.0), None)
    # the stable crossover: the smallest M from which the grouped projection is faster at every larger M too
    stable = None
    for p in reversed(points):
        if p["bmm_over_grouped_time"] <= 1.0:
            break
        stable = p["M"]
    return {"metric": "useful TFLOP/s of one grouped projection vs padded BMM at 1.25x capacity, across M",
            "sweep": "capacity", "unit": "TFLOP/s", "data": "synthetic", "dtype": "bf16",
            "config": {"workload": "capacity sweep", "E": E, "d": dim, "h": dim, "capacity_factor": 1.25,
                       "warmup": warmup, "samples": samples, "kernel": "moe_gemm_down", "bmm": "torch.bmm"},
            "first_M_grouped_faster": cross, "stable_crossover_M": stable, "gate_overruns": timer.gate_overruns,
            "points": points}


def sweep_decomposition(torch, moe, dev, warmup, samples):
    """Fig 39 / Eq 17: one dense [T, 8192] @ [8192, 81920] projection vs the same weight split into
    4 or 8 column-block experts, each multiplying the whole input (the input repeated once per
    expert). Dense runs twice: the vendor GEMM (torch.matmul) and this library with one expert."""
    from workloads import projection_inputs

    K, N = 8192, 81920
    Ts = [1, 16, 128, 256, 1024, 4096, 8192, 16384, 32768, 65536]
    x_all, w1 = projection_inputs(max(Ts), K, N, 1, seed=39, device=dev)
    wd = w1[0]  # [K, N]
    blocks = {n: wd.view(K, n, N // n).permute(1, 0, 2).contiguous() for n in (4, 8)}  # [n, K, N/n]
    timer = QueuedTimer(torch)
    points = []
    for T in Ts:
        x = x_all[:T]
        flops = 2 * T * K * N
        res = {"T": T}
        out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        r = timer(lambda: torch.matmul(x, wd, out=out), warmup, samples)
        res["dense_vendor_TFLOP/s"] = flops / r["mean_ms"] / 1e9
        res["dense_vendor_ms"] = r["mean_ms"]
        offs1 = _offsets_dev(torch, [T], dev)
        r = timer(lambda: moe.moe_gemm_down(x, offs1, w1, y_perm=out), warmup, samples)
        res["dense_ours_TFLOP/s"] = flops / r["mean_ms"] / 1e9
        res["dense_ours_ms"] = r["mean_ms"]
        del out
        for n, wb in blocks.items():
            xr = x.repeat(n, 1)
            yb = torch.empty((n * T, N // n), dtype=torch.bfloat16, device=dev)
            offs = _offsets_dev(torch, [T] * n, dev)
            r = timer(lambda: moe.moe_gemm_down(xr, offs, wb, y_perm=yb), warmup, samples)
            res[f"grouped{n}_TFLOP/s"] = flops / r["mean_ms"] / 1e9
            res[f"grouped{n}_ms"] = r["mean_ms"]
            res[f"grouped{n}_over_dense_vendor"] = res[f"grouped{n}_TFLOP/s"] / res["dense_vendor_TFLOP/s"]
            del xr, yb
        points.append(res)
        _progress(f"decomposition sweep: T={T} " + ", ".join(f"{k} {v:.1f}" for k, v in res.items() if "TFLOP" in k))
    return {"metric": "useful TFLOP/s of one dense projection vs 4 and 8 column-block experts (Eq 17)",
            "sweep": "decomposition", "unit": "TFLOP/s", "data": "synthetic", "dtype": "bf16",
            "config": {"workload": "decomposition sweep", "K": K, "N": N, "experts": [4, 8], "warmup": warmup,
                       "samples": samples, "kernel": "moe_gemm_down", "dense_vendor": "torch.matmul"},
            "gate_overruns": timer.gate_overruns, "points": points}


def sweep_backward(torch, moe, dev, warmup, samples):
    """The expert step's backward on the zipf64 workload (OLMo report Sec 9.5, Eq 15): unpermute
    backward, Dgrad and Wgrad of the down projection ([E, h, d]), recompute of the gate/up
    pre-activation U, SwiGLU backward, Dgrad and Wgrad of the gate/up projection ([E, 2h, d]) and the
    permute backward, each timed on its own (queued samples, HIP events). ``value`` is the useful
    backward work, 12*M*d*h (the four backward GEMMs, 2*M*d_in*d_out each), over the summed time of
    every kernel of the chain, the U recompute included. ``with_saved_u`` gives the chain without the
    recompute, and what keeping U costs the forward's gate/up launch (moe_gemm_up_swiglu_u)."""
    import numpy as np

    from workloads import make_workload

    wl = make_workload("zipf64")
    T, k, E, d, h = wl.T, wl.k, wl.E, wl.d, wl.h
    S = T * k

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    x, w_ug, w_down = bf(wl.x), bf(wl.w_ug), bf(wl.w_down)
    ids = torch.from_numpy(wl.expert_ids).to(dev)
    rw = torch.from_numpy(wl.routing_w).to(dev)
    y, p, h_buf, y_perm = moe.moe_expert_forward(x, ids, rw, w_ug, w_down, fused_gather=False)
    M = int(p.offsets[-1].item())
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    dy = torch.randn((T, d), generator=g, device=dev).to(torch.bfloat16)
    dy_perm = torch.empty((S, d), dtype=torch.bfloat16, device=dev)
    d_rw = torch.empty((T, k), dtype=torch.float32, device=dev)
    dh = torch.empty((S, h), dtype=torch.bfloat16, device=dev)
    u = torch.empty((S, 2 * h), dtype=torch.bfloat16, device=dev)
    du = torch.empty((S, 2 * h), dtype=torch.bfloat16, device=dev)
    dxp = torch.empty((S, d), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    dwd = torch.empty_like(w_down)
    dwu = torch.empty_like(w_ug)
    ws = torch.empty((max(moe.wgrad_workspace_bytes(S, d, 2 * h, E), moe.wgrad_workspace_bytes(S, h, d, E), 16),),
                     dtype=torch.uint8, device=dev)
    timer = QueuedTimer(torch)
    stages = [
        ("unpermute_backward", lambda: moe.moe_unpermute_backward(dy, y_perm, p.inv_map, rw, dy_perm=dy_perm,
                                                                  d_routing_w=d_rw), None,
         2 * T * d + 4 * M * d + 16 * S),
        ("dgrad_down", lambda: moe.moe_grouped_dgrad(dy_perm, p.offsets, w_down, "in_out", dx=dh), 2 * M * h * d, None),
        ("wgrad_down", lambda: moe.moe_grouped_wgrad(h_buf, dy_perm, p.offsets, "in_out", dw=dwd, workspace=ws),
         2 * M * h * d, None),
        ("recompute_u", lambda: moe.moe_grouped_projection(p.x_perm, p.offsets, w_ug, "out_in", y=u), None, None),
        ("swiglu_backward", lambda: moe.moe_swiglu_backward(dh, u, p.offsets, du=du), None, 10 * M * h),
        ("dgrad_gate_up", lambda: moe.moe_grouped_dgrad(du, p.offsets, w_ug, "out_in", dx=dxp), 4 * M * h * d, None),
        ("wgrad_gate_up", lambda: moe.moe_grouped_wgrad(p.x_perm, du, p.offsets, "out_in", dw=dwu, workspace=ws),
         4 * M * h * d, None),
        ("permute_backward", lambda: moe.moe_permute_backward(dxp, p.inv_map, dx=dx), None, 2 * M * d + 2 * T * d + 4 * S),
    ]
    res, total_ms, gemm_flops = {}, 0.0, 0
    for name, fn, flops, nbytes in stages:
        r = timer(fn, warmup, samples)
        entry = {"ms": r["mean_ms"], "median_ms": r["median_ms"]}
        if flops:
            entry["TFLOP/s"] = flops / r["mean_ms"] / 1e9
            gemm_flops += flops
        elif nbytes:
            entry["GB/s"] = nbytes / r["mean_ms"] / 1e6
        else:  # the U recompute: forward-shaped GEMM, not useful backward work
            entry["TFLOP/s"] = 4 * M * h * d / r["mean_ms"] / 1e9
        total_ms += r["mean_ms"]
        res[name] = entry
        _progress(f"backward: {name} {r['mean_ms']:.4f} ms")
    # A forward that keeps U (moe_gemm_up_swiglu_u) lets the backward drop the recompute; the
    # forward's gate/up launch pays for the extra U stores instead.
    h2 = torch.empty_like(h_buf)
    fwd = {}
    for name, fn in (("gate_up", lambda: moe.moe_gemm_up_swiglu(p.x_perm, p.offsets, w_ug, h_buf=h2)),
                     ("gate_up_save_u", lambda: moe.moe_gemm_up_swiglu_u(p.x_perm, p.offsets, w_ug, h_buf=h2,
                                                                          u_buf=u))):
        r = timer(fn, warmup, samples)
        fwd[name] = {"ms": r["mean_ms"], "TFLOP/s": 4 * M * h * d / r["mean_ms"] / 1e9}
        _progress(f"backward: forward {name} {r['mean_ms']:.4f} ms")
    saved_ms = total_ms - res["recompute_u"]["ms"]
    return {"metric": "useful TFLOP/s of the expert step's backward (12*M*d*h over every kernel of the chain)",
            "sweep": "backward", "value": gemm_flops / total_ms / 1e9, "unit": "TFLOP/s", "data": "synthetic",
            "dtype": "bf16",
            "config": {"workload": "zipf64 backward", "T": T, "k": k, "E": E, "d": d, "h": h, "M": M,
                       "warmup": warmup, "samples": samples},
            "backward_ms": total_ms, "stages": res,
            "with_saved_u": {"backward_ms": saved_ms, "TFLOP/s": gemm_flops / saved_ms / 1e9,
                             "forward_gate_up": fwd,
                             "forward_extra_ms": fwd["gate_up_save_u"]["ms"] - fwd["gate_up"]["ms"]},
            "gate_overruns": timer.gate_overruns}


SWEEPS = {"histogram": sweep_histogram, "capacity": sweep_capacity, "decomposition": sweep_decomposition,
          "backward": sweep_backward}


if __name__ == "__main__":
    sys.exit(main())
