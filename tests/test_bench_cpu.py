"""bench.py's host-side contract, on the CPU: one GPU only, and its FLOP and byte models."""

import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    err = capsys.readouterr().err
    assert "one GPU only" in err


def test_world_size_above_one_exits(monkeypatch, capsys):
    monkeypatch.setenv("WORLD_SIZE", "8")
    assert bench.main([]) == 2
    assert "WORLD_SIZE=8" in capsys.readouterr().err


def test_useful_flops_follow_the_six_mdh_convention():
    # the four-expert toy: M = 10 rows, d = 64, h = 128 -> 491,520 useful FLOP
    assert bench.useful_flops(10, 64, 128) == 491_520
    # one GPU's share of the Zipf-skewed layer: 65,536 rows, d = 2048, h = 768
    assert bench.useful_flops(65536, 2048, 768) == 618_475_290_624


def test_algorithmic_bytes_of_the_fused_step():
    T, k, M, d, h, E = 8192, 8, 65536, 2048, 768, 60
    b = bench.algorithmic_bytes(T, k, M, d, h, E, fused=True)
    gemm1 = 2 * T * d + E * 2 * (2 * h) * d + 2 * M * h
    assert b["gemm_up_swiglu"] == gemm1 == 511_705_088
    unfused = bench.algorithmic_bytes(T, k, M, d, h, E, fused=False)
    # the unfused path copies rows into x_perm: the permute reads X and writes x_perm, GEMM 1 reads x_perm
    assert unfused["permute"] - b["permute"] == 2 * T * d + 2 * M * d
    assert unfused["gemm_up_swiglu"] - b["gemm_up_swiglu"] == 2 * M * d - 2 * T * d


@pytest.mark.parametrize("peak,bw,intensity,expect", [(2500.0, 8000.0, 1000.0, 2500.0), (2500.0, 8000.0, 0.1, 800.0)])
def test_roofline_attainable(peak, bw, intensity, expect):
    assert bench.roofline_attainable(intensity, bw, peak) == pytest.approx(expect)


def test_telemetry_summary_keeps_the_steady_part_and_skips_unavailable_readings():
    # (time, per-XCD clocks, socket power, activity); the driver marks missing readings "N/A"
    samples = [(0.1, [1000] * 8, 500, 50),            # inside the settle window: dropped
               (0.5, [2000, 2100, "N/A", 1900], 1300, 99),
               (0.7, [1800] * 8, "N/A", 100),
               (0.9, ["N/A"] * 8, 1350, "N/A"),
               (1.5, [2400] * 8, 1400, 100)]           # after the loop ended: dropped
    out = bench.summarize_telemetry(samples, t0=0.0, t1=1.0)
    assert out["samples"] == 3
    assert out["gfx_clock_mhz"] == {"median": 2000.0, "min": 1800.0, "max": 2000.0}
    assert out["socket_power_w"] == {"median": 1350.0, "min": 1300.0, "max": 1350.0}
    assert out["gfx_activity_pct"]["max"] == 100.0
    assert bench.summarize_telemetry([], 0.0, 1.0)["gfx_clock_mhz"] is None


def test_energy_average_power_picks_the_timestamp_unit():
    # 2 s at 1,350 W in 15.3 uJ counts, timestamps in nanoseconds and in 10 ns ticks
    counts = 1350.0 * 2.0 / 15.3e-6
    e0 = {"energy_accumulator": 1000, "counter_resolution": 15.3, "timestamp": 5_000_000_000}
    for unit in (1e9, 1e8):
        e1 = {"energy_accumulator": 1000 + counts, "counter_resolution": 15.3,
              "timestamp": 5_000_000_000 + int(2.0 * unit)}
        watts, secs = bench.energy_average_power(e0, e1, host_seconds=2.05)
        assert secs == pytest.approx(2.0) and watts == pytest.approx(1350.0, rel=1e-6)
    assert bench.energy_average_power(e0, dict(e0), 1.0) == (None, None)  # no energy counted


def test_histogram_statistics_agree_with_the_oracle():
    # bench.py carries its own copies of Eq 14, 16 and 18 (it may not use the oracle outside its CPU-baseline leg)
    import numpy as np

    import oracle
    from workloads import make_workload

    for counts in ([1, 4, 3, 2], [0, 7, 0, 7], [5], [19346, 8274, 0, 133, 1], list(range(64))):
        assert bench.entropy_deficit(counts) == pytest.approx(oracle.entropy_deficit(np.array(counts)), abs=1e-12)
    for c, mbar, ranks in ((1.25, 2.5, 1), (1.25, 512, 1), (1.25, 103.2, 2), (1.25, 100, 8), (1.25, 1024.0, 1)):
        assert bench.capacity_eq16(c, mbar, ranks) == oracle.capacity_eq16(c, mbar, ranks)
    wl = make_workload("toy")
    st = bench.histogram_stats(np.bincount(wl.expert_ids.reshape(-1), minlength=4).tolist(), tile_rows=2)
    # Figs 35-37: C = 4, 16 rows executed, rho_pad = 0.375, no row past C; 12 tile slots hold 10 rows at 2 rows
    assert st["bmm_capacity_C"] == 4 and st["rho_pad_eq14_at_C"] == 0.375 and st["bmm_rows_dropped"] == 0
    assert st["rho_pad_eq14_unclipped"] == 0.375 and st["capacity_eq16_c1.25_one_rank"] == 8
    assert st["grouped_tile_padding"] == pytest.approx(1 - 10 / 12)
    assert st["I_H_eq18"] == pytest.approx(oracle.entropy_deficit(np.array([1, 4, 3, 2])))
    # an overflowing expert: rows past C are dropped and Eq 14 counts only the rows that fit
    st = bench.histogram_stats([10, 0, 0, 2], tile_rows=8)  # C = ceil(1.25 * 12 / 4) = 4; 4 + 2 rows fit
    assert st["bmm_capacity_C"] == 4 and st["bmm_rows_dropped"] == 6
    assert st["rho_pad_eq14_at_C"] == pytest.approx(1 - 6 / 16)


def test_tile_height_rule():
    # zipf64: 65,536 slots over 64 experts, 6 gate/up column tiles -> 256-row tiles; Qwen3-shaped: 128
    assert bench.gemm_tile_rows(65536, 64, 6) == 256
    assert bench.gemm_tile_rows(32768, 128, 6) == 128
    # the down projection takes 256-row tiles for a mean of 192-256 rows per expert as well
    assert bench.gemm_tile_rows(32768, 128, 8, down=True) == 256
    assert bench.gemm_tile_rows(24576, 128, 8, down=True) == 256
    assert bench.gemm_tile_rows(40960, 128, 8, down=True) == 128
    assert bench.gemm_tile_rows(2048, 16, 16, down=True) == 128
    # the edge workload: blocks are large, but its 256-row tiles could not occupy 256 CUs
    assert bench.gemm_tile_rows(4096, 8, 3) == 128
