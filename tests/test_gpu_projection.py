"""One grouped projection (moe_gemm_down on its own) against the oracle, on an MI355X.

This is the single-projection problem the sweeps time (OLMo report Sec 9.6:
Figs 38 and 40 time one square bf16 expert projection per local expert, Fig 39
and Eq 17 split one dense weight into column-block experts). Small ragged cases
are compared whole; the sweeps' own shapes are compared on sampled rows, which
the oracle computes one expert at a time. Tolerances are those of the step.
"""

import numpy as np
import pytest
import torch

import oracle
import ragged_grouped_gemm_histogram_amd as moe
from gpu_util import bits, say, to_dev, to_dev_bf16
from parity import compare_bf16
from workloads import (SWEEP, balanced_counts, dirichlet_histograms, expert_orders, projection_inputs,
                       to_bf16_bits)

pytestmark = pytest.mark.gpu


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))]).astype(np.int32)


def _sampled_rows(offsets, per_expert, seed):
    """First and last row of every non-empty expert plus ``per_expert`` random rows inside it."""
    rng = np.random.default_rng(seed)
    rows = []
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        pick = {lo, hi - 1} | set(rng.integers(lo, hi, size=per_expert).tolist())
        rows += [(e, r) for r in sorted(pick)]
    return rows


def _check_sampled(a, w, y, offsets, per_expert=2, seed=0, what="y"):
    """Oracle rows for a sample of each expert's rows, compared with the GPU's."""
    rows = _sampled_rows(offsets, per_expert, seed)
    got, ref = [], []
    for e in sorted({e for e, _ in rows}):
        idx = [r for ee, r in rows if ee == e]
        a_rows = bits(a[idx])
        w_e = bits(w[e:e + 1])
        ref.append(oracle.grouped_projection(a_rows, np.array([0, len(idx)], dtype=np.int32), w_e))
        got.append(bits(y[idx]))
    return compare_bf16(np.concatenate(got), np.concatenate(ref), what)


@pytest.mark.parametrize("counts,K,N", [
    ([0, 37, 300, 1, 129, 0, 513], 320, 576),   # ragged, empty experts, 128-row tiles
    ([700, 900, 420, 0, 1100], 192, 8712),       # large blocks, enough tiles to fill the device: 256-row tiles
    ([5, 0, 260, 77], 328, 200),                 # K and N not multiples of 64: zero-staged K remainder
    ([700, 900, 420, 0, 1100], 200, 8712),       # a K remainder on the 256-row tiles
    ([1], 64, 64),                               # one row
], ids=["ragged", "big-tiles", "k-tail", "big-k-tail", "one-row"])
def test_projection_whole(counts, K, N):
    say(f"[gpu] projection counts={counts} K={K} N={N}")
    rng = np.random.default_rng(sum(counts) + K)
    M = sum(counts)
    E = len(counts)
    a = to_bf16_bits(rng.standard_normal((M + 16, K), dtype=np.float32))
    w = to_bf16_bits(0.05 * rng.standard_normal((E, K, N), dtype=np.float32))
    offs = _offsets(counts)
    sentinel = torch.full((M + 16, N), 3.0, dtype=torch.bfloat16, device="cuda:0")
    y = moe.moe_gemm_down(to_dev_bf16(a), to_dev(offs), to_dev_bf16(w), y_perm=sentinel)
    torch.cuda.synchronize()
    ref = oracle.grouped_projection(a, offs, w)
    say("  " + str(compare_bf16(bits(y)[:M], ref, "y")))
    assert (bits(y)[M:] == bits(torch.tensor(3.0, dtype=torch.bfloat16))).all(), "rows past M were written"


@pytest.mark.parametrize("counts,K,N", [
    ([50000] * 4, 64, 512),               # 256-row tiles, one K stage each, ~6 tiles per workgroup
    ([100] * 300 + [0] * 20 + [37] * 280, 64, 1024),  # 128-row tiles (3-slot ring), one K stage each
    ([3000] * 2 + [5], 128, 8192),        # 256-row tiles, two K stages each
], ids=["big-k64", "small-k64", "big-k128"])
def test_projection_stream_across_tiles(counts, K, N):
    """Several tiles per workgroup with fewer K stages than ring slots: the loads of the next
    tile's first stages overlap the current tile's last stage and epilogue."""
    say(f"[gpu] projection stream E={len(counts)} M={sum(counts)} K={K} N={N}")
    rng = np.random.default_rng(len(counts) + K)
    M = sum(counts)
    a = to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    w = to_bf16_bits(0.1 * rng.standard_normal((len(counts), K, N), dtype=np.float32))
    offs = _offsets(counts)
    y = moe.moe_gemm_down(to_dev_bf16(a), to_dev(offs), to_dev_bf16(w))
    torch.cuda.synchronize()
    say("  " + str(compare_bf16(bits(y), oracle.grouped_projection(a, offs, w), "y")))


@pytest.fixture(scope="module")
def sweep_operands():
    E, M, dim = SWEEP["E"], SWEEP["M"], SWEEP["dim"]
    a, w = projection_inputs(M, dim, dim, E, seed=40, device="cuda:0")
    return a, w


def _histogram_cases():
    hists = dirichlet_histograms()
    most = max(hists, key=lambda h: h["imbalance"])
    mid = [h for h in hists if h["bin"] == 5][0]
    return {"balanced": balanced_counts(SWEEP["E"], SWEEP["M"]), "mid": mid["counts"], "most": most["counts"]}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", ["balanced", "mid", "most"])
def test_histogram_sweep_shape(sweep_operands, case):
    """Fig 40's operands (16 experts, 65,536 rows, d = h = 4096) under three of its histograms."""
    a, w = sweep_operands
    counts = _histogram_cases()[case]
    order = expert_orders(SWEEP["E"], 4)[1]
    per_expert = np.empty_like(counts)
    per_expert[order] = counts
    offs = _offsets(per_expert)
    say(f"[gpu] histogram sweep case={case} counts={per_expert.tolist()}")
    y = moe.moe_gemm_down(a, to_dev(offs), w)
    torch.cuda.synchronize()
    say("  " + str(_check_sampled(a, w, y, offs, per_expert=3, seed=1)))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M", [64, 131072])
def test_capacity_sweep_ends(M):
    """Fig 38's smallest and largest balanced points: 4 and 8192 rows per expert."""
    E, dim = 16, 4096
    say(f"[gpu] capacity sweep M={M}")
    a, w = projection_inputs(M, dim, dim, E, seed=38, device="cuda:0")
    offs = _offsets(balanced_counts(E, M))
    y = moe.moe_gemm_down(a, to_dev(offs), w)
    torch.cuda.synchronize()
    say("  " + str(_check_sampled(a, w, y, offs, per_expert=2, seed=2)))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M", [3072, 4096])
def test_down_tall_tiles_balanced(M):
    """The down projection takes 256-row tiles for a mean of 192-256 rows per expert: balanced
    16-expert d = h = 4096 projections at 192 and 256 rows per expert (Fig 38's operands)."""
    E, dim = 16, 4096
    say(f"[gpu] down projection, tall tiles, balanced M={M}")
    a, w = projection_inputs(M, dim, dim, E, seed=38, device="cuda:0")
    offs = _offsets(balanced_counts(E, M))
    y = moe.moe_gemm_down(a, to_dev(offs), w)
    torch.cuda.synchronize()
    say("  " + str(_check_sampled(a, w, y, offs, per_expert=4, seed=3)))


def test_down_tall_tiles_ragged():
    """Ragged experts averaging 224 rows (256-row tiles for the down projection): each expert's last tile
    holds 1 to 255 rows, so the waves skipping their matrix work vary from tile to tile; compared whole."""
    rng = np.random.default_rng(224)
    E, K, N = 32, 256, 2048
    counts = rng.integers(150, 299, size=E)
    counts[3], counts[17] = 0, 1
    counts[5] += 224 * E - int(counts.sum())
    assert 192 * E <= counts.sum() <= 256 * E and counts.min() >= 0
    M = int(counts.sum())
    say(f"[gpu] down projection, tall tiles, ragged counts={counts.tolist()}")
    a = to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    w = to_bf16_bits(0.05 * rng.standard_normal((E, K, N), dtype=np.float32))
    offs = _offsets(counts)
    y = moe.moe_gemm_down(to_dev_bf16(a), to_dev(offs), to_dev_bf16(w))
    torch.cuda.synchronize()
    say("  " + str(compare_bf16(bits(y), oracle.grouped_projection(a, offs, w), "y")))


@pytest.mark.parametrize("T,K,N", [(300, 1024, 4096), (128, 8192, 81920)], ids=["small", "fig39-T128"])
def test_decomposition_eq17(T, K, N):
    """Eq 17 on the GPU: 4 or 8 column-block experts over the repeated input give the dense
    projection's columns. Every expert multiplies the same rows with the same K order, so the
    grouped outputs equal the one-expert (dense) launch bit for bit; the dense launch is held
    to the oracle on sampled rows (all rows for the small case)."""
    say(f"[gpu] decomposition T={T} K={K} N={N}")
    x, w1 = projection_inputs(T, K, N, 1, seed=39, device="cuda:0")
    dense = moe.moe_gemm_down(x, to_dev(np.array([0, T], dtype=np.int32)), w1)
    for n in (4, 8):
        blocks = w1[0].view(K, n, N // n).permute(1, 0, 2).contiguous()
        yb = moe.moe_gemm_down(x.repeat(n, 1), to_dev(_offsets([T] * n)), blocks)
        side = torch.cat([yb[e * T:(e + 1) * T] for e in range(n)], dim=1)
        torch.cuda.synchronize()
        assert torch.equal(side.view(torch.int16), dense.view(torch.int16)), f"{n} column blocks != dense"
    if T * K * N <= 2 ** 31:
        ref = oracle.grouped_projection(bits(x), np.array([0, T], dtype=np.int32), bits(w1))
        say("  " + str(compare_bf16(bits(dense), ref, "dense")))
    else:
        say("  " + str(_check_sampled(x, w1, dense, np.array([0, T]), per_expert=4, seed=3, what="dense")))
