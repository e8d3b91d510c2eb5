"""Backward kernels against the oracle, through the C ABI, on an MI355X.

Dgrad and Wgrad of one grouped projection (OLMo report Sec 9.5, Eq 15 and
Table 15) in both weight layouts, and the atomic-free backward of the two
permutations (halo notes, permute/unpermute paragraphs). bf16 outputs are held
to the step's tolerances (parity.py); the routing-weight gradient, an fp32 dot
product, to a relative bound set by fp32 summation over d terms.
"""

import numpy as np
import pytest
import torch

import oracle
import ragged_grouped_gemm_histogram_amd as moe
from gpu_util import DeviceInputs, bits, say, to_dev, to_dev_bf16
from parity import compare_bf16
from workloads import make_random, make_workload, to_bf16_bits

pytestmark = pytest.mark.gpu


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))]).astype(np.int32)


def _case(seed, counts, d_in, d_out, extra_rows=8, x_sigma=1.0, w_sigma=0.05):
    rng = np.random.default_rng(seed)
    M = sum(counts)
    x = to_bf16_bits(x_sigma * rng.standard_normal((M + extra_rows, d_in), dtype=np.float32))
    dy = to_bf16_bits(rng.standard_normal((M + extra_rows, d_out), dtype=np.float32))
    w = to_bf16_bits(w_sigma * rng.standard_normal((len(counts), d_in, d_out), dtype=np.float32))
    return x, dy, w, _offsets(counts)


CASES = [
    # counts, d_in, d_out
    ([0, 37, 300, 1, 129, 0, 513], 320, 576),      # ragged, empty experts, 128-row forward tiles
    ([700, 900, 420], 6656, 256),                   # 256-row forward tiles (Dgrad), tails in every expert's last stage
    ([5, 0, 260, 77], 328, 200),                    # widths not multiples of 64
    ([1], 64, 64),                                  # one row
    ([64, 128, 65, 63], 264, 136),                  # contraction lengths at and around one stage
    ([3000] * 3 + [0] * 2 + [17], 512, 768),        # many stages per expert, several output tiles
    ([9000, 0, 4097, 4096, 8192, 3], 256, 264),     # Wgrad splits experts above 4096 rows into chunks
]
IDS = ["ragged", "big", "k-tail", "one-row", "stage-edges", "deep", "split-rows"]


@pytest.mark.parametrize("layout", ["in_out", "out_in"])
@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_dgrad_whole(case, layout):
    counts, d_in, d_out = case
    say(f"[gpu] dgrad {layout} counts={counts[:8]} d_in={d_in} d_out={d_out}")
    x, dy, w, offs = _case(sum(counts) + d_in, counts, d_in, d_out)
    w_l = w if layout == "in_out" else np.ascontiguousarray(np.swapaxes(w, 1, 2))
    M = sum(counts)
    sentinel = torch.full((M + 8, d_in), 3.0, dtype=torch.bfloat16, device="cuda:0")
    dx = moe.moe_grouped_dgrad(to_dev_bf16(dy), to_dev(offs), to_dev_bf16(w_l), layout, dx=sentinel)
    torch.cuda.synchronize()
    say("  " + str(compare_bf16(bits(dx)[:M], oracle.grouped_dgrad(dy, offs, w_l, layout), "dx")))
    assert (bits(dx)[M:] == bits(torch.tensor(3.0, dtype=torch.bfloat16))).all(), "rows past M were written"


@pytest.mark.parametrize("layout", ["in_out", "out_in"])
@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_wgrad_whole(case, layout):
    counts, d_in, d_out = case
    say(f"[gpu] wgrad {layout} counts={counts[:8]} d_in={d_in} d_out={d_out}")
    x, dy, w, offs = _case(sum(counts) + d_out, counts, d_in, d_out)
    dw = moe.moe_grouped_wgrad(to_dev_bf16(x), to_dev_bf16(dy), to_dev(offs), layout)
    torch.cuda.synchronize()
    ref = oracle.grouped_wgrad(x, dy, offs, layout)
    got = bits(dw)
    for e, c in enumerate(counts):  # experts with no rows: exact zeros
        if c == 0:
            assert (got[e] == 0).all(), f"expert {e} has no rows but a non-zero gradient"
    say("  " + str(compare_bf16(got, ref, "dw")))


def test_wgrad_empty_capacity_writes_zeros():
    say("[gpu] wgrad with no rows at all")
    E, d_in, d_out = 3, 64, 128
    dw = torch.full((E, d_in, d_out), 5.0, dtype=torch.bfloat16, device="cuda:0")
    x = torch.empty((0, d_in), dtype=torch.bfloat16, device="cuda:0")
    dy = torch.empty((0, d_out), dtype=torch.bfloat16, device="cuda:0")
    moe.moe_grouped_wgrad(x, dy, torch.zeros(E + 1, dtype=torch.int32, device="cuda:0"), dw=dw)
    torch.cuda.synchronize()
    assert (bits(dw) == 0).all()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["zipf64", "qwen3_30b", "square"])
def test_backward_at_expert_shapes(name):
    """The backward GEMMs of a named expert step at full size (zipf64: 64 experts, d = 2048, h = 768,
    65,536 rows, experts above the Wgrad split; Qwen3-shaped: 128 experts of about 256 rows;
    square: d = h = 2880): Dgrad and Wgrad of the down projection ([E, h, d]) and of the gate/up
    projection ([E, 2h, d]), checked on sampled rows of every output against the oracle."""
    wl = make_workload(name)
    di = DeviceInputs(wl)
    y, p, h_buf, y_perm = moe.moe_expert_forward(di.x, di.ids, di.w, di.w_ug, di.w_down, fused_gather=False)
    M = int(p.offsets[-1].item())
    offs = p.offsets.cpu().numpy()
    rng = np.random.default_rng(5)
    g_y = torch.from_numpy(to_bf16_bits(rng.standard_normal((wl.S, wl.d), dtype=np.float32)).view(np.int16)).view(
        torch.bfloat16).to("cuda:0")
    g_u = torch.from_numpy(to_bf16_bits(rng.standard_normal((wl.S, 2 * wl.h), dtype=np.float32)).view(np.int16)).view(
        torch.bfloat16).to("cuda:0")
    say(f"[gpu] {name} down projection: Dgrad (h <- d) and Wgrad [E, h, d]")
    dh = moe.moe_grouped_dgrad(g_y, p.offsets, di.w_down, "in_out")
    dwd = moe.moe_grouped_wgrad(h_buf, g_y, p.offsets, "in_out")
    say(f"[gpu] {name} gate/up projection: Dgrad (d <- 2h) and Wgrad [E, 2h, d]")
    dx = moe.moe_grouped_dgrad(g_u, p.offsets, di.w_ug, "out_in")
    dwu = moe.moe_grouped_wgrad(p.x_perm, g_u, p.offsets, "out_in")
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([rng.integers(offs[e], offs[e + 1], size=2) for e in range(wl.E)
                                     if offs[e + 1] > offs[e]] + [np.array([0, M - 1])]))
    e_of = np.searchsorted(offs, rows, side="right") - 1
    gy, gu = bits(g_y), bits(g_u)

    def dgrad_rows(g, w_bits, layout, out):
        ref = np.concatenate([oracle.grouped_dgrad(g[r:r + 1], np.array([0, 1]), w_bits[e:e + 1], layout)
                              for r, e in zip(rows, e_of)])
        return compare_bf16(bits(out)[rows], ref, "dx rows")

    say("  down Dgrad " + str(dgrad_rows(gy, wl.w_down, "in_out", dh)))
    say("  gate/up Dgrad " + str(dgrad_rows(gu, wl.w_ug, "out_in", dx)))
    # Wgrad: two output rows of every non-empty expert's gradient, each a contraction over its rows
    hb, xb = bits(h_buf), bits(p.x_perm)
    got_d, ref_d, got_u, ref_u = [], [], [], []
    for e in range(wl.E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            assert (bits(dwd[e]) == 0).all() and (bits(dwu[e]) == 0).all()
            continue
        sub = np.array([0, hi - lo], dtype=np.int32)
        i_d = rng.integers(0, wl.h, size=2)
        ref = oracle.grouped_wgrad(hb[lo:hi][:, i_d], gy[lo:hi], sub, "in_out")[0]  # rows i_d of dW_down[e]
        ref_d.append(ref)
        got_d.append(bits(dwd[e])[i_d])
        i_u = rng.integers(0, 2 * wl.h, size=2)
        ref = oracle.grouped_wgrad(xb[lo:hi], gu[lo:hi][:, i_u], sub, "out_in")[0]  # rows i_u of dW_ug[e]
        ref_u.append(ref)
        got_u.append(bits(dwu[e])[i_u])
    say("  down Wgrad " + str(compare_bf16(np.concatenate(got_d), np.concatenate(ref_d), "dW_down rows")))
    say("  gate/up Wgrad " + str(compare_bf16(np.concatenate(got_u), np.concatenate(ref_u), "dW_ug rows")))


@pytest.mark.parametrize("name", ["edge", "square"])
def test_permutation_backward_named(name):
    _check_permutation_backward(make_workload(name), seed=11)


@pytest.mark.parametrize("case", [
    dict(T=300, k=3, E=5, d=200, h=8, seed=1, drop_frac=0.3),
    dict(T=33, k=2, E=6, d=64, h=8, seed=6, drop_frac=1.0),
    dict(T=1, k=1, E=1, d=8, h=8, seed=2, drop_frac=0.0),
    dict(T=2000, k=4, E=16, d=2056, h=8, seed=3, drop_frac=0.1),
    dict(T=4096, k=8, E=128, d=2048, h=8, seed=4, drop_frac=0.05),
], ids=["ragged", "all-dropped", "one-token", "wide", "qwen3-shaped"])
def test_permutation_backward_random(case):
    _check_permutation_backward(make_random(**case), seed=12)


def _check_permutation_backward(wl, seed):
    say(f"[gpu] permutation backward {wl.name} T={wl.T} k={wl.k} d={wl.d}")
    ref = oracle.moe_expert_forward(wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down, with_gemm=False)
    M, T, k, d = ref.M, wl.T, wl.k, wl.d
    rng = np.random.default_rng(seed)
    S = T * k
    g_perm = to_bf16_bits(rng.standard_normal((S, d), dtype=np.float32))
    y_perm = to_bf16_bits(rng.standard_normal((S, d), dtype=np.float32))
    dy = to_bf16_bits(rng.standard_normal((T, d), dtype=np.float32))
    inv = to_dev(ref.inv_map.astype(np.int32))
    dx = moe.moe_permute_backward(to_dev_bf16(g_perm), inv)
    sentinel = torch.full((S, d), 7.0, dtype=torch.bfloat16, device="cuda:0")
    dyp, dw = moe.moe_unpermute_backward(to_dev_bf16(dy), to_dev_bf16(y_perm), inv,
                                         to_dev(wl.routing_w.astype(np.float32)), dy_perm=sentinel)
    torch.cuda.synchronize()
    say("  dx " + str(compare_bf16(bits(dx), oracle.permute_backward(g_perm[:M], ref.inv_map, T, k), "dx")))
    ref_dyp, ref_dw = oracle.unpermute_backward(dy, y_perm[:M], ref.inv_map, wl.routing_w, T, k, M)
    say("  dy_perm " + str(compare_bf16(bits(dyp)[:M], ref_dyp, "dy_perm")))
    assert (bits(dyp)[M:] == bits(torch.tensor(7.0, dtype=torch.bfloat16))).all(), "rows past M were written"
    got_dw = dw.cpu().numpy()
    # fp32 dot product of d bf16 pairs: per-lane sums of d/64 terms, then a 6-level tree, so
    # |error| <= (d/64 + 6) * 2^-24 * sum_c |dy * y_perm|; the bound below is 4x that
    inv = ref.inv_map
    keep = inv >= 0
    abs_sum = np.zeros((T, k))
    dyf, ypf = np.abs(oracle.bf16_bits_to_f64(dy)), np.abs(oracle.bf16_bits_to_f64(y_perm[:M]))
    for j in range(k):
        abs_sum[keep[:, j], j] = np.sum(dyf[keep[:, j]] * ypf[inv[keep[:, j], j]], axis=1)
    bound = 4 * (d / 64 + 6) * 2.0**-24 * abs_sum
    err = np.abs(got_dw.astype(np.float64) - ref_dw.astype(np.float64))
    assert np.all(err <= bound + 1e-30), f"routing-weight gradient off by {err.max()} (bound {bound.max()})"
    assert np.all(got_dw[~keep] == 0.0)


@pytest.mark.parametrize("layout", ["in_out", "out_in"])
@pytest.mark.parametrize("case", CASES[:4], ids=IDS[:4])
def test_projection_layouts(case, layout):
    counts, d_in, d_out = case
    say(f"[gpu] projection {layout} counts={counts[:8]} d_in={d_in} d_out={d_out}")
    x, dy, w, offs = _case(sum(counts) + 3 * d_in, counts, d_in, d_out)
    w_l = w if layout == "in_out" else np.ascontiguousarray(np.swapaxes(w, 1, 2))
    y = moe.moe_grouped_projection(to_dev_bf16(x), to_dev(offs), to_dev_bf16(w_l), layout)
    torch.cuda.synchronize()
    M = sum(counts)
    say("  " + str(compare_bf16(bits(y)[:M], oracle.grouped_projection(x, offs, w), "y")))


@pytest.mark.parametrize("counts,h", [([0, 37, 300, 1, 129, 0, 513], 384), ([5], 8), ([2000, 3000], 768)],
                         ids=["ragged", "one-chunk", "wide"])
def test_swiglu_backward(counts, h):
    say(f"[gpu] SwiGLU backward counts={counts} h={h}")
    rng = np.random.default_rng(len(counts) + h)
    M = sum(counts)
    u = to_bf16_bits(2.0 * rng.standard_normal((M + 4, 2 * h), dtype=np.float32))
    dh = to_bf16_bits(rng.standard_normal((M + 4, h), dtype=np.float32))
    sentinel = torch.full((M + 4, 2 * h), 9.0, dtype=torch.bfloat16, device="cuda:0")
    du = moe.moe_swiglu_backward(to_dev_bf16(dh), to_dev_bf16(u), to_dev(_offsets(counts)), du=sentinel)
    torch.cuda.synchronize()
    say("  " + str(compare_bf16(bits(du)[:M], oracle.swiglu_backward(dh[:M], u[:M]), "du")))
    assert (bits(du)[M:] == bits(torch.tensor(9.0, dtype=torch.bfloat16))).all(), "rows past M were written"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", [
    dict(T=1500, k=4, E=12, d=320, h=256, seed=31, drop_frac=0.1, empty_experts=(4,), x_sigma=1.0, w_sigma=0.05),
    dict(T=700, k=2, E=3, d=136, h=72, seed=32, drop_frac=0.0, x_sigma=1.0, w_sigma=0.1),
], ids=["ragged", "k-tails"])
def test_expert_backward_chain(case):
    """The whole expert backward through the library's calls against the oracle's composed backward.

    Chained results (dU, dX, dW) are held to the data-scaled guards only: the oracle's own chain
    evaluated in float32 (the kernels' accumulation precision) already puts 13 of 2M gate/up
    Wgrad elements outside the elementwise bound, because a bf16 rounding of dU decided one ulp
    apart is multiplied by x in the contraction; each kernel is held to the elementwise bound on
    its own in the tests above."""
    wl = make_random(**case)
    say(f"[gpu] expert backward T={wl.T} k={wl.k} E={wl.E} d={wl.d} h={wl.h}")
    di = DeviceInputs(wl)
    y, p, h_buf, y_perm = moe.moe_expert_forward(di.x, di.ids, di.w, di.w_ug, di.w_down)
    rng = np.random.default_rng(case["seed"])
    dy = to_bf16_bits(rng.standard_normal((wl.T, wl.d), dtype=np.float32))
    got = moe.moe_expert_backward(to_dev_bf16(dy), p, di.w, di.w_ug, di.w_down, h_buf, y_perm)
    torch.cuda.synchronize()
    ref = oracle.expert_backward(dy, wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down)
    M = int(ref["offsets"][-1])
    say("  dx " + str(compare_bf16(bits(got["dx"]), ref["dx"], "dx", elementwise=False)))
    say("  dw_ug " + str(compare_bf16(bits(got["dw_ug"]), ref["dw_ug"], "dw_ug", elementwise=False)))
    say("  dw_down " + str(compare_bf16(bits(got["dw_down"]), ref["dw_down"], "dw_down", elementwise=False)))
    say("  du " + str(compare_bf16(bits(got["du"])[:M], ref["du"], "du", elementwise=False)))
    g_rw, r_rw = got["d_routing_w"].cpu().numpy().astype(np.float64), ref["d_routing_w"].astype(np.float64)
    assert np.linalg.norm(g_rw - r_rw) <= 1e-2 * np.linalg.norm(r_rw)
