"""Pins that tie the oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
something the pages print, a closed form, a textbook/library routine applied
to a special case, brute force on a tiny input, or an exact invariance. The
functions take the oracle package as an argument so the mutation tests can run
them against an oracle with a planted mistake and see them fail.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from workloads import make_random, make_workload, to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "toy_figs35_37.json")


def golden() -> dict:
    with open(GOLDEN) as f:
        return json.load(f)


def _bits_to_f64(b):
    return torch.from_numpy(np.asarray(b, dtype=np.uint16).view(np.int16).copy()).view(torch.bfloat16).double()


def _torch_bf16_bits(t64: torch.Tensor) -> np.ndarray:
    """Library rounding for the independent references: float64 -> float32 -> bfloat16 (torch)."""
    return t64.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _ulps(a, b):
    a = np.asarray(a, dtype=np.uint16).astype(np.int64)
    b = np.asarray(b, dtype=np.uint16).astype(np.int64)
    oa = np.where(a & 0x8000, -(a & 0x7FFF), a & 0x7FFF)
    ob = np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(oa - ob)


def _assert_close_bits(got, ref, what, min_exact=0.99, max_ulp=1):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    u = _ulps(got, ref)
    exact = float(np.mean(u == 0)) if u.size else 1.0
    assert exact >= min_exact, f"{what}: only {exact:.4f} of elements bit-identical"
    assert (u.max() if u.size else 0) <= max_ulp, f"{what}: max ulp difference {u.max()}"


# ---------------------------------------------------------------- printed toy


def pin_toy_golden(orc) -> None:
    """Figs 35-37: rows (1,4,3,2) -> offsets [1,5,8,10], C=4, rho=0.375, 16 rows, 12 tiles."""
    g = golden()["toy"]
    wl = make_workload("toy")
    counts = orc.route_histogram(wl.expert_ids, wl.E)
    assert counts.tolist() == g["rows_per_expert"]
    offsets = orc.exclusive_offsets(counts)
    assert offsets[0] == 0 and offsets[1:].tolist() == g["cumulative_offsets_inclusive"]
    M = int(offsets[-1])
    assert M == g["routed_rows_M"]
    assert M / wl.E == g["mean_load"]
    C = orc.capacity_ceil(g["capacity_factor"], M, wl.E)
    assert C == g["capacity_C"]
    assert wl.E * C == g["rows_multiplied_padded"]
    assert wl.E * C - M == g["padding_rows"]
    assert orc.padding_fraction(counts, C) == g["padding_fraction"]
    slices = [[int(offsets[e]), int(offsets[e + 1])] for e in range(wl.E)]
    assert slices == g["problem_row_slices"]
    assert orc.tile_count(counts, g["tile_rows"], g["tile_col_blocks"]) == g["tiles"]
    perm, inv = orc.stable_route_order(wl.expert_ids, wl.E, offsets)
    assert sorted(inv.tolist()) == list(range(*g["computed_rows"]))
    # every sorted row carries its own expert's id
    flat = wl.expert_ids.reshape(-1)
    for e, (lo, hi) in enumerate(slices):
        assert all(flat[perm[p]] == e for p in range(lo, hi))


def pin_printed_arithmetic(orc) -> None:
    """Fig 38 / Fig 39 / Sec 9.6 numbers recomputed from the FLOP convention and Eq 14."""
    gd = golden()
    f = gd["fig38"]
    # One projection of a gated expert is a third of 6*M*d*h (two FLOPs per multiply-add).
    proj = orc.useful_flops(f["M"], f["d"], f["h"]) // 3
    assert proj == 2 * f["M"] * f["d"] * f["h"]
    lo_t, hi_t = f["grouped_ms"] - 5e-4, f["grouped_ms"] + 5e-4  # printed to 3 decimals
    assert proj / (hi_t * 1e-3) / 1e12 <= f["grouped_tflops"] <= proj / (lo_t * 1e-3) / 1e12
    lo_b, hi_b = f["bmm_ms"] - 5e-4, f["bmm_ms"] + 5e-4
    assert proj / (hi_b * 1e-3) / 1e12 <= f["bmm_useful_tflops"] + 0.5
    assert f["bmm_useful_tflops"] - 0.5 <= proj / (lo_b * 1e-3) / 1e12
    C = orc.capacity_ceil(1.25, f["M"], f["experts"])
    assert C == f["bmm_capacity_C"] and f["experts"] * C == f["bmm_rows"]
    padded = 2 * f["bmm_rows"] * f["d"] * f["h"]
    assert padded / (hi_b * 1e-3) / 1e12 <= f["bmm_padded_tflops"] + 0.5
    assert f["bmm_padded_tflops"] - 0.5 <= padded / (lo_b * 1e-3) / 1e12
    counts = np.full(f["experts"], f["rows_per_expert"])
    assert orc.padding_fraction(counts, C) == gd["sec96_capacity"]["padding_fraction_balanced"]
    f39 = gd["fig39"]
    assert round(2 * f39["T"] * f39["K"] * f39["N"] / 1e12, 2) == f39["tflop_rounded"]
    # Eq 16 on the toy with one EP rank: 8 * ceil(floor(1.25 * 2.5) / 8) = 8 (derived)
    assert orc.capacity_eq16(1.25, 2.5, 1) == 8
    assert orc.capacity_eq16(1.25, 512, 1) == 640
    # Eq 16 with several EP ranks, evaluated by hand. Two ranks, Mbar = 103.2: each rank's share
    # floor(1.25 * 103.2 / 2) = floor(64.5) = 64 rows, already a multiple of 8, so C = 2 * 8 * 8 = 128
    # (a ceiling in place of the floor gives 2 * 8 * ceil(65 / 8) = 144; aligning the undivided
    # floor(129) gives 2 * 8 * 17 = 272; dropping the factor M_E gives 64).
    assert orc.capacity_eq16(1.25, 103.2, 2) == 128
    # Eight ranks, Mbar = 100: floor(15.625) = 15 rows per rank, aligned up to 16: C = 8 * 16 = 128.
    assert orc.capacity_eq16(1.25, 100, 8) == 128
    # One rank, a share that is not a multiple of 8: floor(1.25 * 13.6) = 17 -> 8 * ceil(17 / 8) = 24
    # (the ceiling slip gives ceil(17.0) = 17 too, so this case checks the alignment step alone).
    assert orc.capacity_eq16(1.25, 13.6, 1) == 24
    e18 = gd["eq18"]
    assert orc.entropy_deficit(np.full(16, 7)) == e18["uniform"]
    assert abs(orc.entropy_deficit(np.eye(16, dtype=int)[3] * 99) - e18["single_expert"]) < 1e-15


# ------------------------------------------------------------ library routines


def pin_histogram_and_order(orc, seeds=(0, 1, 2)) -> None:
    """counts = numpy.bincount, offsets = [0, cumsum], perm = stable argsort (library routines)."""
    for seed in seeds:
        wl = make_random(T=97, k=3, E=7, d=8, h=8, seed=seed, drop_frac=0.2)
        flat = wl.expert_ids.reshape(-1).astype(np.int64)
        valid = (flat >= 0) & (flat < wl.E)
        counts = orc.route_histogram(wl.expert_ids, wl.E)
        np.testing.assert_array_equal(counts, np.bincount(flat[valid], minlength=wl.E))
        offsets = orc.exclusive_offsets(counts)
        np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
        perm, inv = orc.stable_route_order(wl.expert_ids, wl.E, offsets)
        slots = np.flatnonzero(valid)
        order = slots[np.argsort(flat[valid], kind="stable")]
        M = int(valid.sum())
        np.testing.assert_array_equal(perm[:M], order)
        assert np.all(inv[~valid] == -1)
        assert np.all(perm[inv[valid]] == slots)
        assert sorted(inv[valid].tolist()) == list(range(M))


def pin_permute_unpermute_identity(orc) -> None:
    """Unpermute(permute(X)) = X: bit-exact at k=1, w=1; and at k>1 when the weights sum to 1."""
    wl = make_random(T=64, k=1, E=5, d=24, h=8, seed=11, drop_frac=0.15)
    wl.routing_w[:] = 1.0
    r = orc.moe_expert_forward(wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down, with_gemm=False)
    y = orc.unpermute(r.x_perm, r.inv_map, wl.routing_w, wl.T, wl.k)
    kept = (r.inv_map[:, 0] >= 0)
    np.testing.assert_array_equal(y[kept], wl.x[kept])
    assert np.all(y[~kept] == 0)
    wl = make_random(T=64, k=4, E=5, d=24, h=8, seed=12, drop_frac=0.0)  # softmax weights, sum 1
    r = orc.moe_expert_forward(wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down, with_gemm=False)
    y = orc.unpermute(r.x_perm, r.inv_map, wl.routing_w, wl.T, wl.k)
    np.testing.assert_array_equal(y, wl.x)


def _dense_swiglu_torch(x_bits, wg_bits, wu_bits, wd_bits):
    """A dense SwiGLU MLP through torch library ops in float64, bf16-rounded (torch) at the
    points the method stores bf16: U, H, Y."""
    x = _bits_to_f64(x_bits)
    g = _bits_to_f64(_torch_bf16_bits(F.linear(x, _bits_to_f64(wg_bits))))
    u = _bits_to_f64(_torch_bf16_bits(F.linear(x, _bits_to_f64(wu_bits))))
    hid = _bits_to_f64(_torch_bf16_bits(F.silu(g) * u))
    return _torch_bf16_bits(hid @ _bits_to_f64(wd_bits))


def pin_single_expert_is_dense_mlp(orc) -> None:
    """E = 1 with k = 1 and w = 1: the expert step is a dense SwiGLU MLP (torch F.linear / F.silu)."""
    rng = np.random.default_rng(5)
    T, d, h = 48, 40, 24  # d != h and d != 2h so a transposed operand cannot pass
    x = to_bf16_bits(rng.standard_normal((T, d), dtype=np.float32))
    w_ug = to_bf16_bits(0.2 * rng.standard_normal((1, 2 * h, d), dtype=np.float32))
    w_dn = to_bf16_bits(0.2 * rng.standard_normal((1, h, d), dtype=np.float32))
    ids = np.zeros((T, 1), dtype=np.int32)
    w = np.ones((T, 1), dtype=np.float32)
    r = orc.moe_expert_forward(x, ids, w, w_ug, w_dn)
    ref = _dense_swiglu_torch(x, w_ug[0, :h], w_ug[0, h:], w_dn[0])
    _assert_close_bits(r.y, ref, "E=1 dense SwiGLU", min_exact=0.99, max_ulp=1)


def pin_column_partition(orc) -> None:
    """Eq 17: with every token on every expert and w = 1, the experts are column blocks of one
    dense SwiGLU MLP of hidden width E*h (gate blocks, up blocks and down blocks concatenated)."""
    rng = np.random.default_rng(9)
    T, E, d, h = 20, 3, 32, 16
    x = to_bf16_bits(rng.standard_normal((T, d), dtype=np.float32))
    w_ug = to_bf16_bits(0.2 * rng.standard_normal((E, 2 * h, d), dtype=np.float32))
    w_dn = to_bf16_bits(0.2 * rng.standard_normal((E, h, d), dtype=np.float32))
    ids = np.tile(np.arange(E, dtype=np.int32), (T, 1))
    w = np.ones((T, E), dtype=np.float32)
    r = orc.moe_expert_forward(x, ids, w, w_ug, w_dn)
    wg = np.concatenate([w_ug[e, :h] for e in range(E)], axis=0)  # [E*h, d]
    wu = np.concatenate([w_ug[e, h:] for e in range(E)], axis=0)
    wd = np.concatenate([w_dn[e] for e in range(E)], axis=0)  # [E*h, d]
    xt = _bits_to_f64(x)
    g = _bits_to_f64(_torch_bf16_bits(F.linear(xt, _bits_to_f64(wg))))
    u = _bits_to_f64(_torch_bf16_bits(F.linear(xt, _bits_to_f64(wu))))
    hid = _bits_to_f64(_torch_bf16_bits(F.silu(g) * u))
    dense = (hid @ _bits_to_f64(wd)).numpy()  # unrounded dense result
    got = _bits_to_f64(r.y).numpy()
    # the grouped form rounds each expert's Y_e to bf16 before the sum: E half-ulps of |Y_e|
    tol = (E + 1) * 2.0**-8 * np.abs(dense).max()
    assert np.max(np.abs(got - dense)) <= tol, f"Eq 17 partition off by {np.max(np.abs(got - dense))}"
    assert np.linalg.norm(got - dense) <= 2.0**-7 * np.linalg.norm(dense)


def pin_brute_force(orc) -> None:
    """Pure-Python loops over every index of Eq 13 and the weighted scatter-back on a tiny case."""
    T, k, E, d, h = 7, 2, 3, 8, 8  # d == h: a transposed weight would still type-check here
    wl = make_random(T=T, k=k, E=E, d=d, h=h, seed=21, drop_frac=0.2, w_sigma=0.3)
    r = orc.moe_expert_forward(wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down)
    xv = _bits_to_f64(wl.x).tolist()
    wug = _bits_to_f64(wl.w_ug).tolist()
    wdn = _bits_to_f64(wl.w_down).tolist()

    def rb(v):  # torch's float32 -> bfloat16 rounding, one scalar
        return float(torch.tensor(v, dtype=torch.float64).float().to(torch.bfloat16).double())

    ref = np.zeros((T, d), dtype=np.uint16)
    for t in range(T):
        acc = [0.0] * d
        for j in range(k):
            e = int(wl.expert_ids[t, j])
            if not 0 <= e < E:
                continue
            U = [rb(sum(xv[t][c] * wug[e][n][c] for c in range(d))) for n in range(2 * h)]
            H = [rb(U[n] / (1.0 + math.exp(-U[n])) * U[h + n]) for n in range(h)]
            Y = [rb(sum(H[n] * wdn[e][n][c] for n in range(h))) for c in range(d)]
            wj = float(wl.routing_w[t, j])
            acc = [acc[c] + wj * Y[c] for c in range(d)]
        ref[t] = _torch_bf16_bits(torch.tensor(acc, dtype=torch.float64))
    _assert_close_bits(r.y, ref, "brute force", min_exact=0.97, max_ulp=1)


def pin_invariances(orc) -> None:
    """Exact invariances: w -> 2w doubles y; relabeling experts (with their weights), adding an
    empty expert, or shuffling tokens (with ids and weights) leaves every token's y unchanged."""
    wl = make_random(T=40, k=3, E=6, d=32, h=16, seed=31, drop_frac=0.1, w_sigma=0.2)
    base = orc.moe_expert_forward(wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down)
    ref = _bits_to_f64(base.y).numpy()
    r2 = orc.moe_expert_forward(wl.x, wl.expert_ids, 2 * wl.routing_w, wl.w_ug, wl.w_down)
    np.testing.assert_array_equal(_bits_to_f64(r2.y).numpy(), 2 * ref)
    rng = np.random.default_rng(3)
    relabel = rng.permutation(wl.E)  # old id -> new id
    ids = wl.expert_ids.copy()
    valid = (ids >= 0) & (ids < wl.E)
    ids[valid] = relabel[ids[valid]]
    inv_label = np.argsort(relabel)
    r3 = orc.moe_expert_forward(wl.x, ids, wl.routing_w, wl.w_ug[inv_label], wl.w_down[inv_label])
    np.testing.assert_array_equal(r3.y, base.y)
    extra_ug = np.concatenate([wl.w_ug, to_bf16_bits(rng.standard_normal((1,) + wl.w_ug.shape[1:],
                                                                          dtype=np.float32))])
    extra_dn = np.concatenate([wl.w_down, to_bf16_bits(rng.standard_normal((1,) + wl.w_down.shape[1:],
                                                                           dtype=np.float32))])
    ids4 = wl.expert_ids.copy()
    ids4[ids4 == wl.E] = -1  # with E+1 experts, an id equal to the old E would become valid
    r4 = orc.moe_expert_forward(wl.x, ids4, wl.routing_w, extra_ug, extra_dn)
    np.testing.assert_array_equal(r4.y, base.y)
    sh = rng.permutation(wl.T)
    r5 = orc.moe_expert_forward(wl.x[sh], wl.expert_ids[sh], wl.routing_w[sh], wl.w_ug, wl.w_down)
    np.testing.assert_array_equal(r5.y, base.y[sh])


def pin_f32_within_bound(orc) -> None:
    """The float32 loop (the precision the method names for accumulation) and the float64 loop
    round to the same bf16 values, except where a value lies within the float32 error bound
    K*2^-24*sum|a_i b_i| of a rounding boundary: there U differs by one ulp, and H = SiLU(g)*u,
    fed by two such U values, by at most two."""
    wl = make_random(T=64, k=2, E=4, d=256, h=128, seed=41, drop_frac=0.05, w_sigma=0.05)
    r64 = orc.moe_expert_forward(wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down, precision="f64")
    r32 = orc.moe_expert_forward(wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down, precision="f32")
    for name in ("h", "y_perm", "y"):
        _assert_close_bits(getattr(r32, name), getattr(r64, name), f"f32 vs f64 {name}", min_exact=0.97, max_ulp=2)


def pin_token_form(orc) -> None:
    """The per-token form used for sampled checks equals the per-expert loop."""
    wl = make_random(T=30, k=3, E=5, d=48, h=32, seed=51, drop_frac=0.1, w_sigma=0.1)
    r = orc.moe_expert_forward(wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down)
    rows = np.stack([orc.token_forward(wl.x[t], wl.expert_ids[t], wl.routing_w[t], wl.w_ug, wl.w_down)
                     for t in range(wl.T)])
    _assert_close_bits(rows, r.y, "token form", min_exact=0.99, max_ulp=1)


def pin_projection_column_partition(orc) -> None:
    """Eq 17 for one projection: the experts' weights are column blocks of one dense weight and
    every expert multiplies the same rows, so the grouped outputs, laid side by side, are the
    dense product (torch float64 matmul, torch bf16 rounding)."""
    rng = np.random.default_rng(13)
    T, K, N, E = 24, 40, 48, 4  # K != N / E: a transposed block cannot type-check
    x = to_bf16_bits(rng.standard_normal((T, K), dtype=np.float32))
    w = to_bf16_bits(0.2 * rng.standard_normal((K, N), dtype=np.float32))
    nb = N // E
    blocks = np.stack([w[:, e * nb:(e + 1) * nb] for e in range(E)])  # [E, K, N/E]
    a = np.concatenate([x] * E, axis=0)  # the input repeated once per expert
    offsets = np.arange(E + 1, dtype=np.int32) * T
    got = orc.grouped_projection(a, offsets, blocks)
    side = np.concatenate([got[e * T:(e + 1) * T] for e in range(E)], axis=1)  # [T, N]
    dense = _torch_bf16_bits(_bits_to_f64(x) @ _bits_to_f64(w))
    _assert_close_bits(side, dense, "Eq 17 projection partition", min_exact=0.999, max_ulp=1)


def pin_projection_brute_force(orc) -> None:
    """Pure-Python loops over every output of a ragged grouped projection with an empty expert."""
    rng = np.random.default_rng(17)
    K, N = 6, 10
    counts = [3, 0, 5, 1]
    E = len(counts)
    M = sum(counts)
    a = to_bf16_bits(rng.standard_normal((M + 2, K), dtype=np.float32))  # two rows past M stay unused
    w = to_bf16_bits(rng.standard_normal((E, K, N), dtype=np.float32))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    got = orc.grouped_projection(a, offsets, w)
    av = _bits_to_f64(a).tolist()
    wv = _bits_to_f64(w).tolist()
    ref = np.zeros((M, N), dtype=np.uint16)
    row = 0
    for e, c in enumerate(counts):
        for _ in range(c):
            vals = [sum(av[row][q] * wv[e][q][n] for q in range(K)) for n in range(N)]
            ref[row] = _torch_bf16_bits(torch.tensor(vals, dtype=torch.float64))
            row += 1
    _assert_close_bits(got, ref, "projection brute force", min_exact=1.0, max_ulp=0)


def pin_projection_is_down_step(orc) -> None:
    """The down projection inside the expert step is the grouped projection of H (same rows,
    same weights, one bf16 rounding)."""
    wl = make_random(T=30, k=2, E=5, d=48, h=32, seed=61, drop_frac=0.1, w_sigma=0.1, empty_experts=(3,))
    r = orc.moe_expert_forward(wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down)
    y = orc.grouped_projection(r.h, r.offsets, wl.w_down)
    np.testing.assert_array_equal(y, r.y_perm)


def _ragged_projection_case(seed, counts, d_in, d_out):
    rng = np.random.default_rng(seed)
    M = sum(counts)
    x = to_bf16_bits(rng.standard_normal((M, d_in), dtype=np.float32))
    dy = to_bf16_bits(rng.standard_normal((M, d_out), dtype=np.float32))
    w = to_bf16_bits(0.2 * rng.standard_normal((len(counts), d_in, d_out), dtype=np.float32))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return x, dy, w, offsets


def pin_backward_is_autograd(orc) -> None:
    """Eq 15 through torch autograd: a per-expert loop Y_e = X_e W_e (and Y_e = X_e W_e^T for the
    [E, d_out, d_in] layout) in float64, differentiated by autograd against a fixed dY, gives the
    oracle's Dgrad and Wgrad (torch bf16 rounding of autograd's float64 sums)."""
    counts = [5, 0, 9, 1, 3]
    d_in, d_out = 12, 20  # d_in != d_out: a missing transpose cannot type-check
    x, dy, w, offsets = _ragged_projection_case(71, counts, d_in, d_out)
    for layout in ("in_out", "out_in"):
        w_l = w if layout == "in_out" else np.ascontiguousarray(np.swapaxes(w, 1, 2))
        xt = _bits_to_f64(x).requires_grad_(True)
        wt = _bits_to_f64(w_l).requires_grad_(True)
        ys = []
        for e in range(len(counts)):
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            we = wt[e] if layout == "in_out" else wt[e].T
            ys.append(xt[lo:hi] @ we)
        y = torch.cat(ys)
        (y * _bits_to_f64(dy)).sum().backward()
        _assert_close_bits(orc.grouped_dgrad(dy, offsets, w_l, layout), _torch_bf16_bits(xt.grad.detach()),
                           f"Dgrad {layout}", min_exact=0.999, max_ulp=1)
        _assert_close_bits(orc.grouped_wgrad(x, dy, offsets, layout), _torch_bf16_bits(wt.grad.detach()),
                           f"Wgrad {layout}", min_exact=0.999, max_ulp=1)


def pin_backward_brute_force(orc) -> None:
    """Pure-Python loops over every element of Dgrad and Wgrad on a ragged case with an empty expert."""
    counts = [2, 0, 3]
    d_in, d_out = 4, 5
    x, dy, w, offsets = _ragged_projection_case(73, counts, d_in, d_out)
    xv, gv, wv = _bits_to_f64(x).tolist(), _bits_to_f64(dy).tolist(), _bits_to_f64(w).tolist()
    ref_dx = np.zeros((sum(counts), d_in), dtype=np.uint16)
    ref_dw = np.zeros((len(counts), d_in, d_out), dtype=np.uint16)
    for e in range(len(counts)):
        rows = range(int(offsets[e]), int(offsets[e + 1]))
        for r in rows:
            ref_dx[r] = _torch_bf16_bits(torch.tensor([sum(gv[r][o] * wv[e][i][o] for o in range(d_out))
                                                       for i in range(d_in)], dtype=torch.float64))
        for i in range(d_in):
            ref_dw[e, i] = _torch_bf16_bits(torch.tensor([sum(xv[r][i] * gv[r][o] for r in rows)
                                                          for o in range(d_out)], dtype=torch.float64))
    _assert_close_bits(orc.grouped_dgrad(dy, offsets, w), ref_dx, "Dgrad brute force", min_exact=1.0, max_ulp=0)
    _assert_close_bits(orc.grouped_wgrad(x, dy, offsets), ref_dw, "Wgrad brute force", min_exact=1.0, max_ulp=0)


def pin_permutation_backward_is_autograd(orc) -> None:
    """The two permutations' backward through torch autograd: the row gather X[perm/k] (whose
    autograd backward is a scatter-add) and the weighted gather-sum of the unpermute."""
    wl = make_random(T=25, k=3, E=4, d=16, h=8, seed=81, drop_frac=0.2)
    r = orc.moe_expert_forward(wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down, with_gemm=False)
    M, T, k = r.M, wl.T, wl.k
    rng = np.random.default_rng(82)
    g_perm = to_bf16_bits(rng.standard_normal((M, wl.d), dtype=np.float32))
    xt = _bits_to_f64(wl.x).requires_grad_(True)
    xp = xt[torch.from_numpy(r.perm[:M].astype(np.int64) // k)]
    (xp * _bits_to_f64(g_perm)).sum().backward()
    _assert_close_bits(orc.permute_backward(g_perm, r.inv_map, T, k), _torch_bf16_bits(xt.grad.detach()),
                       "permute backward", min_exact=0.999, max_ulp=1)
    y_perm = to_bf16_bits(rng.standard_normal((M, wl.d), dtype=np.float32))
    dy = to_bf16_bits(rng.standard_normal((T, wl.d), dtype=np.float32))
    ypt = _bits_to_f64(y_perm).requires_grad_(True)
    wt = torch.from_numpy(wl.routing_w.astype(np.float64)).requires_grad_(True)
    inv = torch.from_numpy(r.inv_map.astype(np.int64))
    keep = (inv >= 0).double()
    gathered = ypt[inv.clamp(min=0)] * keep[..., None]  # [T, k, d]
    y = (wt[..., None] * gathered).sum(1)
    (y * _bits_to_f64(dy)).sum().backward()
    dyp, dw = orc.unpermute_backward(dy, y_perm, r.inv_map, wl.routing_w, T, k, M)
    _assert_close_bits(dyp, _torch_bf16_bits(ypt.grad.detach()), "unpermute backward rows", min_exact=1.0, max_ulp=0)
    np.testing.assert_allclose(dw, wt.grad.detach().numpy().astype(np.float32), rtol=1e-6, atol=1e-6)


def pin_swiglu_backward_is_autograd(orc) -> None:
    """The SwiGLU backward equals torch autograd of F.silu(g) * up in float64 on the bf16 U."""
    rng = np.random.default_rng(91)
    M, h = 37, 24
    u = to_bf16_bits(2.0 * rng.standard_normal((M, 2 * h), dtype=np.float32))
    dh = to_bf16_bits(rng.standard_normal((M, h), dtype=np.float32))
    ut = _bits_to_f64(u).requires_grad_(True)
    hid = F.silu(ut[:, :h]) * ut[:, h:]
    (hid * _bits_to_f64(dh)).sum().backward()
    _assert_close_bits(orc.swiglu_backward(dh, u), _torch_bf16_bits(ut.grad.detach()), "SwiGLU backward",
                       min_exact=0.999, max_ulp=1)


def pin_expert_backward_is_autograd(orc) -> None:
    """The composed expert backward against torch autograd of the whole step in float64 (Eq 13 per
    expert, gather, weighted scatter-back), rounding points of the forward taken as identities. The
    oracle rounds U, H, Y and every stored gradient to bf16, so the two agree to bf16 accuracy; a
    wrong sign, transpose, expert or missing term is off by O(1)."""
    wl = make_random(T=24, k=2, E=4, d=16, h=12, seed=93, drop_frac=0.15, w_sigma=0.3, empty_experts=(2,))
    rng = np.random.default_rng(94)
    dy = to_bf16_bits(rng.standard_normal((wl.T, wl.d), dtype=np.float32))
    got = orc.expert_backward(dy, wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down)
    x = _bits_to_f64(wl.x).requires_grad_(True)
    wug = _bits_to_f64(wl.w_ug).requires_grad_(True)
    wdn = _bits_to_f64(wl.w_down).requires_grad_(True)
    rw = torch.from_numpy(wl.routing_w.astype(np.float64)).requires_grad_(True)
    y = torch.zeros((wl.T, wl.d), dtype=torch.float64)
    h = wl.h
    for t in range(wl.T):
        for j in range(wl.k):
            e = int(wl.expert_ids[t, j])
            if not 0 <= e < wl.E:
                continue
            u = x[t] @ wug[e].T
            y = y.index_add(0, torch.tensor([t]), (rw[t, j] * ((F.silu(u[:h]) * u[h:]) @ wdn[e]))[None])
    (y * _bits_to_f64(dy)).sum().backward()
    for name, ref in (("dx", x.grad), ("dw_ug", wug.grad), ("dw_down", wdn.grad)):
        g = _bits_to_f64(got[name]).numpy()
        r = ref.detach().numpy()
        assert np.linalg.norm(g - r) <= 2e-2 * np.linalg.norm(r), f"{name}: rel err {np.linalg.norm(g - r) / np.linalg.norm(r)}"
    r = rw.grad.detach().numpy()
    assert np.linalg.norm(got["d_routing_w"] - r) <= 2e-2 * np.linalg.norm(r)
    assert np.all(_bits_to_f64(got["dw_ug"]).numpy()[2] == 0) and np.all(_bits_to_f64(got["dw_down"]).numpy()[2] == 0)


ALL_PINS = [
    pin_toy_golden,
    pin_printed_arithmetic,
    pin_histogram_and_order,
    pin_permute_unpermute_identity,
    pin_single_expert_is_dense_mlp,
    pin_column_partition,
    pin_brute_force,
    pin_invariances,
    pin_f32_within_bound,
    pin_token_form,
    pin_projection_column_partition,
    pin_projection_brute_force,
    pin_projection_is_down_step,
    pin_backward_is_autograd,
    pin_backward_brute_force,
    pin_permutation_backward_is_autograd,
    pin_swiglu_backward_is_autograd,
    pin_expert_backward_is_autograd,
]
