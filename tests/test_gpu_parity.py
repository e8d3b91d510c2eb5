"""HIP path against the oracle, through the C ABI, on an MI355X.

Integer outputs (counts, offsets, perm[0, M), inv_map) and the permuted rows are
compared bit for bit. bf16 outputs y_perm rows [0, M) and y are held to
|got - ref| <= 1e-2 + 1e-2*|ref| plus the data-scaled guards in parity.py. The
SwiGLU activations h_buf are checked through their pre-activation: U from the
U-keeping launch (whose h_buf must equal the path's bit for bit) against the
oracle's U with the same bound, and h_buf against the oracle's SwiGLU of that U
within one bf16 step (parity.py states why). The oracle runs its per-expert
loop in float32. The five named workloads run at full size in the launch
configuration the benchmark times; small random cases cover empty experts,
invalid ids, tails and degenerate sizes.
"""

import numpy as np
import pytest
import torch

import oracle
import ragged_grouped_gemm_histogram_amd as moe
from gpu_util import DeviceInputs, bits, oracle_result, say, to_dev, to_dev_bf16, workload
from parity import assert_fails, compare_bf16, compare_swiglu_of_u
from workloads import WORKLOADS, make_counts, make_random

pytestmark = pytest.mark.gpu

NAMES = list(WORKLOADS)


def run_path(wl, sync=True, fused=False, di=None):
    di = di or DeviceInputs(wl)
    y, p, h_buf, y_perm = moe.moe_expert_forward(di.x, di.ids, di.w, di.w_ug, di.w_down, fused_gather=fused)
    if sync:
        torch.cuda.synchronize()
    return y, p, h_buf, y_perm


def check_permute(p, ref, wl):
    M = ref.M
    np.testing.assert_array_equal(p.counts.cpu().numpy(), ref.counts)
    np.testing.assert_array_equal(p.offsets.cpu().numpy(), ref.offsets)
    np.testing.assert_array_equal(p.perm.cpu().numpy()[:M], ref.perm[:M])
    np.testing.assert_array_equal(p.inv_map.cpu().numpy(), ref.inv_map)
    if p.x_perm is not None:  # the fused-gather path never materialises x_perm
        np.testing.assert_array_equal(bits(p.x_perm)[:M], ref.x_perm)


def check_h_through_u(h_buf, u, ref_u, ref_h, M, what="h_buf"):
    """U against the oracle's U (contract bound); h_buf against the oracle's SwiGLU of the GPU's own U
    (one bf16 step); h_buf against the oracle's H under the data-scaled guards."""
    ub = bits(u)[:M]
    hb = bits(h_buf)[:M]
    s_u = compare_bf16(ub, ref_u, f"U ({what})")
    s_s = compare_swiglu_of_u(hb, oracle.swiglu_rows(ub), f"{what} vs SwiGLU(U)")
    s_h = compare_bf16(hb, ref_h, what, elementwise=False)
    say(f"  U {s_u}\n  {what} vs SwiGLU(own U) {s_s}\n  {what} vs oracle H {s_h}")


def u_of_path(di, p, wl):
    """U from the U-keeping launch on the path's sorted rows (x_perm rebuilt when the path fused the gather)."""
    x_perm = p.x_perm if p.x_perm is not None else moe.moe_permute(di.x, di.ids, wl.E).x_perm
    return moe.moe_gemm_up_swiglu_u(x_perm, p.offsets, di.w_ug)


def check_all(wl, ref, y, p, h_buf, y_perm, di=None):
    check_permute(p, ref, wl)
    M = ref.M
    di = di or DeviceInputs(wl)
    h_u, u = u_of_path(di, p, wl)
    torch.cuda.synchronize()
    assert torch.equal(h_u[:M], h_buf[:M]), "the U-keeping launch's h_buf differs from the path's"
    check_h_through_u(h_buf, u, ref.u, ref.h, M)
    del h_u, u
    s_yp = compare_bf16(bits(y_perm)[:M], ref.y_perm, "y_perm")
    s_y = compare_bf16(bits(y), ref.y, "y")
    say(f"  y_perm {s_yp}\n  y {s_y}")
    return s_y


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,fused", [(n, f) for n in NAMES for f in (False, True)],
                         ids=[f"{n}-{'fused' if f else 'xperm'}" for n in NAMES for f in (False, True)])
def test_named_workload_full_size(name, fused):
    wl = workload(name)
    say(f"[gpu] full path {name} fused_gather={fused}")
    di = DeviceInputs(wl)
    y, p, h_buf, y_perm = run_path(wl, fused=fused, di=di)
    ref = oracle_result(name)
    check_all(wl, ref, y, p, h_buf, y_perm, di)


def _fuzz_cases():
    rng = np.random.default_rng(2024)
    cases = []
    for i in range(24):
        E = int(rng.integers(1, 10))
        T = int(rng.integers(0, 41))
        k = int(rng.integers(1, 5))
        d = 8 * int(rng.integers(1, 34))
        h = 8 * int(rng.integers(1, 34))
        empty = tuple(sorted(set(rng.integers(0, E, size=int(rng.integers(0, 3))).tolist())))
        cases.append(dict(T=T, k=k, E=E, d=d, h=h, seed=100 + i, drop_frac=float(rng.choice([0, 0.1, 0.5])),
                          empty_experts=empty))
    # tails and multi-tile shapes: K not a multiple of 64, N not a multiple of the tile, >1 tile in M
    cases += [
        dict(T=300, k=2, E=3, d=200, h=136, seed=1, drop_frac=0.05),
        dict(T=520, k=1, E=2, d=72, h=264, seed=2, drop_frac=0.0),
        dict(T=129, k=3, E=5, d=520, h=392, seed=3, drop_frac=0.2, empty_experts=(1, 3)),
        dict(T=64, k=4, E=1, d=8, h=8, seed=4, drop_frac=0.0),
        dict(T=40, k=2, E=1024, d=64, h=64, seed=5, drop_frac=0.1),
        dict(T=33, k=2, E=6, d=64, h=64, seed=6, drop_frac=1.0),  # every slot dropped: M = 0
        # K % 64 == 0 with N and M tails: large blocks (>= 384 rows per expert) whose 256-row tiles
        # can fill the device take the 256 x 256 tile, others the 128 x 256 tile
        dict(T=900, k=2, E=3, d=320, h=192, seed=7, drop_frac=0.05),
        # (weights scaled down, as in the named workloads, so that the long contractions keep
        # activations of order one and the contract's absolute bound stays meaningful)
        dict(T=1000, k=2, E=3, d=128, h=4480, seed=12, drop_frac=0.05, w_sigma=0.04),  # 256-row tiles, gate/up side
        dict(T=1000, k=2, E=3, d=8768, h=64, seed=13, drop_frac=0.05, empty_experts=(1,), w_sigma=0.015),  # down side
        dict(T=200, k=3, E=4, d=320, h=192, seed=8, drop_frac=0.05, empty_experts=(2,)),
        dict(T=1100, k=1, E=2, d=576, h=448, seed=9, drop_frac=0.0),
        # many tiles per workgroup with one or two K stages per tile: the load stream runs
        # across tile boundaries (256-row tiles on the gate/up side, 128-row on the down side)
        dict(T=20000, k=2, E=8, d=64, h=256, seed=10, drop_frac=0.02),
        dict(T=6000, k=4, E=96, d=128, h=64, seed=11, drop_frac=0.1, empty_experts=(5, 50)),
        # many slots per token (duplicates within a token included): the unpermute sums 16 rows
        dict(T=300, k=16, E=40, d=136, h=96, seed=14, drop_frac=0.1, empty_experts=(7,)),
        # 256-row gate/up tiles over three and four K stages: the second wave of each SIMD issues its
        # half of a stage's loads one slice after the first (and the first two stages start together)
        dict(T=4096, k=2, E=4, d=192, h=1024, seed=15, drop_frac=0.03),
        dict(T=4096, k=2, E=4, d=256, h=1024, seed=16, drop_frac=0.0, empty_experts=(2,)),
        # the permute's one-workgroup path (at most 64 chunks of 256 slots and 8192 table entries) at
        # its boundary, one chunk past it, and with too many experts for its table
        dict(T=8192, k=2, E=16, d=64, h=64, seed=17, drop_frac=0.1),
        dict(T=8193, k=2, E=16, d=64, h=64, seed=18, drop_frac=0.1),
        dict(T=2048, k=4, E=1024, d=64, h=64, seed=19, drop_frac=0.05),
        # the two-launch permute (histogram, then scan and scatter in one launch) at its table limit of
        # 2^16 entries (64 experts x 1024 chunks) and one chunk past it (three launches)
        dict(T=32768, k=8, E=64, d=64, h=64, seed=20, drop_frac=0.05, empty_experts=(9,)),
        dict(T=32800, k=8, E=64, d=64, h=64, seed=21, drop_frac=0.05),
    ]
    return cases


FUZZ = _fuzz_cases()


@pytest.mark.parametrize("case", FUZZ, ids=[f"T{c['T']}k{c['k']}E{c['E']}d{c['d']}h{c['h']}s{c['seed']}" for c in FUZZ])
def test_random_cases(case):
    wl = make_random(**case)
    say(f"[gpu] random case {case}")
    di = DeviceInputs(wl)
    y, p, h_buf, y_perm = run_path(wl, di=di)
    ref = oracle.moe_expert_forward(wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down, keep_u=True)
    check_all(wl, ref, y, p, h_buf, y_perm, di)
    # the down projection alone, from the GPU's own h_buf: its error without GEMM 1's roundings
    M = ref.M
    chained = oracle.grouped_projection(bits(h_buf)[:M], ref.offsets, wl.w_down)
    say("  y_perm from the GPU's h_buf " + str(compare_bf16(bits(y_perm)[:M], chained, "y_perm (chained)")))
    # the fused-gather path runs the same arithmetic on the same rows: identical bits
    y2, p2, h2, yp2 = run_path(wl, fused=True)
    assert torch.equal(y2, y) and torch.equal(h2[:M], h_buf[:M]) and torch.equal(yp2[:M], y_perm[:M])


# Exact expert sizes whose last row tile ends on and next to every wave-row boundary: in the last tile of an
# expert, waves whose rows all lie past the block skip their matrix work (they keep only their loads and
# barriers). The 256-row tiles have wave rows of 64 (gate/up, waves 4x2) and 128 (down, waves 2x4), the
# 128-row tiles of 64; remainders of 1, 64, 65, 128, 129, 192, 193, 255 and 256 rows cover every count of
# skipping waves in both, and the shapes are large enough that each side takes the tile height named.
COUNT_CASES = [
    # 256-row tiles on both sides (>= 384 rows per expert, enough 256-row tiles to occupy the device)
    dict(T=8192, k=2, E=9, d=1024, h=1024, seed=31, w_sigma=0.03,
         counts=[6 * 256 + r for r in (1, 64, 65, 128, 129, 192, 193, 255, 256)]),
    # 128-row tiles (too few 256-row tiles to occupy the device)
    dict(T=2048, k=2, E=9, d=1024, h=1024, seed=32, w_sigma=0.03,
         counts=[2 * 128 + r for r in (1, 32, 63, 64, 65, 96, 127, 128, 0)]),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", COUNT_CASES, ids=["tiles256", "tiles128"])
def test_expert_tails_at_wave_row_boundaries(case):
    wl = make_counts(**case)
    say(f"[gpu] exact-count case {case}")
    di = DeviceInputs(wl)
    y, p, h_buf, y_perm = run_path(wl, di=di)
    ref = oracle.moe_expert_forward(wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down, keep_u=True)
    np.testing.assert_array_equal(ref.counts, np.asarray(case["counts"]))
    check_all(wl, ref, y, p, h_buf, y_perm, di)
    M = ref.M
    chained = oracle.grouped_projection(bits(h_buf)[:M], ref.offsets, wl.w_down)
    say("  y_perm from the GPU's h_buf " + str(compare_bf16(bits(y_perm)[:M], chained, "y_perm (chained)")))


def test_negative_controls_fail_the_comparison():
    name = "qwen3_30b"  # the workload whose outputs are small enough for the plain bound to be vacuous
    wl = workload(name)
    ref = oracle_result(name)
    zeros = np.zeros_like(ref.y)
    assert_fails(compare_bf16, zeros, ref.y, "zeros")
    swapped_ug = wl.w_ug.copy()
    swapped_ug[[0, 1]] = swapped_ug[[1, 0]]
    swapped_dn = wl.w_down.copy()
    swapped_dn[[0, 1]] = swapped_dn[[1, 0]]
    say("[gpu] qwen3_30b with experts 0 and 1 swapped")
    di = DeviceInputs(wl)
    y, _, _, _ = moe.moe_expert_forward(di.x, di.ids, di.w, to_dev_bf16(swapped_ug), to_dev_bf16(swapped_dn))
    torch.cuda.synchronize()
    assert_fails(compare_bf16, bits(y), ref.y, "swapped experts")


def test_deterministic_and_stage_calls_match():
    wl = workload("edge")
    say("[gpu] determinism on edge")
    y1, p1, h1, yp1 = run_path(wl)
    y2, p2, h2, yp2 = run_path(wl)
    M = int(p1.offsets[-1].item())
    assert torch.equal(y1, y2) and torch.equal(h1[:M], h2[:M]) and torch.equal(yp1[:M], yp2[:M])
    di = DeviceInputs(wl)
    hb = moe.moe_gemm_up_swiglu(p1.x_perm, p1.offsets, di.w_ug)
    yp = moe.moe_gemm_down(hb, p1.offsets, di.w_down)
    torch.cuda.synchronize()
    assert torch.equal(hb[:M], h1[:M]) and torch.equal(yp[:M], yp1[:M])


def test_rows_past_M_are_left_untouched():
    wl = make_random(T=50, k=3, E=4, d=96, h=64, seed=9, drop_frac=0.3)
    di = DeviceInputs(wl)
    S = wl.T * wl.k
    sentinel = torch.full((S, wl.d), 7.0, dtype=torch.bfloat16, device="cuda:0")
    x_perm, y_perm = sentinel.clone(), sentinel.clone()
    h_buf = torch.full((S, wl.h), 7.0, dtype=torch.bfloat16, device="cuda:0")
    perm = torch.full((S,), -7, dtype=torch.int32, device="cuda:0")
    say("[gpu] rows past M untouched")
    p = moe.moe_permute(di.x, di.ids, wl.E, x_perm=x_perm, perm=perm)
    moe.grouped_swiglu_expert(p.x_perm, p.offsets, di.w_ug, di.w_down, h_buf=h_buf, y_perm=y_perm)
    torch.cuda.synchronize()
    M = int(p.offsets[-1].item())
    assert M < S
    assert torch.all(x_perm[M:] == 7.0) and torch.all(h_buf[M:] == 7.0) and torch.all(y_perm[M:] == 7.0)
    assert torch.all(perm[M:] == -7)


def test_permute_then_unpermute_is_identity():
    wl = make_random(T=300, k=1, E=7, d=136, h=8, seed=13, drop_frac=0.2)
    di = DeviceInputs(wl)
    ones = torch.ones((wl.T, 1), dtype=torch.float32, device="cuda:0")
    say("[gpu] permute/unpermute identity k=1")
    p = moe.moe_permute(di.x, di.ids, wl.E)
    y = moe.moe_unpermute(p.x_perm, p.inv_map, ones)
    torch.cuda.synchronize()
    kept = (p.inv_map[:, 0] >= 0)
    assert torch.equal(y[kept], di.x[kept])
    assert torch.all(y[~kept] == 0)
    wl = make_random(T=200, k=4, E=5, d=64, h=8, seed=14, drop_frac=0.0)  # softmax weights sum to 1
    di = DeviceInputs(wl)
    p = moe.moe_permute(di.x, di.ids, wl.E)
    y = moe.moe_unpermute(p.x_perm, p.inv_map, di.w)
    torch.cuda.synchronize()
    ref = oracle.unpermute(bits(p.x_perm), p.inv_map.cpu().numpy(), wl.routing_w, wl.T, wl.k)
    np.testing.assert_array_equal(bits(y), ref)
    np.testing.assert_array_equal(bits(y), wl.x)


def test_relabel_and_shuffle_invariance():
    wl = make_random(T=160, k=3, E=6, d=200, h=136, seed=17, drop_frac=0.1)
    say("[gpu] relabel / shuffle invariance")
    base, _, _, _ = run_path(wl)
    rng = np.random.default_rng(5)
    relabel = rng.permutation(wl.E)
    ids = wl.expert_ids.copy()
    valid = (ids >= 0) & (ids < wl.E)
    ids[valid] = relabel[ids[valid]]
    inv_label = np.argsort(relabel)
    di = DeviceInputs(wl)
    y2, _, _, _ = moe.moe_expert_forward(di.x, to_dev(ids), di.w, to_dev_bf16(wl.w_ug[inv_label]),
                                         to_dev_bf16(wl.w_down[inv_label]))
    sh = rng.permutation(wl.T)
    y3, _, _, _ = moe.moe_expert_forward(di.x[to_dev(sh)], to_dev(wl.expert_ids[sh]), di.w[to_dev(sh)], di.w_ug,
                                         di.w_down)
    y4, _, _, _ = moe.moe_expert_forward(di.x, di.ids, 2 * di.w, di.w_ug, di.w_down)
    torch.cuda.synchronize()
    assert torch.equal(y2, base)
    assert torch.equal(y4.float(), 2 * base.float())
    ref = oracle.moe_expert_forward(wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down)
    compare_bf16(bits(y3), ref.y[sh], "shuffled tokens")


def test_zero_tokens():
    wl = make_random(T=0, k=2, E=3, d=16, h=16, seed=0)
    say("[gpu] T = 0")
    y, p, h_buf, y_perm = run_path(wl)
    assert y.shape == (0, 16)
    assert p.counts.cpu().tolist() == [0, 0, 0] and p.offsets.cpu().tolist() == [0, 0, 0, 0]


def test_out_of_range_offsets_stay_in_bounds():
    # Offsets that overrun the capacity are clamped on the device: rows past cap_rows are never touched.
    wl = make_random(T=30, k=2, E=3, d=64, h=64, seed=21, drop_frac=0.0)
    di = DeviceInputs(wl)
    S = wl.T * wl.k
    x_perm = to_dev_bf16(wl.x[np.arange(S) % wl.T])
    bad = torch.tensor([-5, 25, 40, 10_000], dtype=torch.int32, device="cuda:0")
    say("[gpu] clamped offsets")
    h_buf, y_perm = moe.grouped_swiglu_expert(x_perm, bad, di.w_ug, di.w_down)
    h_u, u = moe.moe_gemm_up_swiglu_u(x_perm, bad, di.w_ug)
    torch.cuda.synchronize()
    assert torch.equal(h_u, h_buf)
    clamped = np.array([0, 25, 40, S], dtype=np.int32)  # what the device clamp makes of them
    h_ref, yp_ref, u_ref = oracle.expert_forward(bits(x_perm), clamped, wl.w_ug, wl.w_down, return_u=True)
    check_h_through_u(h_buf, u, u_ref, h_ref, S, "h_buf (clamped offsets)")
    compare_bf16(bits(y_perm), yp_ref, "y_perm (clamped offsets)")
