"""The non-allocating permute against the allocating one, through the C ABI, on an MI355X.

moe_permute_noalloc keeps its per-chunk histogram table in the library's fixed
per-device array instead of a caller workspace. Its outputs (counts, offsets,
perm[0, M), inv_map and the permuted rows) are integers and row copies, so they
must equal moe_permute's bit for bit on the same ids. Two calls in a row, the
second smaller than the first, show that a call never depends on what the
previous one left in the shared table; entries past M stay untouched.
"""

import numpy as np
import pytest
import torch

import ragged_grouped_gemm_histogram_amd as moe
from gpu_util import bits, say, to_dev, to_dev_bf16
from workloads import make_random

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _sentinel_outputs(T, k, E, d, gather):
    S = T * k
    return dict(
        x_perm=torch.full((S, d), 5.0, dtype=torch.bfloat16, device=DEV) if gather else None,
        counts=torch.full((E,), -3, dtype=torch.int32, device=DEV),
        offsets=torch.full((E + 1,), -3, dtype=torch.int32, device=DEV),
        perm=torch.full((S,), -3, dtype=torch.int32, device=DEV),
        inv_map=torch.full((T, k), -3, dtype=torch.int32, device=DEV),
    )


def _run_both(wl, gather):
    x, ids = to_dev_bf16(wl.x), to_dev(wl.expert_ids.astype(np.int32))
    ref = moe.moe_permute(x, ids, wl.E, gather=gather)
    got = moe.moe_permute_noalloc(x, ids, wl.E, **_sentinel_outputs(wl.T, wl.k, wl.E, wl.d, gather))
    torch.cuda.synchronize()
    M = int(ref.offsets[-1].item())
    assert torch.equal(got.counts, ref.counts)
    assert torch.equal(got.offsets, ref.offsets)
    assert torch.equal(got.perm[:M], ref.perm[:M])
    assert torch.equal(got.inv_map, ref.inv_map)
    assert torch.all(got.perm[M:] == -3), "perm entries past M were written"
    if gather:
        np.testing.assert_array_equal(bits(got.x_perm)[:M], bits(ref.x_perm)[:M])
        assert torch.all(got.x_perm[M:] == 5.0), "x_perm rows past M were written"
    return M


@pytest.mark.parametrize("gather", [True, False], ids=["gather", "no-gather"])
def test_noalloc_permute_equals_permute_twice_in_a_row(gather):
    first = make_random(T=8192, k=8, E=64, d=64, h=8, seed=61, drop_frac=0.05)   # 256 chunks: the table path
    second = make_random(T=5000, k=4, E=40, d=24, h=8, seed=62, drop_frac=0.1)   # smaller, still 79 chunks
    for wl in (first, second):
        say(f"[gpu] moe_permute_noalloc T={wl.T} k={wl.k} E={wl.E} d={wl.d} gather={gather}")
        M = _run_both(wl, gather)
        say(f"  identical to moe_permute, M={M}")


def test_noalloc_permute_one_workgroup_path_and_limit():
    # at most 64 chunks: the one-workgroup path, which keeps its table in LDS
    wl = make_random(T=2000, k=2, E=12, d=40, h=8, seed=63, drop_frac=0.2)
    say(f"[gpu] moe_permute_noalloc small T={wl.T} k={wl.k} E={wl.E}")
    _run_both(wl, True)
    # past the fixed table: rejected on the host before any launch
    T, k, E = 70000, 4, 1024  # 1024 * ceil(280000 / 256) = 1,120,256 > 2^20 entries
    x = torch.zeros((T, 8), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    say("[gpu] moe_permute_noalloc beyond its table")
    with pytest.raises(moe.MoeError, match="MOE_ERR_TOO_LARGE"):
        moe.moe_permute_noalloc(x, ids, E, **_sentinel_outputs(T, k, E, 8, False))
