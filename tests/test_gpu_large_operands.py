"""Grouped GEMMs whose operands reach 2 GiB, on an MI355X.

With K not a multiple of 64 the pipelined loop loads through buffer resources whose 32-bit
ranges must stay below 2 GiB; a larger token matrix or expert weight takes the
register-staged loop instead. These cases keep that loop covered: its output is held to
the oracle on sampled rows or columns (OLMo report Eq 13, one expert projection per block),
and the gathered gate/up projection to the pipelined loop's result on the permuted copy of
the same rows, bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import ragged_grouped_gemm_histogram_amd as moe
from gpu_util import bits, say, to_dev
from parity import compare_bf16
from workloads import projection_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
def test_projection_weight_above_2gib():
    """One expert's weight of 8200 x 131072 bf16 (2.15 GB), K % 64 = 8: register-staged loop."""
    E, K, N, M = 1, 8200, 131072, 300
    assert K * N * 2 > 2**31 and K % 64 != 0
    say(f"[gpu] projection with a 2.15 GB expert weight: M={M} K={K} N={N}")
    a, w = projection_inputs(M, K, N, E, seed=41, device="cuda:0")
    offs = np.array([0, M], dtype=np.int32)
    y = moe.moe_gemm_down(a, to_dev(offs), w)
    torch.cuda.synchronize()
    rng = np.random.default_rng(41)
    cols = np.unique(np.concatenate([np.arange(256), np.arange(N - 256, N), rng.integers(0, N, size=256)]))
    cols_dev = torch.from_numpy(cols).to("cuda:0")
    w_cols = bits(w[:, :, cols_dev].contiguous())
    ref = oracle.grouped_projection(bits(a), offs, w_cols)
    say("  " + str(compare_bf16(bits(y[:, cols_dev].contiguous()), ref, "y")))


@pytest.mark.timeout(600)
def test_gathered_gate_up_token_matrix_above_2gib():
    """Token matrix of 131072 x 8200 bf16 (2.15 GB) read through perm, K % 64 = 8: the gathered launch
    takes the register-staged loop and must equal the pipelined loop on the permuted copy bit for bit."""
    T, d, h, E, k = 131072, 8200, 64, 2, 1
    assert T * d * 2 > 2**31 and d % 64 != 0
    say(f"[gpu] gathered gate/up projection over a 2.15 GB token matrix: T={T} d={d} h={h} E={E}")
    x, _ = projection_inputs(T, d, 8, 1, seed=42, device="cuda:0")
    g = torch.Generator(device="cuda:0")
    g.manual_seed(42)
    w_ug = (torch.randn((E, 2 * h, d), generator=g, device="cuda:0") * 0.02).to(torch.bfloat16)
    ids = torch.randint(0, E, (T, k), generator=g, device="cuda:0", dtype=torch.int32)
    p = moe.moe_permute(x, ids, E, gather=True)
    h_gather = moe.moe_gemm_up_swiglu_gather(x, p.perm, p.offsets, w_ug, k)
    h_copy = moe.moe_gemm_up_swiglu(p.x_perm, p.offsets, w_ug)
    torch.cuda.synchronize()
    M = int(p.offsets[-1].item())
    assert M == T * k
    assert torch.equal(h_gather[:M], h_copy[:M]), "gathered (register-staged) and permuted-copy h_buf differ"
    # sampled sorted rows against the oracle: their token rows, the experts' weights
    offs = p.offsets.cpu().numpy()
    rng = np.random.default_rng(42)
    got, ref = [], []
    for e in range(E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, size=126)]))
        rows_dev = torch.from_numpy(rows).to("cuda:0")
        tokens = p.perm[rows_dev].long() // k
        a_rows = bits(x[tokens].contiguous())
        u = oracle.grouped_projection(a_rows, np.array([0, len(rows)], dtype=np.int32),
                                      bits(w_ug[e:e + 1].transpose(1, 2).contiguous()))
        ref.append(oracle.swiglu_rows(u))
        got.append(bits(h_gather[rows_dev].contiguous()))
    say("  " + str(compare_bf16(np.concatenate(got), np.concatenate(ref), "h_buf", elementwise=False)))
