"""The gate/up projection that also keeps U for the backward, through the C ABI, on an MI355X.

U = [G | Up] = bf16(x_perm W_ug[e]^T) per expert block (OLMo report Eq 13's
pre-activation). The saving launch must leave h_buf exactly as the plain launch
writes it, store U exactly as the plain grouped projection computes it (the
same MFMA sequence per element), match the oracle's U within the step's
tolerance, and let the backward skip its recompute with identical results.
"""

import numpy as np
import pytest
import torch

import oracle
import ragged_grouped_gemm_histogram_amd as moe
from gpu_util import DeviceInputs, bits, say, to_dev, to_dev_bf16
from parity import compare_bf16
from workloads import make_random, to_bf16_bits

pytestmark = pytest.mark.gpu


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))]).astype(np.int32)


@pytest.mark.parametrize("counts,d,h", [
    ([700, 900, 420], 128, 4480),                 # large blocks, enough tiles to fill the device: 256-row tiles
    ([0, 37, 300, 1, 129, 0, 513], 320, 288),     # 128-row tiles, empty experts, partial last column tile
    ([5, 0, 260, 77], 328, 200),                  # K not a multiple of 64: zero-staged K remainder
    ([700, 900, 420], 200, 4480),                 # a K remainder on the 256-row tiles
    ([1], 64, 64),                                # one row
], ids=["big-tiles", "ragged", "k-tail", "big-k-tail", "one-row"])
def test_save_u_forward(counts, d, h):
    say(f"[gpu] save-U forward counts={counts} d={d} h={h}")
    rng = np.random.default_rng(sum(counts) + d + h)
    M, E = sum(counts), len(counts)
    x = to_bf16_bits(rng.standard_normal((M + 16, d), dtype=np.float32))
    w_ug = to_bf16_bits(0.05 * rng.standard_normal((E, 2 * h, d), dtype=np.float32))
    offs = _offsets(counts)
    xd, od, wd = to_dev_bf16(x), to_dev(offs), to_dev_bf16(w_ug)
    three = bits(torch.tensor(3.0, dtype=torch.bfloat16))
    h_plain = moe.moe_gemm_up_swiglu(xd, od, wd)
    h_sent = torch.full((M + 16, h), 3.0, dtype=torch.bfloat16, device="cuda:0")
    u_sent = torch.full((M + 16, 2 * h), 3.0, dtype=torch.bfloat16, device="cuda:0")
    h_u, u = moe.moe_gemm_up_swiglu_u(xd, od, wd, h_buf=h_sent, u_buf=u_sent)
    u_proj = moe.moe_grouped_projection(xd, od, wd, "out_in")
    torch.cuda.synchronize()
    assert np.array_equal(bits(h_u)[:M], bits(h_plain)[:M]), "h_buf differs from the plain launch"
    assert np.array_equal(bits(u)[:M], bits(u_proj)[:M]), "U differs from the grouped projection"
    assert (bits(h_u)[M:] == three).all() and (bits(u)[M:] == three).all(), "rows past M were written"
    ref = oracle.grouped_projection(x, offs, np.swapaxes(w_ug, 1, 2))
    say("  " + str(compare_bf16(bits(u)[:M], ref, "u")))


@pytest.mark.timeout(600)
def test_backward_with_saved_u_matches_recompute():
    wl = make_random(T=1500, k=4, E=12, d=320, h=256, seed=33, drop_frac=0.1, empty_experts=(4,))
    say(f"[gpu] backward with saved U T={wl.T} k={wl.k} E={wl.E} d={wl.d} h={wl.h}")
    di = DeviceInputs(wl)
    y, p, h_buf, y_perm = moe.moe_expert_forward(di.x, di.ids, di.w, di.w_ug, di.w_down)
    h_u, u = moe.moe_gemm_up_swiglu_u(p.x_perm, p.offsets, di.w_ug)
    M = int(p.offsets[-1].item())
    rng = np.random.default_rng(34)
    dy = to_dev_bf16(to_bf16_bits(rng.standard_normal((wl.T, wl.d), dtype=np.float32)))
    a = moe.moe_expert_backward(dy, p, di.w, di.w_ug, di.w_down, h_buf, y_perm)
    b = moe.moe_expert_backward(dy, p, di.w, di.w_ug, di.w_down, h_u, y_perm, u=u)
    torch.cuda.synchronize()
    assert torch.equal(h_u[:M].view(torch.int16), h_buf[:M].view(torch.int16))
    for key in ("dx", "dw_ug", "dw_down", "du"):
        ga, gb = a[key], b[key]
        if key == "du":
            ga, gb = ga[:M], gb[:M]
        assert torch.equal(ga.view(torch.int16), gb.view(torch.int16)), f"{key} differs with the saved U"
    assert torch.equal(a["d_routing_w"], b["d_routing_w"])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["zipf64", "qwen3_30b", "square"])
def test_save_u_at_full_size(name):
    """The named workloads' gate/up launch with U kept: h_buf equal to the plain launch's and U equal to the
    grouped projection's, bit for bit (each element runs the same MFMA sequence in the three launches)."""
    from gpu_util import workload
    wl = workload(name)
    say(f"[gpu] save-U at full size: {name}")
    di = DeviceInputs(wl)
    p = moe.moe_permute(di.x, di.ids, wl.E, gather=True)
    h_plain = moe.moe_gemm_up_swiglu(p.x_perm, p.offsets, di.w_ug)
    h_u, u = moe.moe_gemm_up_swiglu_u(p.x_perm, p.offsets, di.w_ug)
    u_proj = moe.moe_grouped_projection(p.x_perm, p.offsets, di.w_ug, "out_in")
    torch.cuda.synchronize()
    M = int(p.offsets[-1].item())
    assert torch.equal(h_u[:M].view(torch.int16), h_plain[:M].view(torch.int16)), "h_buf differs from the plain launch"
    assert torch.equal(u[:M].view(torch.int16), u_proj[:M].view(torch.int16)), "U differs from the grouped projection"
