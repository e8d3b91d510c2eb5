"""The forward step captured in a HIP graph and replayed (the library allocates, synchronises and
copies nothing, so its calls are capturable as they stand).

Every replay is checked against the eager result bit for bit (the kernels are deterministic), with
eager work and synchronisations between replays, and the inputs are rewritten in place between
replays so a replay must read live device data rather than a captured snapshot.
"""

import numpy as np
import pytest
import torch

import ragged_grouped_gemm_histogram_amd as moe
from gpu_util import DeviceInputs, say
from workloads import make_random, make_workload

pytestmark = pytest.mark.gpu


def _buffers(wl, dev):
    S = wl.T * wl.k
    return dict(
        h_buf=torch.empty((S, wl.h), dtype=torch.bfloat16, device=dev),
        y_perm=torch.empty((S, wl.d), dtype=torch.bfloat16, device=dev),
        y=torch.empty((wl.T, wl.d), dtype=torch.bfloat16, device=dev),
        counts=torch.empty((wl.E,), dtype=torch.int32, device=dev),
        offsets=torch.empty((wl.E + 1,), dtype=torch.int32, device=dev),
        perm=torch.empty((S,), dtype=torch.int32, device=dev),
        inv=torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev),
        ws=torch.empty((max(moe.permute_workspace_bytes(wl.T, wl.k, wl.E), 4),), dtype=torch.uint8, device=dev),
    )


def _step(di, b, k):
    p = moe.moe_permute(di.x, di.ids, di.w_ug.shape[0], counts=b["counts"], offsets=b["offsets"], perm=b["perm"],
                        inv_map=b["inv"], workspace=b["ws"], gather=False)
    moe.moe_gemm_up_swiglu_gather(di.x, p.perm, p.offsets, di.w_ug, k, h_buf=b["h_buf"])
    moe.moe_gemm_down(b["h_buf"], p.offsets, di.w_down, y_perm=b["y_perm"])
    moe.moe_unpermute(b["y_perm"], p.inv_map, di.w, y=b["y"])


@pytest.mark.parametrize("name", ["edge", "random"])
def test_forward_step_graph_replays(name):
    wl = make_workload(name) if name != "random" else make_random(T=500, k=3, E=7, d=136, h=72, seed=8,
                                                                    drop_frac=0.2, empty_experts=(3,))
    say(f"[gpu] graph capture of the forward step: {wl.name} T={wl.T} k={wl.k} E={wl.E}")
    dev = torch.device("cuda:0")
    di = DeviceInputs(wl)
    b = _buffers(wl, dev)
    _step(di, b, wl.k)  # eager warm-up: first-call device queries and kernel attributes happen here
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _step(di, b, wl.k)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    for rep in range(3):
        # new token rows and routing weights in place, then the eager reference on copies
        di.x.copy_(torch.from_numpy(rng.standard_normal(tuple(di.x.shape)).astype(np.float32)).to(torch.bfloat16))
        di.w.copy_(torch.from_numpy(rng.random(tuple(di.w.shape)).astype(np.float32)))
        torch.cuda.synchronize()
        ref = _buffers(wl, dev)
        _step(di, ref, wl.k)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in ("counts", "offsets", "inv", "h_buf", "y_perm", "y"):
            M = int(ref["offsets"][-1].item())
            a, r = b[key], ref[key]
            if key in ("h_buf", "y_perm"):
                a, r = a[:M], r[:M]
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               r.view(torch.int16) if r.dtype == torch.bfloat16 else r), f"replay {rep}: {key} differs"
        say(f"  replay {rep} matches the eager step")


def _train_buffers(wl, dev):
    S, T, k, d, h, E = wl.T * wl.k, wl.T, wl.k, wl.d, wl.h, wl.E
    bf = dict(dtype=torch.bfloat16, device=dev)
    b = _buffers(wl, dev)
    b.update(
        x_perm=torch.empty((S, d), **bf), u=torch.empty((S, 2 * h), **bf), dy_perm=torch.empty((S, d), **bf),
        d_rw=torch.empty((T, k), dtype=torch.float32, device=dev), dh=torch.empty((S, h), **bf),
        du=torch.empty((S, 2 * h), **bf), dx_perm=torch.empty((S, d), **bf), dx=torch.empty((T, d), **bf),
        dw_down=torch.empty((E, h, d), **bf), dw_ug=torch.empty((E, 2 * h, d), **bf),
        wws=torch.empty((max(moe.wgrad_workspace_bytes(S, d, 2 * h, E), moe.wgrad_workspace_bytes(S, h, d, E), 16),),
                        dtype=torch.uint8, device=dev),
    )
    return b


def _train_step(di, b, dy):
    """Forward keeping U, then the backward from it: every call writes into b."""
    p = moe.moe_permute(di.x, di.ids, di.w_ug.shape[0], x_perm=b["x_perm"], counts=b["counts"], offsets=b["offsets"],
                        perm=b["perm"], inv_map=b["inv"], workspace=b["ws"], gather=True)
    moe.moe_gemm_up_swiglu_u(p.x_perm, p.offsets, di.w_ug, h_buf=b["h_buf"], u_buf=b["u"])
    moe.moe_gemm_down(b["h_buf"], p.offsets, di.w_down, y_perm=b["y_perm"])
    moe.moe_unpermute(b["y_perm"], p.inv_map, di.w, y=b["y"])
    moe.moe_unpermute_backward(dy, b["y_perm"], p.inv_map, di.w, dy_perm=b["dy_perm"], d_routing_w=b["d_rw"])
    moe.moe_grouped_dgrad(b["dy_perm"], p.offsets, di.w_down, "in_out", dx=b["dh"])
    moe.moe_grouped_wgrad(b["h_buf"], b["dy_perm"], p.offsets, "in_out", dw=b["dw_down"], workspace=b["wws"])
    moe.moe_swiglu_backward(b["dh"], b["u"], p.offsets, du=b["du"])
    moe.moe_grouped_dgrad(b["du"], p.offsets, di.w_ug, "out_in", dx=b["dx_perm"])
    moe.moe_grouped_wgrad(p.x_perm, b["du"], p.offsets, "out_in", dw=b["dw_ug"], workspace=b["wws"])
    moe.moe_permute_backward(b["dx_perm"], p.inv_map, dx=b["dx"])


def test_training_step_graph_replays():
    """Forward (keeping U) and backward of the expert step captured in one graph; replays match eager runs."""
    wl = make_random(T=1200, k=4, E=9, d=256, h=192, seed=12, drop_frac=0.1, empty_experts=(2,))
    say(f"[gpu] graph capture of the training step: T={wl.T} k={wl.k} E={wl.E} d={wl.d} h={wl.h}")
    dev = torch.device("cuda:0")
    di = DeviceInputs(wl)
    b = _train_buffers(wl, dev)
    dy = torch.empty((wl.T, wl.d), dtype=torch.bfloat16, device=dev)
    rng = np.random.default_rng(5)
    dy.copy_(torch.from_numpy(rng.standard_normal((wl.T, wl.d)).astype(np.float32)).to(torch.bfloat16))
    _train_step(di, b, dy)  # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _train_step(di, b, dy)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        di.x.copy_(torch.from_numpy(rng.standard_normal(tuple(di.x.shape)).astype(np.float32)).to(torch.bfloat16))
        dy.copy_(torch.from_numpy(rng.standard_normal((wl.T, wl.d)).astype(np.float32)).to(torch.bfloat16))
        torch.cuda.synchronize()
        ref = _train_buffers(wl, dev)
        _train_step(di, ref, dy)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        M = int(ref["offsets"][-1].item())
        for key in ("y", "dx", "dw_down", "dw_ug", "d_rw", "u", "du"):
            a, r = b[key], ref[key]
            if key in ("u", "du"):
                a, r = a[:M], r[:M]
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               r.view(torch.int16) if r.dtype == torch.bfloat16 else r), f"replay {rep}: {key} differs"
        say(f"  replay {rep} matches the eager training step")
