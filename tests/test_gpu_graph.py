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
