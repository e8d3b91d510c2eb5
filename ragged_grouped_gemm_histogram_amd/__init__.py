"""Python binding of libmoe_grouped, the routed MoE expert step on MI355X (gfx950).

Argument marshalling only: every step runs in the HIP library's kernels. torch
supplies device memory and the current stream. The functions mirror the C ABI
declared in ``include/moe_grouped.h``; the optional ``out=`` tensors let a
caller keep fixed capacity-shaped buffers across calls.

The library must have been built (``python -m ragged_grouped_gemm_histogram_amd.build``);
every call raises ImportError when it is missing. There is no other code path.
"""

from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_grouped.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "moe_grouped.h")
MAX_EXPERTS = 1024

MOE_OK = 0

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_SIGNATURES = {
    "moe_permute_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "moe_permute": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_permute_noalloc": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "grouped_swiglu_expert": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
    "moe_gemm_up_swiglu": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp]),
    "moe_gemm_up_swiglu_u": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
    "moe_gemm_down": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp]),
    "moe_gemm_up_swiglu_gather": (ctypes.c_int, [_vp, _vp, _i64, _i32, _vp, _vp, _i64, _i64, _i32, _vp, _vp]),
    "grouped_swiglu_expert_gather": (ctypes.c_int,
                                     [_vp, _vp, _i64, _i32, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp, _vp]),
    "moe_unpermute": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i32, _i64, _vp, _vp]),
    "moe_grouped_projection": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp]),
    "moe_swiglu_backward": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i64, _vp, _vp]),
    "moe_grouped_dgrad": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp]),
    "moe_grouped_wgrad_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "moe_grouped_wgrad": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp, _sz, _vp]),
    "moe_permute_backward": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i64, _vp, _vp]),
    "moe_unpermute_backward": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i64, _vp, _vp, _vp]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

W_LAYOUTS = {"in_out": 0, "out_in": 1}  # [E, d_in, d_out] / [E, d_out, d_in]


_LIB = None


def load_library() -> ctypes.CDLL:
    """Load libmoe_grouped.so (once). Raises ImportError when it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m ragged_grouped_gemm_histogram_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


class MoeError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {load_library().moe_status_string(status).decode()}")


def header_functions() -> list[str]:
    """Names of the functions declared in include/moe_grouped.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return re.findall(r"^\s*(?:moe_status|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def _check(status: int, call: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, call)


def _stream(t: torch.Tensor) -> int:
    # The library launches on the current HIP device; a stream of another device would fail the launch.
    if t.device.index is not None and t.device.index != torch.cuda.current_device():
        raise ValueError(f"tensors are on {t.device} but the current device is cuda:{torch.cuda.current_device()}; "
                         "call inside torch.cuda.device(...)")
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _want(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple, device) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _out(t, name, dtype, shape, device):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _want(t, name, dtype, shape, device)


@dataclass
class Permuted:
    x_perm: torch.Tensor  # bf16 [T*k, d]; rows [0, M) valid
    counts: torch.Tensor  # int32 [E]
    offsets: torch.Tensor  # int32 [E+1]
    perm: torch.Tensor  # int32 [T*k]; entries [0, M) valid
    inv_map: torch.Tensor  # int32 [T, k]; -1 for dropped slots


def permute_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(load_library().moe_permute_workspace_bytes(T, k, E))


def moe_permute(x: torch.Tensor, expert_ids: torch.Tensor, num_experts: int, *, x_perm=None, counts=None,
                offsets=None, perm=None, inv_map=None, workspace=None, gather: bool = True) -> Permuted:
    """Histogram, offsets, stable order, inverse map and permuted gather (one stream, no sync).

    ``gather=False`` skips the row copy (``x_perm`` is None); a ``*_gather`` GEMM then reads X through perm.
    """
    if x.dim() != 2 or expert_ids.dim() != 2:
        raise ValueError("x must be [T, d] and expert_ids [T, k]")
    T, d = x.shape
    k = expert_ids.shape[1]
    dev = x.device
    _want(x, "x", torch.bfloat16, (T, d), dev)
    _want(expert_ids, "expert_ids", torch.int32, (T, k), dev)
    S = T * k
    E = int(num_experts)
    x_perm = _out(x_perm, "x_perm", torch.bfloat16, (S, d), dev) if gather else None
    counts = _out(counts, "counts", torch.int32, (E,), dev)
    offsets = _out(offsets, "offsets", torch.int32, (E + 1,), dev)
    perm = _out(perm, "perm", torch.int32, (S,), dev)
    inv_map = _out(inv_map, "inv_map", torch.int32, (T, k), dev)
    need = permute_workspace_bytes(T, k, E)
    if workspace is None:
        workspace = torch.empty((max(need, 4),), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the same device")
    _check(load_library().moe_permute(_ptr(x) if gather else None, _ptr(expert_ids), T, k, d, E, _ptr(x_perm),
                                      _ptr(counts), _ptr(offsets),
                           _ptr(perm), _ptr(inv_map), _ptr(workspace), workspace.numel(), _stream(x)),
           "moe_permute")
    return Permuted(x_perm, counts, offsets, perm, inv_map)


def moe_permute_noalloc(x: torch.Tensor, expert_ids: torch.Tensor, num_experts: int, *, x_perm: torch.Tensor | None,
                        counts: torch.Tensor, offsets: torch.Tensor, perm: torch.Tensor,
                        inv_map: torch.Tensor) -> Permuted:
    """moe_permute without a workspace, for callers that cannot allocate: the histogram table is the library's
    fixed per-device array (at most ``E * ceil(T*k/256) <= 2**20`` entries). Every output is the caller's own
    tensor, so this call allocates nothing; ``x_perm=None`` skips the row copy. Calls that overlap on one GPU
    share the table and race."""
    if x.dim() != 2 or expert_ids.dim() != 2:
        raise ValueError("x must be [T, d] and expert_ids [T, k]")
    T, d = x.shape
    k = expert_ids.shape[1]
    dev = x.device
    _want(x, "x", torch.bfloat16, (T, d), dev)
    _want(expert_ids, "expert_ids", torch.int32, (T, k), dev)
    S, E = T * k, int(num_experts)
    if x_perm is not None:
        _want(x_perm, "x_perm", torch.bfloat16, (S, d), dev)
    _want(counts, "counts", torch.int32, (E,), dev)
    _want(offsets, "offsets", torch.int32, (E + 1,), dev)
    _want(perm, "perm", torch.int32, (S,), dev)
    _want(inv_map, "inv_map", torch.int32, (T, k), dev)
    _check(load_library().moe_permute_noalloc(_ptr(x) if x_perm is not None else None, _ptr(expert_ids), T, k, d,
                                              E, _ptr(x_perm), _ptr(counts), _ptr(offsets), _ptr(perm),
                                              _ptr(inv_map), _stream(x)), "moe_permute_noalloc")
    return Permuted(x_perm, counts, offsets, perm, inv_map)


def _gemm_shapes(a: torch.Tensor, offsets: torch.Tensor, w: torch.Tensor):
    if a.dim() != 2 or w.dim() != 3 or offsets.dim() != 1:
        raise ValueError("expected a 2-D activation buffer, 1-D offsets and 3-D expert weights")
    return a.shape[0], a.device


def moe_gemm_up_swiglu(x_perm: torch.Tensor, offsets: torch.Tensor, w_ug: torch.Tensor, *, h_buf=None) -> torch.Tensor:
    """h_buf[rows_e] = bf16(SiLU(bf16(G)) * bf16(U)), [G|U] = x_perm[rows_e] @ W_ug[e]^T (one launch)."""
    cap, dev = _gemm_shapes(x_perm, offsets, w_ug)
    E, two_h, d = w_ug.shape
    h = two_h // 2
    _want(x_perm, "x_perm", torch.bfloat16, (cap, d), dev)
    _want(offsets, "offsets", torch.int32, (E + 1,), dev)
    _want(w_ug, "w_ug", torch.bfloat16, (E, 2 * h, d), dev)
    h_buf = _out(h_buf, "h_buf", torch.bfloat16, (cap, h), dev)
    _check(load_library().moe_gemm_up_swiglu(_ptr(x_perm), _ptr(offsets), _ptr(w_ug), cap, d, h, E, _ptr(h_buf),
                                  _stream(x_perm)), "moe_gemm_up_swiglu")
    return h_buf


def moe_gemm_up_swiglu_u(x_perm: torch.Tensor, offsets: torch.Tensor, w_ug: torch.Tensor, *, h_buf=None,
                         u_buf=None) -> tuple[torch.Tensor, torch.Tensor]:
    """moe_gemm_up_swiglu that also stores the pre-activation u_buf = [G | U] = bf16(x_perm[rows_e] @ W_ug[e]^T)
    ([cap, 2h], gate block first) for the backward; returns (h_buf, u_buf). One launch."""
    cap, dev = _gemm_shapes(x_perm, offsets, w_ug)
    E, two_h, d = w_ug.shape
    h = two_h // 2
    _want(x_perm, "x_perm", torch.bfloat16, (cap, d), dev)
    _want(offsets, "offsets", torch.int32, (E + 1,), dev)
    _want(w_ug, "w_ug", torch.bfloat16, (E, 2 * h, d), dev)
    h_buf = _out(h_buf, "h_buf", torch.bfloat16, (cap, h), dev)
    u_buf = _out(u_buf, "u_buf", torch.bfloat16, (cap, 2 * h), dev)
    _check(load_library().moe_gemm_up_swiglu_u(_ptr(x_perm), _ptr(offsets), _ptr(w_ug), cap, d, h, E, _ptr(h_buf),
                                               _ptr(u_buf), _stream(x_perm)), "moe_gemm_up_swiglu_u")
    return h_buf, u_buf


def moe_gemm_up_swiglu_gather(x: torch.Tensor, perm: torch.Tensor, offsets: torch.Tensor, w_ug: torch.Tensor,
                              k: int, *, h_buf=None) -> torch.Tensor:
    """moe_gemm_up_swiglu on token rows gathered through perm: sorted row p reads x[perm[p] // k] (one launch)."""
    if x.dim() != 2 or w_ug.dim() != 3:
        raise ValueError("expected x [T, d] and w_ug [E, 2h, d]")
    T, d = x.shape
    E, two_h, _ = w_ug.shape
    h = two_h // 2
    S = T * int(k)
    dev = x.device
    _want(x, "x", torch.bfloat16, (T, d), dev)
    _want(perm, "perm", torch.int32, (S,), dev)
    _want(offsets, "offsets", torch.int32, (E + 1,), dev)
    _want(w_ug, "w_ug", torch.bfloat16, (E, 2 * h, d), dev)
    h_buf = _out(h_buf, "h_buf", torch.bfloat16, (S, h), dev)
    _check(load_library().moe_gemm_up_swiglu_gather(_ptr(x), _ptr(perm), T, int(k), _ptr(offsets), _ptr(w_ug), d, h,
                                                    E, _ptr(h_buf), _stream(x)), "moe_gemm_up_swiglu_gather")
    return h_buf


def grouped_swiglu_expert_gather(x: torch.Tensor, perm: torch.Tensor, offsets: torch.Tensor, w_ug: torch.Tensor,
                                 w_down: torch.Tensor, k: int, *, h_buf=None, y_perm=None):
    """grouped_swiglu_expert with the permuted gather fused into the gate/up loads: returns (h_buf, y_perm)."""
    if x.dim() != 2 or w_ug.dim() != 3 or w_down.dim() != 3:
        raise ValueError("expected x [T, d], w_ug [E, 2h, d], w_down [E, h, d]")
    T, d = x.shape
    E, two_h, _ = w_ug.shape
    h = two_h // 2
    S = T * int(k)
    dev = x.device
    _want(x, "x", torch.bfloat16, (T, d), dev)
    _want(perm, "perm", torch.int32, (S,), dev)
    _want(offsets, "offsets", torch.int32, (E + 1,), dev)
    _want(w_ug, "w_ug", torch.bfloat16, (E, 2 * h, d), dev)
    _want(w_down, "w_down", torch.bfloat16, (E, h, d), dev)
    h_buf = _out(h_buf, "h_buf", torch.bfloat16, (S, h), dev)
    y_perm = _out(y_perm, "y_perm", torch.bfloat16, (S, d), dev)
    _check(load_library().grouped_swiglu_expert_gather(_ptr(x), _ptr(perm), T, int(k), _ptr(offsets), _ptr(w_ug),
                                                       _ptr(w_down), d, h, E, _ptr(h_buf), _ptr(y_perm), _stream(x)),
           "grouped_swiglu_expert_gather")
    return h_buf, y_perm


def moe_gemm_down(h_buf: torch.Tensor, offsets: torch.Tensor, w_down: torch.Tensor, *, y_perm=None) -> torch.Tensor:
    """y_perm[rows_e] = bf16(h_buf[rows_e] @ W_down[e]) (one launch)."""
    cap, dev = _gemm_shapes(h_buf, offsets, w_down)
    E, h, d = w_down.shape
    _want(h_buf, "h_buf", torch.bfloat16, (cap, h), dev)
    _want(offsets, "offsets", torch.int32, (E + 1,), dev)
    _want(w_down, "w_down", torch.bfloat16, (E, h, d), dev)
    y_perm = _out(y_perm, "y_perm", torch.bfloat16, (cap, d), dev)
    _check(load_library().moe_gemm_down(_ptr(h_buf), _ptr(offsets), _ptr(w_down), cap, d, h, E, _ptr(y_perm), _stream(h_buf)),
           "moe_gemm_down")
    return y_perm


def grouped_swiglu_expert(x_perm: torch.Tensor, offsets: torch.Tensor, w_ug: torch.Tensor, w_down: torch.Tensor, *,
                          h_buf=None, y_perm=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Eq 13 for every expert's row block: returns (h_buf, y_perm), both [cap, *] with rows [0, M) valid."""
    cap, dev = _gemm_shapes(x_perm, offsets, w_ug)
    E, two_h, d = w_ug.shape
    h = two_h // 2
    _want(x_perm, "x_perm", torch.bfloat16, (cap, d), dev)
    _want(offsets, "offsets", torch.int32, (E + 1,), dev)
    _want(w_ug, "w_ug", torch.bfloat16, (E, 2 * h, d), dev)
    _want(w_down, "w_down", torch.bfloat16, (E, h, d), dev)
    h_buf = _out(h_buf, "h_buf", torch.bfloat16, (cap, h), dev)
    y_perm = _out(y_perm, "y_perm", torch.bfloat16, (cap, d), dev)
    _check(load_library().grouped_swiglu_expert(_ptr(x_perm), _ptr(offsets), _ptr(w_ug), _ptr(w_down), cap, d, h, E,
                                     _ptr(h_buf), _ptr(y_perm), _stream(x_perm)), "grouped_swiglu_expert")
    return h_buf, y_perm


def moe_unpermute(y_perm: torch.Tensor, inv_map: torch.Tensor, routing_w: torch.Tensor, *, y=None) -> torch.Tensor:
    """y[t] = bf16(sum_j w[t,j] * y_perm[inv_map[t,j]]) over kept slots (atomic-free gather + reduce)."""
    if inv_map.dim() != 2:
        raise ValueError("inv_map must be [T, k]")
    T, k = inv_map.shape
    dev = y_perm.device
    d = y_perm.shape[1]
    _want(y_perm, "y_perm", torch.bfloat16, (T * k, d), dev)
    _want(inv_map, "inv_map", torch.int32, (T, k), dev)
    _want(routing_w, "routing_w", torch.float32, (T, k), dev)
    y = _out(y, "y", torch.bfloat16, (T, d), dev)
    _check(load_library().moe_unpermute(_ptr(y_perm), _ptr(inv_map), _ptr(routing_w), T, k, d, _ptr(y), _stream(y_perm)),
           "moe_unpermute")
    return y


def _w_dims(w: torch.Tensor, layout: str):
    if layout not in W_LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(W_LAYOUTS)}, got {layout!r}")
    if w.dim() != 3:
        raise ValueError("expert weights must be 3-D")
    E, a, b = w.shape
    return (E, a, b) if layout == "in_out" else (E, b, a)  # E, d_in, d_out


def moe_grouped_projection(x: torch.Tensor, offsets: torch.Tensor, w: torch.Tensor, layout: str = "in_out", *,
                           y=None) -> torch.Tensor:
    """Y[rows_e] = bf16(X[rows_e] @ W_e) with W_e [d_in, d_out] stored per ``layout`` (one launch)."""
    E, d_in, d_out = _w_dims(w, layout)
    if x.dim() != 2:
        raise ValueError("x must be [cap_rows, d_in]")
    cap, dev = x.shape[0], x.device
    _want(x, "x", torch.bfloat16, (cap, d_in), dev)
    _want(offsets, "offsets", torch.int32, (E + 1,), dev)
    _want(w, "w", torch.bfloat16, tuple(w.shape), dev)
    y = _out(y, "y", torch.bfloat16, (cap, d_out), dev)
    _check(load_library().moe_grouped_projection(_ptr(x), _ptr(offsets), _ptr(w), W_LAYOUTS[layout], cap, d_in, d_out,
                                                 E, _ptr(y), _stream(x)), "moe_grouped_projection")
    return y


def moe_swiglu_backward(dh: torch.Tensor, u: torch.Tensor, offsets: torch.Tensor, *, du=None) -> torch.Tensor:
    """dU = [dG | dUp] of H = SiLU(G) * Up over the sorted rows [0, offsets[E]) (one launch)."""
    if dh.dim() != 2 or u.dim() != 2 or offsets.dim() != 1:
        raise ValueError("expected dh [cap, h], u [cap, 2h] and offsets [E+1]")
    cap, h = dh.shape
    E = offsets.shape[0] - 1
    dev = dh.device
    _want(dh, "dh", torch.bfloat16, (cap, h), dev)
    _want(u, "u", torch.bfloat16, (cap, 2 * h), dev)
    _want(offsets, "offsets", torch.int32, (E + 1,), dev)
    du = _out(du, "du", torch.bfloat16, (cap, 2 * h), dev)
    _check(load_library().moe_swiglu_backward(_ptr(dh), _ptr(u), _ptr(offsets), E, cap, h, _ptr(du), _stream(dh)),
           "moe_swiglu_backward")
    return du


def moe_expert_backward(dy: torch.Tensor, p: "Permuted", routing_w: torch.Tensor, w_ug: torch.Tensor,
                        w_down: torch.Tensor, h_buf: torch.Tensor, y_perm: torch.Tensor, u: torch.Tensor | None = None
                        ) -> dict:
    """The expert step's backward from its forward tensors (``p`` must hold x_perm): returns dx,
    d_routing_w, dw_ug, dw_down. ``u`` is the pre-activation kept by moe_gemm_up_swiglu_u; without it, U is
    recomputed with the gate/up projection. Every step is one of the library's calls above."""
    if p.x_perm is None:
        raise ValueError("the backward needs the permuted rows: run moe_permute with gather=True")
    dy_perm, d_rw = moe_unpermute_backward(dy, y_perm, p.inv_map, routing_w)
    dh = moe_grouped_dgrad(dy_perm, p.offsets, w_down, "in_out")
    dw_down = moe_grouped_wgrad(h_buf, dy_perm, p.offsets, "in_out")
    if u is None:
        u = moe_grouped_projection(p.x_perm, p.offsets, w_ug, "out_in")
    du = moe_swiglu_backward(dh, u, p.offsets)
    dx_perm = moe_grouped_dgrad(du, p.offsets, w_ug, "out_in")
    dw_ug = moe_grouped_wgrad(p.x_perm, du, p.offsets, "out_in")
    dx = moe_permute_backward(dx_perm, p.inv_map)
    return {"dx": dx, "d_routing_w": d_rw, "dw_ug": dw_ug, "dw_down": dw_down, "dy_perm": dy_perm, "dh": dh,
            "u": u, "du": du, "dx_perm": dx_perm}


def moe_grouped_dgrad(dy: torch.Tensor, offsets: torch.Tensor, w: torch.Tensor, layout: str = "in_out", *,
                      dx=None) -> torch.Tensor:
    """dX[rows_e] = bf16(dY[rows_e] @ W_e^T) for the projection Y_e = X_e W_e (one launch)."""
    E, d_in, d_out = _w_dims(w, layout)
    if dy.dim() != 2:
        raise ValueError("dy must be [cap_rows, d_out]")
    cap, dev = dy.shape[0], dy.device
    _want(dy, "dy", torch.bfloat16, (cap, d_out), dev)
    _want(offsets, "offsets", torch.int32, (E + 1,), dev)
    _want(w, "w", torch.bfloat16, tuple(w.shape), dev)
    dx = _out(dx, "dx", torch.bfloat16, (cap, d_in), dev)
    _check(load_library().moe_grouped_dgrad(_ptr(dy), _ptr(offsets), _ptr(w), W_LAYOUTS[layout], cap, d_in, d_out, E,
                                            _ptr(dx), _stream(dy)), "moe_grouped_dgrad")
    return dx


def wgrad_workspace_bytes(cap_rows: int, d_in: int, d_out: int, E: int) -> int:
    return int(load_library().moe_grouped_wgrad_workspace_bytes(cap_rows, d_in, d_out, E))


def moe_grouped_wgrad(x: torch.Tensor, dy: torch.Tensor, offsets: torch.Tensor, layout: str = "in_out", *,
                      dw=None, workspace=None) -> torch.Tensor:
    """dW_e = bf16(X[rows_e]^T @ dY[rows_e]) in the weight's layout; zeros for experts with no rows (one launch)."""
    if x.dim() != 2 or dy.dim() != 2 or offsets.dim() != 1:
        raise ValueError("expected x [cap, d_in], dy [cap, d_out] and offsets [E+1]")
    cap, d_in = x.shape
    d_out = dy.shape[1]
    E = offsets.shape[0] - 1
    dev = x.device
    _want(x, "x", torch.bfloat16, (cap, d_in), dev)
    _want(dy, "dy", torch.bfloat16, (cap, d_out), dev)
    _want(offsets, "offsets", torch.int32, (E + 1,), dev)
    if layout not in W_LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(W_LAYOUTS)}, got {layout!r}")
    shape = (E, d_in, d_out) if layout == "in_out" else (E, d_out, d_in)
    dw = _out(dw, "dw", torch.bfloat16, shape, dev)
    need = wgrad_workspace_bytes(cap, d_in, d_out, E)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    if (workspace.device != dev or not workspace.is_contiguous()
            or workspace.numel() * workspace.element_size() < need):
        raise ValueError(f"workspace must be a contiguous tensor of at least {need} bytes on {dev}")
    _check(load_library().moe_grouped_wgrad(_ptr(x), _ptr(dy), _ptr(offsets), W_LAYOUTS[layout], cap, d_in, d_out, E,
                                            _ptr(dw), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _stream(x)), "moe_grouped_wgrad")
    return dw


def moe_permute_backward(dx_perm: torch.Tensor, inv_map: torch.Tensor, *, dx=None) -> torch.Tensor:
    """dX[t] = bf16(sum over kept j of dx_perm[inv_map[t, j]]) (gather + reduce, no atomics)."""
    if inv_map.dim() != 2:
        raise ValueError("inv_map must be [T, k]")
    T, k = inv_map.shape
    dev = dx_perm.device
    d = dx_perm.shape[1]
    _want(dx_perm, "dx_perm", torch.bfloat16, (T * k, d), dev)
    _want(inv_map, "inv_map", torch.int32, (T, k), dev)
    dx = _out(dx, "dx", torch.bfloat16, (T, d), dev)
    _check(load_library().moe_permute_backward(_ptr(dx_perm), _ptr(inv_map), T, k, d, _ptr(dx), _stream(dx_perm)),
           "moe_permute_backward")
    return dx


def moe_unpermute_backward(dy: torch.Tensor, y_perm: torch.Tensor, inv_map: torch.Tensor, routing_w: torch.Tensor, *,
                           dy_perm=None, d_routing_w=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Backward of moe_unpermute: (dy_perm with rows inv_map[t, j] = bf16(w[t, j] * dy[t]), d_routing_w fp32)."""
    if inv_map.dim() != 2:
        raise ValueError("inv_map must be [T, k]")
    T, k = inv_map.shape
    dev = dy.device
    d = dy.shape[1]
    _want(dy, "dy", torch.bfloat16, (T, d), dev)
    _want(y_perm, "y_perm", torch.bfloat16, (T * k, d), dev)
    _want(inv_map, "inv_map", torch.int32, (T, k), dev)
    _want(routing_w, "routing_w", torch.float32, (T, k), dev)
    dy_perm = _out(dy_perm, "dy_perm", torch.bfloat16, (T * k, d), dev)
    d_routing_w = _out(d_routing_w, "d_routing_w", torch.float32, (T, k), dev)
    _check(load_library().moe_unpermute_backward(_ptr(dy), _ptr(y_perm), _ptr(inv_map), _ptr(routing_w), T, k, d,
                                                 _ptr(dy_perm), _ptr(d_routing_w), _stream(dy)),
           "moe_unpermute_backward")
    return dy_perm, d_routing_w


def moe_expert_forward(x, expert_ids, routing_w, w_ug, w_down, fused_gather: bool = False):
    """The whole step: permute, grouped SwiGLU expert, unpermute. Returns (y, Permuted, h_buf, y_perm).

    ``fused_gather=True`` skips x_perm: the gate/up GEMM reads X through perm.
    """
    p = moe_permute(x, expert_ids, w_ug.shape[0], gather=not fused_gather)
    if fused_gather:
        h_buf, y_perm = grouped_swiglu_expert_gather(x, p.perm, p.offsets, w_ug, w_down, expert_ids.shape[1])
    else:
        h_buf, y_perm = grouped_swiglu_expert(p.x_perm, p.offsets, w_ug, w_down)
    y = moe_unpermute(y_perm, p.inv_map, routing_w)
    return y, p, h_buf, y_perm


__all__ = [
    "LIB_PATH", "MAX_EXPERTS", "MoeError", "Permuted", "grouped_swiglu_expert", "header_functions", "load_library",
    "grouped_swiglu_expert_gather", "moe_expert_forward", "moe_gemm_down", "moe_gemm_up_swiglu",
    "moe_gemm_up_swiglu_gather", "moe_gemm_up_swiglu_u", "moe_permute", "moe_permute_noalloc", "moe_unpermute",
    "permute_workspace_bytes", "W_LAYOUTS", "moe_grouped_dgrad", "moe_grouped_wgrad", "moe_permute_backward", "wgrad_workspace_bytes",
    "moe_grouped_projection", "moe_swiglu_backward", "moe_expert_backward",
    "moe_unpermute_backward",
]
