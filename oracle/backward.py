"""Backward of one grouped projection and of the two permutations (test infrastructure only).

OLMo report, "Section 09: Grouped GEMM", Sec 9.5 (Eq 15, Table 15): for a
grouped projection Y_e = X_e W_e with X_e [M_e, d_in] and W_e [d_in, d_out],
the input gradient (Dgrad) is dX_e = dY_e W_e^T -- a forward-shaped grouped
problem with M_e as its output rows -- and the weight gradient (Wgrad) is
dW_e = X_e^T dY_e, which contracts over the ragged M_e. halo notes, "Grouped
GEMM", permute/unpermute paragraphs: the backward of a duplicate-valued row
gather is taken as a gather through the inverse map followed by a reduction,
never as an atomic scatter-add.

Weights come in one of two stored layouts: ``"in_out"`` is [E, d_in, d_out]
(the down projection's W_down [E, h, d]) and ``"out_in"`` is [E, d_out, d_in]
(the gate/up projection's W_ug [E, 2h, d], used transposed in the forward).

Readings taken where the pages are silent (each is listed in the design notes):

* Every gradient the step stores is bf16 (round-to-nearest-even of the exact
  sum), like the forward's stored tensors; the report's Wgrad path is a bf16
  grouped GEMM. Accumulation is exact here (float64 on bf16 values).
* An expert with no rows has dW_e = 0 (a contraction over nothing).
* The permute backward sums a token's kept slots, j ascending, with no weights
  (the forward permute copies rows unweighted); a token with no kept slot gets 0.
* The unpermute backward returns dy_perm[inv[t, j]] = bf16(w[t, j] * dy[t]) for
  kept slots (rows of dropped slots do not exist) and the routing-weight
  gradient dw[t, j] = sum_c dy[t, c] * y_perm[inv[t, j], c] in float32, 0 for
  dropped slots.
* The pages define the projections' backward, not the activation's: the
  SwiGLU backward here is the derivative of SiLU(g) * up with the forward's
  bf16 roundings taken as identities, evaluated from the stored bf16 U (which
  the backward recomputes as the forward projection X_e W_ug[e]^T).
"""

from __future__ import annotations

import numpy as np

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits
from .moe import _ftype

_LAYOUTS = ("in_out", "out_in")


def _w_in_out(w_e_f, layout: str):
    """One expert's weight as [d_in, d_out] (a view; no copy)."""
    if layout == "in_out":
        return w_e_f
    if layout == "out_in":
        return w_e_f.T
    raise ValueError(f"layout must be one of {_LAYOUTS}, got {layout!r}")


def grouped_dgrad(dy_bits, offsets, w_bits, layout: str = "in_out", precision: str = "f64") -> np.ndarray:
    """Eq 15, Dgrad: ``dX[rows_e] = bf16(dY[rows_e] @ W_e^T)`` for every expert with rows.

    ``dy_bits`` uint16 [>= M, d_out], ``offsets`` int [E+1], ``w_bits`` uint16 in
    ``layout``. Returns uint16 [M, d_in].
    """
    ft = _ftype(precision)
    offsets = np.asarray(offsets).astype(np.int64)
    E = offsets.shape[0] - 1
    M = int(offsets[E])
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if w_bits.ndim != 3 or w_bits.shape[0] != E:
        raise ValueError(f"w must be [E={E}, ., .], got {w_bits.shape}")
    d_in = w_bits.shape[1] if layout == "in_out" else w_bits.shape[2]
    dy = np.asarray(dy_bits, dtype=np.uint16)
    out = np.zeros((M, d_in), dtype=np.uint16)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        g = bf16_bits_to_f64(dy[lo:hi]).astype(ft)  # [m, d_out]
        w = _w_in_out(bf16_bits_to_f64(w_bits[e]).astype(ft), layout)  # [d_in, d_out]
        out[lo:hi] = f64_to_bf16_bits(np.matmul(g, w.T))
    return out


def grouped_wgrad(x_bits, dy_bits, offsets, layout: str = "in_out", precision: str = "f64") -> np.ndarray:
    """Eq 15, Wgrad: ``dW_e = bf16(X[rows_e]^T @ dY[rows_e])``, contracting over the expert's rows.

    ``x_bits`` uint16 [>= M, d_in], ``dy_bits`` uint16 [>= M, d_out]. Returns
    uint16 [E, d_in, d_out] (``"in_out"``) or [E, d_out, d_in] (``"out_in"``);
    experts with no rows get zeros.
    """
    ft = _ftype(precision)
    offsets = np.asarray(offsets).astype(np.int64)
    E = offsets.shape[0] - 1
    x = np.asarray(x_bits, dtype=np.uint16)
    dy = np.asarray(dy_bits, dtype=np.uint16)
    d_in, d_out = x.shape[1], dy.shape[1]
    if layout not in _LAYOUTS:
        raise ValueError(f"layout must be one of {_LAYOUTS}, got {layout!r}")
    shape = (E, d_in, d_out) if layout == "in_out" else (E, d_out, d_in)
    out = np.zeros(shape, dtype=np.uint16)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        xe = bf16_bits_to_f64(x[lo:hi]).astype(ft)  # [m, d_in]
        ge = bf16_bits_to_f64(dy[lo:hi]).astype(ft)  # [m, d_out]
        dw = np.matmul(xe.T, ge)  # [d_in, d_out]
        out[e] = f64_to_bf16_bits(dw if layout == "in_out" else dw.T)
    return out


def permute_backward(dx_perm_bits, inv, T: int, k: int, precision: str = "f64") -> np.ndarray:
    """Backward of the row gather ``x_perm[p] = X[perm[p] / k]``: ``dX[t] = bf16(sum_j dx_perm[inv[t, j]])``.

    Kept slots only, j ascending, unweighted (halo notes: gather through the
    inverse map plus a reduction instead of a scatter-add). Returns uint16 [T, d].
    """
    ft = _ftype(precision)
    inv = np.asarray(inv).reshape(T, k).astype(np.int64)
    g = bf16_bits_to_f64(dx_perm_bits).astype(ft)
    d = g.shape[1]
    acc = np.zeros((T, d), dtype=ft)
    for j in range(k):
        col = inv[:, j]
        keep = col >= 0
        if np.any(keep):
            acc[keep] = acc[keep] + g[col[keep]]
    return f64_to_bf16_bits(acc)


def unpermute_backward(dy_bits, y_perm_bits, inv, routing_w, T: int, k: int, M: int):
    """Backward of ``y[t] = sum_j w[t, j] * y_perm[inv[t, j]]``.

    Returns ``(dy_perm uint16 [M, d], dw float32 [T, k])`` with
    ``dy_perm[inv[t, j]] = bf16(w[t, j] * dy[t])`` and
    ``dw[t, j] = sum_c dy[t, c] * y_perm[inv[t, j], c]`` (0 on dropped slots).
    """
    inv = np.asarray(inv).reshape(T, k).astype(np.int64)
    w = np.asarray(routing_w, dtype=np.float32).reshape(T, k).astype(np.float64)
    dy = bf16_bits_to_f64(dy_bits)
    yp = bf16_bits_to_f64(y_perm_bits)
    d = dy.shape[1]
    dyp = np.zeros((M, d), dtype=np.float64)
    dw = np.zeros((T, k), dtype=np.float64)
    for j in range(k):
        col = inv[:, j]
        keep = col >= 0
        if np.any(keep):
            dyp[col[keep]] = w[keep, j][:, None] * dy[keep]
            dw[keep, j] = np.sum(dy[keep] * yp[col[keep]], axis=1)
    return f64_to_bf16_bits(dyp), dw.astype(np.float32)


def swiglu_backward(dh_bits, u_bits) -> np.ndarray:
    """Backward of H = SiLU(G) * Up with [G | Up] = U (gate block first, as in the forward).

    ``dh_bits`` uint16 [M, h], ``u_bits`` uint16 [M, 2h] (the stored, bf16-rounded
    pre-activation). With s = sigmoid(g): dG = dH * up * s * (1 + g * (1 - s)),
    dUp = dH * g * s, evaluated in float64 and rounded to bf16 (the forward's
    roundings are taken as identities, as autograd takes them). Returns uint16
    [M, 2h] laid out like U.
    """
    dh = bf16_bits_to_f64(np.asarray(dh_bits, dtype=np.uint16))
    u_all = bf16_bits_to_f64(np.asarray(u_bits, dtype=np.uint16))
    h = dh.shape[1]
    if u_all.shape[1] != 2 * h:
        raise ValueError(f"U must be [M, 2h] with h = {h}, got {u_all.shape}")
    g, up = u_all[:, :h], u_all[:, h:]
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-g))
    dg = dh * up * s * (1.0 + g * (1.0 - s))
    dup = dh * g * s
    return f64_to_bf16_bits(np.concatenate([dg, dup], axis=1))


def expert_backward(dy_bits, x_bits, expert_ids, routing_w, w_ug_bits, w_down_bits):
    """The expert step's backward, composed from the functions above (test infrastructure only).

    Recomputes the forward (oracle) to get the stored bf16 tensors, then:
    unpermute backward -> Dgrad/Wgrad of the down projection -> SwiGLU
    backward -> Dgrad/Wgrad of the gate/up projection -> permute backward.
    Returns a dict with dx [T, d], d_routing_w [T, k], dw_ug [E, 2h, d],
    dw_down [E, h, d] (uint16 bf16 bits, float32 for d_routing_w) and the
    intermediates dy_perm, dh, du, dx_perm.
    """
    from .moe import (exclusive_offsets, expert_forward, grouped_projection, permute_rows, route_histogram,
                      stable_route_order)

    x_bits = np.asarray(x_bits, dtype=np.uint16)
    ids = np.asarray(expert_ids)
    T, k = ids.shape
    w_ug_bits = np.asarray(w_ug_bits, dtype=np.uint16)
    w_down_bits = np.asarray(w_down_bits, dtype=np.uint16)
    E = w_ug_bits.shape[0]
    counts = route_histogram(ids, E)
    offsets = exclusive_offsets(counts)
    M = int(offsets[-1])
    perm, inv = stable_route_order(ids, E, offsets)
    x_perm = permute_rows(x_bits, perm, M, k)
    h_bits, y_perm = expert_forward(x_perm, offsets, w_ug_bits, w_down_bits, precision="f64")
    u_bits = grouped_projection(x_perm, offsets, np.swapaxes(w_ug_bits, 1, 2), precision="f64")  # U_e = bf16(X_e W_ug[e]^T)
    dy_perm, d_rw = unpermute_backward(dy_bits, y_perm, inv, routing_w, T, k, M)
    dh = grouped_dgrad(dy_perm, offsets, w_down_bits, "in_out")
    dw_down = grouped_wgrad(h_bits, dy_perm, offsets, "in_out")
    du = swiglu_backward(dh, u_bits)
    dx_perm = grouped_dgrad(du, offsets, w_ug_bits, "out_in")
    dw_ug = grouped_wgrad(x_perm, du, offsets, "out_in")
    dx = permute_backward(dx_perm, inv, T, k)
    return {"dx": dx, "d_routing_w": d_rw, "dw_ug": dw_ug, "dw_down": dw_down, "dy_perm": dy_perm, "dh": dh,
            "du": du, "dx_perm": dx_perm, "offsets": offsets, "inv_map": inv.reshape(T, k), "u": u_bits}
