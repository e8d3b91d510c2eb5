"""Routed MoE expert step, forward, as a plain per-expert loop (test infrastructure only).

Each function follows one step of the method as the pages state it. Token
``t`` routed to its ``j``-th expert occupies the flat dispatch slot
``s = t*k + j`` (token-major), the order in which a dispatch buffer lists the
routes. Tensors of bf16 values are passed as uint16 bit patterns.

Readings taken where the pages are silent (each is listed in the design notes):

* Ids outside ``[0, E)`` -- the -1 padding of an expert-parallel dispatch, or
  any other out-of-range id -- are dropped before anything is counted
  (halo notes, expert-step paragraph).
* Inside an expert's contiguous block, routes keep ascending slot order: the
  order a stable sort by expert id returns (halo notes, expert-step paragraph;
  the tie-break itself is unstated).
* ``offsets`` has ``E+1`` int32 entries with ``offsets[0] = 0``; entries 1..E
  are the inclusive cumulative offsets the OLMo report prints for its toy
  ([1, 5, 8, 10] in Fig 37).
* SwiGLU(U) = SiLU(U[:, :h]) * U[:, h:], gate block first, SiLU(g) = g*sigmoid(g),
  no clamp (Eq 13 names SwiGLU; the halo notes chunk gate_up into gate then up
  and call the activation a standard SiLU gate).
* Rounding points: U is rounded to bf16 before SwiGLU; SiLU(g)*u is evaluated
  from the rounded g and u without rounding SiLU(g) on its own; H, each
  expert's Y_e and the combined token output y are rounded to bf16 because
  they are stored as bf16.
* Routing weights are float32 [T, k], applied at scatter-back, not
  renormalised when a slot is dropped; a token with no kept slot gets y = 0.
* Working precision: the forward's contractions, SiLU and the weighted sum
  run in float32 on bf16-valued operands by default, the accumulation
  precision the method names; ``precision="f64"`` runs the same loop in
  float64, and the test suite pins the two against each other within the
  float32 error bound.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits, round_to_bf16

_PRECISIONS = {"f64": np.float64, "f32": np.float32}


def _ftype(precision: str):
    try:
        return _PRECISIONS[precision]
    except KeyError:
        raise ValueError(f"precision must be one of {sorted(_PRECISIONS)}, got {precision!r}") from None


# --------------------------------------------------------------------------
# Dispatch preparation: histogram, offsets, stable order, permuted gather
# --------------------------------------------------------------------------


def route_histogram(expert_ids, E: int) -> np.ndarray:
    """Rows per local expert, ``counts[e] = #{s : ids[s] == e}`` (int32 [E]).

    OLMo report, Sec 9.2 / Fig 37 ("batchsize_per_expert", a device tensor);
    ids outside [0, E) are dropped first (halo notes, expert-step paragraph).
    """
    ids = np.asarray(expert_ids).reshape(-1)
    counts = [0] * E
    for e in ids.tolist():
        if 0 <= e < E:
            counts[e] += 1
    return np.asarray(counts, dtype=np.int32)


def exclusive_offsets(counts) -> np.ndarray:
    """``offsets[0] = 0``, ``offsets[e+1] = offsets[e] + counts[e]`` (int32 [E+1]).

    OLMo report, Fig 37 and Sec 9.3: the prefix sum of the counts, each value
    ending one expert's segment; the halo notes require int32 offsets.
    """
    offsets = [0]
    for c in np.asarray(counts).tolist():
        offsets.append(offsets[-1] + int(c))
    if offsets[-1] >= 2**31:
        raise OverflowError("offsets exceed int32")
    return np.asarray(offsets, dtype=np.int32)


def stable_route_order(expert_ids, E: int, offsets) -> tuple[np.ndarray, np.ndarray]:
    """Sorted position of every dispatch slot and its inverse.

    Walking the slots in ascending order, a kept slot of expert ``e`` takes the
    next free row of that expert's block, ``offsets[e] + (number of earlier
    slots of e)``. Returns ``perm`` (int32 [S]; ``perm[p]`` is the slot in
    sorted row ``p`` for ``p < M``, -1 beyond) and ``inv`` (int32 [S]; the
    sorted row of slot ``s``, or -1 for a dropped slot). halo notes: tokens are
    sorted into contiguous per-expert blocks, and the inverse map of sorted
    positions is sentinel-padded.
    """
    ids = np.asarray(expert_ids).reshape(-1).tolist()
    S = len(ids)
    offs = np.asarray(offsets).tolist()
    seen = [0] * E
    perm = [-1] * S
    inv = [-1] * S
    for s, e in enumerate(ids):
        if 0 <= e < E:
            pos = offs[e] + seen[e]
            seen[e] += 1
            perm[pos] = s
            inv[s] = pos
    return np.asarray(perm, dtype=np.int32), np.asarray(inv, dtype=np.int32)


def permute_rows(x_bits, perm, M: int, k: int) -> np.ndarray:
    """``x_perm[p] = X[perm[p] // k]`` for ``p < M`` (uint16 [M, d]).

    The forward gather of the token rows into expert-contiguous order (halo
    notes, permute paragraph).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    perm = np.asarray(perm)[:M].astype(np.int64)
    return x_bits[perm // k].copy()


# --------------------------------------------------------------------------
# Expert compute: Eq 13, one expert at a time
# --------------------------------------------------------------------------


def _silu(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return g / (g.dtype.type(1) + np.exp(-g))


def _swiglu_values(u_full: np.ndarray, h: int, ft) -> np.ndarray:
    """SwiGLU of bf16-valued pre-activations: ``bf16(SiLU(g) * u)`` with g = U[:, :h], u = U[:, h:].

    The gate block comes first (halo notes: gate_up chunked into gate, then
    up); SiLU(g) is not rounded on its own. Returns a bf16-valued float64 array.
    """
    g = u_full[:, :h].astype(ft)
    u = u_full[:, h:].astype(ft)
    return round_to_bf16(_silu(g) * u)


def _swiglu_expert(a: np.ndarray, w_ug: np.ndarray, w_down: np.ndarray, h: int, ft):
    """One expert, Eq 13: U = A W_ug^T, H = SwiGLU(U), Y = H W_down.

    ``a`` [m, d], ``w_ug`` [2h, d], ``w_down`` [h, d], all float arrays of
    bf16 values in the working precision ``ft``. Returns (H, Y, U) as
    bf16-valued float64 arrays.
    """
    u_full = round_to_bf16(np.matmul(a, w_ug.T))  # [m, 2h]
    hid = _swiglu_values(u_full, h, ft)  # [m, h]
    y = round_to_bf16(np.matmul(hid.astype(ft), w_down))  # [m, d]
    return hid, y, u_full


def swiglu_rows(u_bits, precision: str = "f32") -> np.ndarray:
    """The activation step of Eq 13 alone: ``H = bf16(SiLU(U[:, :h]) * U[:, h:])``.

    ``u_bits`` uint16 [rows, 2h] holds bf16 pre-activations, gate block first.
    Used to hold a stored activation to the SwiGLU of the pre-activation it was
    computed from. Returns uint16 [rows, h].
    """
    ft = _ftype(precision)
    u = bf16_bits_to_f64(np.asarray(u_bits, dtype=np.uint16))
    if u.ndim != 2 or u.shape[1] % 2:
        raise ValueError(f"U must be [rows, 2h], got {u.shape}")
    return f64_to_bf16_bits(_swiglu_values(u, u.shape[1] // 2, ft))


def expert_forward(x_perm_bits, offsets, w_ug_bits, w_down_bits, precision: str = "f32", return_u: bool = False):
    """Grouped SwiGLU expert step over the sorted rows (Eq 13 per expert).

    For every expert with ``counts[e] > 0`` its own weights multiply exactly
    its own block of rows ``[offsets[e], offsets[e+1])``; empty experts do no
    arithmetic (grouped-GEMM essay: distinct parameters per expert, zero-row
    experts need no matrix work). Returns ``(h_bits [M, h], y_perm_bits [M, d])``,
    and the bf16 pre-activation ``u_bits [M, 2h]`` (gate block, then up block)
    as a third entry when ``return_u``.
    """
    ft = _ftype(precision)
    offsets = np.asarray(offsets).astype(np.int64)
    E = offsets.shape[0] - 1
    M = int(offsets[E])
    w_ug_bits = np.asarray(w_ug_bits, dtype=np.uint16)
    w_down_bits = np.asarray(w_down_bits, dtype=np.uint16)
    two_h, d = w_ug_bits.shape[1], w_ug_bits.shape[2]
    h = two_h // 2
    x_perm = np.asarray(x_perm_bits, dtype=np.uint16)
    h_out = np.zeros((M, h), dtype=np.uint16)
    y_out = np.zeros((M, d), dtype=np.uint16)
    u_out = np.zeros((M, two_h), dtype=np.uint16) if return_u else None
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        a = bf16_bits_to_f64(x_perm[lo:hi]).astype(ft)
        wug = bf16_bits_to_f64(w_ug_bits[e]).astype(ft)
        wdn = bf16_bits_to_f64(w_down_bits[e]).astype(ft)
        hid, y, u_full = _swiglu_expert(a, wug, wdn, h, ft)
        h_out[lo:hi] = f64_to_bf16_bits(hid)
        y_out[lo:hi] = f64_to_bf16_bits(y)
        if return_u:
            u_out[lo:hi] = f64_to_bf16_bits(u_full)
    return (h_out, y_out, u_out) if return_u else (h_out, y_out)


def grouped_projection(a_bits, offsets, w_bits, precision: str = "f32") -> np.ndarray:
    """One grouped expert projection: ``Y[rows_e] = bf16(A[rows_e] @ W[e])`` per expert.

    The single-projection problem the OLMo report measures in Sec 9.6 (Figs 38
    and 40: one square bf16 expert projection per local expert over its own
    rows; Fig 39 / Eq 17: the experts' weights are column blocks of one dense
    weight). ``a_bits`` uint16 [>= M, K], ``offsets`` int [E+1], ``w_bits``
    uint16 [E, K, N] (row-major, the layout of a down projection). Rows of an
    expert with no rows are never touched. Returns uint16 [M, N].
    """
    ft = _ftype(precision)
    offsets = np.asarray(offsets).astype(np.int64)
    E = offsets.shape[0] - 1
    M = int(offsets[E])
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if w_bits.ndim != 3 or w_bits.shape[0] != E:
        raise ValueError(f"w must be [E={E}, K, N], got {w_bits.shape}")
    N = w_bits.shape[2]
    a_bits = np.asarray(a_bits, dtype=np.uint16)
    out = np.zeros((M, N), dtype=np.uint16)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        a = bf16_bits_to_f64(a_bits[lo:hi]).astype(ft)
        w = bf16_bits_to_f64(w_bits[e]).astype(ft)
        out[lo:hi] = f64_to_bf16_bits(np.matmul(a, w))
    return out


# --------------------------------------------------------------------------
# Scatter-back: atomic-free unpermute through the inverse map
# --------------------------------------------------------------------------


def unpermute(y_perm_bits, inv, routing_w, T: int, k: int, precision: str = "f32") -> np.ndarray:
    """``y[t] = bf16(sum_j w[t,j] * y_perm[inv[t,j]])`` over kept slots, j ascending.

    halo notes: the scatter-back is a gather through the inverse map followed
    by a reduction, with the routing weights applied here. Dropped slots
    (``inv == -1``) contribute nothing. Returns uint16 [T, d].
    """
    ft = _ftype(precision)
    inv = np.asarray(inv).reshape(T, k).astype(np.int64)
    w = np.asarray(routing_w, dtype=np.float32).reshape(T, k).astype(ft)
    yp = bf16_bits_to_f64(y_perm_bits).astype(ft)
    if yp.ndim != 2:
        raise ValueError("unpermute needs y_perm shaped [rows, d]")
    d = yp.shape[1]
    acc = np.zeros((T, d), dtype=ft)
    for j in range(k):
        col = inv[:, j]
        keep = col >= 0
        if np.any(keep):
            acc[keep] = acc[keep] + w[keep, j][:, None] * yp[col[keep]]
    return f64_to_bf16_bits(acc)


# --------------------------------------------------------------------------
# The whole forward step
# --------------------------------------------------------------------------


@dataclass
class MoeOracleResult:
    counts: np.ndarray  # int32 [E]
    offsets: np.ndarray  # int32 [E+1]
    perm: np.ndarray  # int32 [S]; defined for p < M, -1 beyond
    inv_map: np.ndarray  # int32 [T, k]; -1 on dropped slots
    x_perm: np.ndarray  # uint16 [M, d]
    h: np.ndarray  # uint16 [M, h]
    y_perm: np.ndarray  # uint16 [M, d]
    y: np.ndarray  # uint16 [T, d]
    u: np.ndarray | None = None  # uint16 [M, 2h], the bf16 pre-activation, when asked for

    @property
    def M(self) -> int:
        return int(self.offsets[-1])


def moe_expert_forward(x_bits, expert_ids, routing_w, w_ug_bits, w_down_bits, precision: str = "f32",
                       with_gemm: bool = True, keep_u: bool = False) -> MoeOracleResult:
    """Routed expert forward: histogram, offsets, stable order, gather, Eq 13, unpermute.

    Shapes: ``x_bits`` uint16 [T, d], ``expert_ids`` int [T, k],
    ``routing_w`` float32 [T, k], ``w_ug_bits`` uint16 [E, 2h, d] (gate rows
    [0, h), up rows [h, 2h)), ``w_down_bits`` uint16 [E, h, d].
    ``with_gemm=False`` stops after the gather (h, y_perm, y left empty);
    ``keep_u=True`` also returns the bf16 pre-activation U of every sorted row.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    ids = np.asarray(expert_ids)
    T, k = ids.shape
    E = np.asarray(w_ug_bits).shape[0]
    counts = route_histogram(ids, E)
    offsets = exclusive_offsets(counts)
    M = int(offsets[-1])
    perm, inv = stable_route_order(ids, E, offsets)
    x_perm = permute_rows(x_bits, perm, M, k)
    d = x_bits.shape[1]
    if not with_gemm:
        empty = np.zeros((0, 0), dtype=np.uint16)
        return MoeOracleResult(counts, offsets, perm, inv.reshape(T, k), x_perm, empty, empty, empty)
    out = expert_forward(x_perm, offsets, w_ug_bits, w_down_bits, precision, return_u=keep_u)
    h_bits, y_perm = out[0], out[1]
    y = unpermute(y_perm.reshape(M, d), inv, routing_w, T, k, precision)
    return MoeOracleResult(counts, offsets, perm, inv.reshape(T, k), x_perm, h_bits, y_perm, y,
                           out[2] if keep_u else None)


def token_forward(x_row_bits, ids_row, w_row, w_ug_bits, w_down_bits, precision: str = "f32") -> np.ndarray:
    """The same step for one token: its kept slots' experts applied to its row.

    Rows are independent in Eq 13, so a token's output needs only its own row
    and its own experts; this is the form used to check sampled tokens of
    workloads too large to run whole. Returns uint16 [d].
    """
    ft = _ftype(precision)
    w_ug_bits = np.asarray(w_ug_bits, dtype=np.uint16)
    E, two_h, d = w_ug_bits.shape
    h = two_h // 2
    a = bf16_bits_to_f64(np.asarray(x_row_bits, dtype=np.uint16).reshape(1, d)).astype(ft)
    acc = np.zeros((1, d), dtype=ft)
    for j, e in enumerate(np.asarray(ids_row).tolist()):
        if not 0 <= e < E:
            continue
        wug = bf16_bits_to_f64(w_ug_bits[e]).astype(ft)
        wdn = bf16_bits_to_f64(np.asarray(w_down_bits, dtype=np.uint16)[e]).astype(ft)
        _, y, _ = _swiglu_expert(a, wug, wdn, h, ft)
        acc = acc + ft(np.float32(w_row[j])) * y.astype(ft)
    return f64_to_bf16_bits(acc).reshape(d)


# --------------------------------------------------------------------------
# Side quantities the pages define
# --------------------------------------------------------------------------


def useful_flops(M: int, d: int, h: int) -> int:
    """Matrix work of a gated (SwiGLU) expert over M rows: 6*M*d*h.

    Grouped-expert essay, first paragraph: two FLOPs per multiply-add, two
    input projections and one output projection; nonlinearities, routing and
    the permutations add none.
    """
    return 6 * int(M) * int(d) * int(h)


def padding_fraction(counts, C: int, clip: bool = False) -> float:
    """Eq 14: rho_pad = 1 - sum_e M_e / (N_local * C).

    ``clip=True`` counts only the rows that fit, sum_e min(M_e, C), the
    useful rows a capacity-padded BMM actually executes when experts overflow
    (Fig 35's "routed row beyond C").
    """
    counts = np.asarray(counts, dtype=np.int64)
    useful = np.minimum(counts, C).sum() if clip else counts.sum()
    return float(1 - Fraction(int(useful), int(counts.shape[0]) * int(C)))


def capacity_ceil(c, M: int, N_local: int) -> int:
    """Sweep capacity C = ceil(c * Mbar) with Mbar = M / N_local (Fig 35; Sec 9.6 footnote 1)."""
    return math.ceil(Fraction(str(c)) * Fraction(int(M), int(N_local)))


def capacity_eq16(c, Mbar, M_E: int) -> int:
    """Eq 16: C = M_E * 8 * ceil(floor(c * Mbar / M_E) / 8), eight-row aligned per EP rank."""
    inner = math.floor(Fraction(str(c)) * Fraction(str(Mbar)) / int(M_E))
    return int(M_E) * 8 * math.ceil(Fraction(inner, 8))


def entropy_deficit(counts) -> float:
    """Eq 18: I_H = 1 - H(p) / log N_local, p_e = M_e / M, with 0 log 0 = 0.

    N_local counts every local expert, empty ones included. A single expert
    (log 1 = 0) is uniform by definition and returns 0. M = 0 returns 0.
    """
    counts = np.asarray(counts, dtype=np.float64)
    n = counts.shape[0]
    M = counts.sum()
    if n <= 1 or M == 0:
        return 0.0
    p = counts[counts > 0] / M
    H = -float(np.sum(p * np.log(p)))
    return 1.0 - H / math.log(n)


def tile_count(counts, block_rows: int, col_blocks: int) -> int:
    """Tiles of a device-scheduled grouped GEMM: sum_e ceil(M_e / block_rows) * col_blocks.

    Fig 37: the grouped kernel enumerates every problem's output tiles in one
    list (12 toy tiles at 2 rows x 2 column blocks); empty experts add none.
    """
    return sum(-(-int(m) // int(block_rows)) * int(col_blocks) for m in np.asarray(counts).tolist())
