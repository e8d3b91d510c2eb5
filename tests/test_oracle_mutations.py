"""Planted mistakes in the oracle must be caught by at least one pin.

Each case swaps one oracle function (on the CPU, in this process only) for a
copy carrying a plausible mistake: a dropped term, a wrong sign, a wrong index,
a transposed operand, a missing rounding point, an unstable order. The pins
are then run; the case passes only if some pin rejects the mutated oracle.
"""

import numpy as np
import pytest

import oracle
import oracle.moe as om
from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits, round_to_bf16
from oracle_pins import ALL_PINS


def _swiglu_variant(gate_up_swapped=False, round_u=True, use_up=True, transpose_down=False, silu_sign=1.0):
    def f(a, w_ug, w_down, h, ft):
        u_full = np.matmul(a, w_ug.T)
        if round_u:
            u_full = round_to_bf16(u_full)
        g = u_full[:, :h].astype(ft)
        u = u_full[:, h:].astype(ft)
        if gate_up_swapped:
            g, u = u, g
        act = g / (ft(1) + np.exp(-silu_sign * g))
        hid = round_to_bf16(act * u if use_up else act)
        wd = w_down.T if transpose_down else w_down
        return hid, round_to_bf16(np.matmul(hid.astype(ft), wd)), u_full
    return f


def _swiglu_values_sign(u_full, h, ft):
    # the stand-alone activation step with SiLU's sign flipped (SiLU(-g) in place of SiLU(g))
    g = u_full[:, :h].astype(ft)
    u = u_full[:, h:].astype(ft)
    return round_to_bf16(g / (ft(1) + np.exp(g)) * u)


def _expert_forward_shifted(x_perm_bits, offsets, w_ug_bits, w_down_bits, precision="f32", return_u=False):
    # wrong weight index: expert e multiplied by expert (e+1)'s weights
    E = w_ug_bits.shape[0]
    if E > 1:
        w_ug_bits, w_down_bits = np.roll(w_ug_bits, -1, axis=0), np.roll(w_down_bits, -1, axis=0)
    return _orig_expert_forward(x_perm_bits, offsets, w_ug_bits, w_down_bits, precision, return_u)


def _eq16_ceil_inner(c, Mbar, M_E):
    # Eq 16 with the inner floor taken as a ceiling
    from fractions import Fraction
    import math
    inner = math.ceil(Fraction(str(c)) * Fraction(str(Mbar)) / int(M_E))
    return int(M_E) * 8 * math.ceil(Fraction(inner, 8))


def _eq16_rank_factor_dropped(c, Mbar, M_E):
    # Eq 16 without the outer factor M_E (one rank's share returned as the capacity)
    from fractions import Fraction
    import math
    inner = math.floor(Fraction(str(c)) * Fraction(str(Mbar)) / int(M_E))
    return 8 * math.ceil(Fraction(inner, 8))


def _eq16_share_undivided(c, Mbar, M_E):
    # Eq 16 aligning c * Mbar itself instead of each rank's share of it
    from fractions import Fraction
    import math
    inner = math.floor(Fraction(str(c)) * Fraction(str(Mbar)))
    return int(M_E) * 8 * math.ceil(Fraction(inner, 8))


_orig_expert_forward = om.expert_forward
_orig_stable = om.stable_route_order
_orig_unpermute = om.unpermute


def _reverse_within_expert(expert_ids, E, offsets):
    perm, inv = _orig_stable(expert_ids, E, offsets)
    offs = np.asarray(offsets)
    for e in range(E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        perm[lo:hi] = perm[lo:hi][::-1].copy()
    valid = inv >= 0
    inv[np.asarray(perm[: int(offs[-1])])] = np.arange(int(offs[-1]), dtype=np.int32)
    return perm, np.where(valid, inv, -1).astype(np.int32)


def _hist_clip(expert_ids, E):
    ids = np.asarray(expert_ids).reshape(-1)
    ids = ids[ids >= 0]
    return np.bincount(np.minimum(ids, E - 1), minlength=E).astype(np.int32)


def _offsets_inclusive(counts):
    c = np.cumsum(np.asarray(counts, dtype=np.int64))
    return np.concatenate([c, c[-1:]]).astype(np.int32)


def _unpermute_unweighted(y_perm_bits, inv, routing_w, T, k, precision="f32"):
    return _orig_unpermute(y_perm_bits, inv, np.ones_like(np.asarray(routing_w)), T, k, precision)


def _truncate_bf16(x):
    x = np.asarray(x, dtype=np.float64).astype(np.float32)
    return ((x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)).astype(np.float64)


_orig_projection = om.grouped_projection


def _projection_shifted(a_bits, offsets, w_bits, precision="f32"):
    # wrong weight index: expert e multiplied by expert (e+1)'s weights
    return _orig_projection(a_bits, offsets, np.roll(np.asarray(w_bits), -1, axis=0), precision)


def _projection_rows_shifted(a_bits, offsets, w_bits, precision="f32"):
    # off-by-one segment: every expert's block starts one row late
    offs = np.asarray(offsets).astype(np.int64).copy()
    offs[1:-1] += 1
    offs = np.minimum(offs, offs[-1])
    return _orig_projection(a_bits, offs, w_bits, precision)


def _projection_unrounded(a_bits, offsets, w_bits, precision="f32"):
    # the stored Y left in a truncating conversion instead of round-to-nearest-even
    offsets = np.asarray(offsets).astype(np.int64)
    out = np.zeros((int(offsets[-1]), np.asarray(w_bits).shape[2]), dtype=np.uint16)
    for e in range(offsets.shape[0] - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y = bf16_bits_to_f64(np.asarray(a_bits)[lo:hi]) @ bf16_bits_to_f64(np.asarray(w_bits)[e])
            out[lo:hi] = (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return out


import oracle.backward as ob

_orig_dgrad = ob.grouped_dgrad
_orig_wgrad = ob.grouped_wgrad
_orig_permute_bwd = ob.permute_backward
_orig_unpermute_bwd = ob.unpermute_backward


def _dgrad_no_transpose(dy_bits, offsets, w_bits, layout="in_out", precision="f64"):
    # the layout flag ignored: every weight read as [d_in, d_out]
    return _orig_dgrad(dy_bits, offsets, w_bits, "in_out", precision)


def _wgrad_shifted(x_bits, dy_bits, offsets, layout="in_out", precision="f64"):
    # each expert's gradient written to the next expert's slot
    return np.roll(_orig_wgrad(x_bits, dy_bits, offsets, layout, precision), 1, axis=0)


def _wgrad_rows_off_by_one(x_bits, dy_bits, offsets, layout="in_out", precision="f64"):
    # the contraction stops one row short of each expert's block
    offs = np.asarray(offsets).astype(np.int64)
    out = _orig_wgrad(x_bits, dy_bits, offs, layout, precision)
    for e in range(offs.shape[0] - 1):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi - lo >= 1:
            sub = np.array([0, hi - lo - 1], dtype=np.int64)
            out[e] = _orig_wgrad(np.asarray(x_bits)[lo:hi], np.asarray(dy_bits)[lo:hi], sub, layout, precision)[0]
    return out


def _permute_bwd_first_slot_only(dx_perm_bits, inv, T, k, precision="f64"):
    inv = np.asarray(inv).reshape(T, k).copy()
    inv[:, 1:] = -1
    return _orig_permute_bwd(dx_perm_bits, inv, T, k, precision)


_orig_swiglu_bwd = ob.swiglu_backward


def _swiglu_bwd_no_sigmoid_term(dh_bits, u_bits):
    # the sigmoid's own derivative dropped from dG
    dh = bf16_bits_to_f64(np.asarray(dh_bits, dtype=np.uint16))
    u_all = bf16_bits_to_f64(np.asarray(u_bits, dtype=np.uint16))
    h = dh.shape[1]
    g, up = u_all[:, :h], u_all[:, h:]
    s = 1.0 / (1.0 + np.exp(-g))
    return f64_to_bf16_bits(np.concatenate([dh * up * s, dh * g * s], axis=1))


def _swiglu_bwd_halves_swapped(dh_bits, u_bits):
    out = _orig_swiglu_bwd(dh_bits, u_bits)
    h = out.shape[1] // 2
    return np.concatenate([out[:, h:], out[:, :h]], axis=1)


def _unpermute_bwd_unweighted(dy_bits, y_perm_bits, inv, routing_w, T, k, M):
    return _orig_unpermute_bwd(dy_bits, y_perm_bits, inv, np.ones_like(np.asarray(routing_w)), T, k, M)


MUTATIONS = {
    "silu_sign": [("_swiglu_expert", _swiglu_variant(silu_sign=-1.0))],
    "gate_up_swapped": [("_swiglu_expert", _swiglu_variant(gate_up_swapped=True))],
    "u_not_rounded": [("_swiglu_expert", _swiglu_variant(round_u=False))],
    "up_term_dropped": [("_swiglu_expert", _swiglu_variant(use_up=False))],
    "down_transposed": [("_swiglu_expert", _swiglu_variant(transpose_down=True))],
    "wrong_expert_weights": [("expert_forward", _expert_forward_shifted)],
    "unstable_order": [("stable_route_order", _reverse_within_expert)],
    "out_of_range_ids_counted": [("route_histogram", _hist_clip)],
    "inclusive_offsets": [("exclusive_offsets", _offsets_inclusive)],
    "weights_ignored": [("unpermute", _unpermute_unweighted)],
    "truncating_rounding": [("round_to_bf16", _truncate_bf16)],
    "swiglu_step_sign": [("_swiglu_values", _swiglu_values_sign)],
    "eq16_ceil_inner": [("capacity_eq16", _eq16_ceil_inner)],
    "eq16_rank_factor_dropped": [("capacity_eq16", _eq16_rank_factor_dropped)],
    "eq16_share_undivided": [("capacity_eq16", _eq16_share_undivided)],
    "projection_wrong_expert": [("grouped_projection", _projection_shifted)],
    "projection_rows_shifted": [("grouped_projection", _projection_rows_shifted)],
    "projection_truncated": [("grouped_projection", _projection_unrounded)],
    "dgrad_layout_ignored": [("grouped_dgrad", _dgrad_no_transpose)],
    "wgrad_wrong_expert": [("grouped_wgrad", _wgrad_shifted)],
    "wgrad_row_short": [("grouped_wgrad", _wgrad_rows_off_by_one)],
    "permute_backward_one_slot": [("permute_backward", _permute_bwd_first_slot_only)],
    "unpermute_backward_unweighted": [("unpermute_backward", _unpermute_bwd_unweighted)],
    "swiglu_backward_sigmoid_term_dropped": [("swiglu_backward", _swiglu_bwd_no_sigmoid_term)],
    "swiglu_backward_halves_swapped": [("swiglu_backward", _swiglu_bwd_halves_swapped)],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    for attr, fn in MUTATIONS[name]:
        monkeypatch.setattr(ob if hasattr(ob, attr) and not hasattr(om, attr) else om, attr, fn)
        if hasattr(oracle, attr):
            monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(oracle)
        except Exception as exc:  # AssertionError, or a shape error from a transposed operand
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"planted mistake {name!r} passed every pin"
