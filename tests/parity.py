"""Comparison helpers shared by the tests (no GPU and no oracle code in here).

The contract for bf16 outputs is elementwise ``|got - ref| <= atol + rtol*|ref|``
with atol = rtol = 1e-2. At the workloads' value scales (outputs of order 1e-4
for the Qwen3-shaped layer) that bound would accept an all-zero output, so two
guards that scale with the data are checked as well:

* relative L2 error ``||got - ref||_2 / ||ref||_2 <= 1e-2``;
* ``max |got - ref| <= 1e-2 * max |ref|``.

bf16 rounding of the stored intermediates changes an element by about 2^-8 of
its magnitude, so both guards hold with margin for a correct kernel while a
zero output or a swapped pair of experts fails them.
"""

from __future__ import annotations

import numpy as np

ATOL = 1e-2
RTOL = 1e-2
REL_L2 = 1e-2
REL_MAX = 1e-2

# The stored SwiGLU activations H = bf16(SiLU(g) * u) are not held to the oracle's H
# directly with the elementwise bound: g and u are themselves bf16 roundings of fp32 sums
# whose order differs between the kernel and the oracle, and a one-step flip in either is
# amplified by SiLU's slope 1 + g(1 - sigmoid(g)) (up to about 1.28) before H is rounded
# again. The check is split at U instead:
#   * U (stored by the U-keeping launch, whose h_buf must equal the plain launch's bit for
#     bit) is held to the oracle's U with the elementwise contract bound;
#   * H is held to the oracle's SwiGLU of the GPU's own U. Both sides evaluate SiLU(g) * u
#     in fp32 from the same bf16 g and u; the kernel's hardware exponential and reciprocal
#     differ from the oracle's by a few fp32 ulps, which moves the bf16 rounding of H by one
#     step only where the fp32 value lies within those few ulps of a rounding boundary:
#     at most H_MAX_ULP steps, and (a few times 2^-24 against a bf16 step of 2^-8, about
#     1e-4 of the elements at most) at least H_MIN_EXACT of the elements bit-identical
#     (small outputs may hold up to H_MIN_FLIPS differing elements).
H_MAX_ULP = 1
H_MIN_EXACT = 0.999
H_MIN_FLIPS = 4


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_ordinal(bits) -> np.ndarray:
    """Map bf16 bit patterns to integers whose difference counts ulps (signed zeros coincide)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_diff(a_bits, b_bits) -> np.ndarray:
    return np.abs(bf16_ordinal(a_bits) - bf16_ordinal(b_bits))


def compare_bf16(got_bits, ref_bits, what: str = "output", atol=ATOL, rtol=RTOL, rel_l2=REL_L2,
                 rel_max=REL_MAX, elementwise: bool = True) -> dict:
    """Check bf16 outputs against the reference; raise AssertionError with a summary on failure.

    ``elementwise=False`` keeps only the two data-scaled guards (relative L2 and max-abs against
    max|ref|); it is for results chained through several bf16-rounded intermediates, where one
    rounding decided differently upstream is multiplied by an unrelated operand downstream."""
    got = bf16_to_f64(got_bits)
    ref = bf16_to_f64(ref_bits)
    if got.shape != ref.shape:
        raise AssertionError(f"{what}: shape {got.shape} != reference {ref.shape}")
    if not np.all(np.isfinite(got)):
        raise AssertionError(f"{what}: {int((~np.isfinite(got)).sum())} non-finite values")
    diff = np.abs(got - ref)
    stats = {
        "n": int(ref.size),
        "max_abs_err": float(diff.max()) if diff.size else 0.0,
        "max_abs_ref": float(np.abs(ref).max()) if ref.size else 0.0,
        "exact_frac": float(np.mean(np.asarray(got_bits) == np.asarray(ref_bits))) if ref.size else 1.0,
        "max_ulp": int(ulp_diff(got_bits, ref_bits).max()) if ref.size else 0,
    }
    if ref.size == 0:
        return stats
    bad = diff > atol + rtol * np.abs(ref) if elementwise else np.zeros(diff.shape, dtype=bool)
    if np.any(bad):
        i = int(np.flatnonzero(bad.reshape(-1))[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside atol+rtol*|ref| "
                             f"(first flat index {i}: got {got.reshape(-1)[i]!r} ref {ref.reshape(-1)[i]!r})")
    ref_norm = float(np.linalg.norm(ref))
    err_norm = float(np.linalg.norm(got - ref))
    stats["rel_l2"] = err_norm / ref_norm if ref_norm > 0 else (0.0 if err_norm == 0 else float("inf"))
    if ref_norm == 0.0:
        if err_norm != 0.0:
            raise AssertionError(f"{what}: reference is all zero but output is not")
        return stats
    if stats["rel_l2"] > rel_l2:
        raise AssertionError(f"{what}: relative L2 error {stats['rel_l2']:.3e} > {rel_l2:g}")
    if stats["max_abs_err"] > rel_max * stats["max_abs_ref"]:
        raise AssertionError(f"{what}: max abs error {stats['max_abs_err']:.3e} > {rel_max:g} * "
                             f"max|ref| {stats['max_abs_ref']:.3e}")
    return stats


def assert_fails(fn, *args, **kwargs) -> None:
    """The comparison must reject this input (used for the negative controls)."""
    try:
        fn(*args, **kwargs)
    except AssertionError:
        return
    raise AssertionError("negative control was accepted by the comparison")


def compare_swiglu_of_u(h_bits, h_from_u_bits, what: str = "h_buf vs SwiGLU(U)") -> dict:
    """H against the SwiGLU of the same U: at most H_MAX_ULP bf16 steps apart, at least H_MIN_EXACT identical."""
    h_bits = np.asarray(h_bits, dtype=np.uint16)
    h_from_u_bits = np.asarray(h_from_u_bits, dtype=np.uint16)
    if h_bits.shape != h_from_u_bits.shape:
        raise AssertionError(f"{what}: shape {h_bits.shape} != {h_from_u_bits.shape}")
    if h_bits.size == 0:
        return {"n": 0}
    u = ulp_diff(h_bits, h_from_u_bits)
    exact = float(np.mean(u == 0))
    stats = {"n": int(u.size), "max_ulp": int(u.max()), "exact_frac": exact}
    if stats["max_ulp"] > H_MAX_ULP:
        i = int(np.argmax(u.reshape(-1)))
        raise AssertionError(f"{what}: {stats['max_ulp']} bf16 steps apart at flat index {i}")
    flips = int((u != 0).sum())
    if flips > max(H_MIN_FLIPS, (1.0 - H_MIN_EXACT) * u.size):
        raise AssertionError(f"{what}: {flips} of {u.size} elements differ (only {exact:.5f} identical)")
    return stats
