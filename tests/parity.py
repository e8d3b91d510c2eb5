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

# The stored SwiGLU activations H = bf16(SiLU(g) * u) are formed from two values
# that were themselves rounded to bf16 (g and u, the halves of U). An fp32
# accumulation order different from the reference's can leave g and u each one
# bf16 step (at most 2^-7 relative) from the reference's, and H's own rounding
# adds another step; where SiLU(g) is large (g > 0) the three add up to
# 3 * 2^-7 relative. For g < 0 the relative sensitivity grows like |g| but
# |SiLU(g)| < 0.28, so the absolute bound covers it. y keeps the contract bound.
RTOL_H = 3 * 2.0**-7


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
