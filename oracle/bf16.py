"""bfloat16 rounding for the oracle (test infrastructure only).

The method stores activations and weights as bf16 (1 sign bit, 8 exponent
bits with bias 127, 7 stored mantissa bits, so 8 significant bits for normal
numbers). The pages fix bf16 storage but not a rounding mode; the oracle uses
IEEE round-to-nearest, ties-to-even.

The rounding here is written from the definition of the format, not from a
bit trick: a finite value |x| in [2^(e-1), 2^e) has the bf16 spacing
2^(e-8) when it is in the normal range (|x| >= 2^-126) and the fixed
subnormal spacing 2^-133 below it; the rounded value is the nearest multiple
of that spacing, ties going to the even multiple (numpy's ``rint``).
"""

from __future__ import annotations

import numpy as np

_BF16_MIN_NORMAL_EXP = -125  # frexp exponent of 2^-126, the smallest bf16 normal
_BF16_SIG_BITS = 8  # significant bits of a normal bf16 (7 stored + hidden bit)
_BF16_SUBNORMAL_QUANTUM_EXP = -133  # 2^-126 * 2^-7
_BF16_OVERFLOW = 2.0**128  # anything that rounds to this magnitude is +-inf


def round_to_bf16(x) -> np.ndarray:
    """Round real values to the nearest bf16 value (ties to even), as float64.

    Input: any array-like of finite floats (float32 or float64). Output: a
    float64 array holding bf16-representable values (or +-inf on overflow).
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise FloatingPointError("oracle: non-finite value reached a bf16 rounding point")
    _, e = np.frexp(x)
    q = np.where(e >= _BF16_MIN_NORMAL_EXP, e - _BF16_SIG_BITS, _BF16_SUBNORMAL_QUANTUM_EXP)
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    return np.where(np.abs(r) >= _BF16_OVERFLOW, np.copysign(np.inf, r), r)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round to bf16 and return the 16-bit patterns (uint16)."""
    r = round_to_bf16(x).astype(np.float32)  # exact: every bf16 value is an fp32 value
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(b) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 values (exact)."""
    b = np.asarray(b, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # NaN patterns widen to NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
