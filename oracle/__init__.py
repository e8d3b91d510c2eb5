"""CPU oracle for the routed MoE expert step (test infrastructure only).

This package is the plain, slow, obviously correct CPU statement of what the
hot path computes. It exists to check the HIP library, nothing else: only the
test suite, the smoke check and the benchmark's CPU-baseline leg import it.
The HIP library and its Python binding never import, link or execute anything
from here, and this package imports nothing from them.

Sources (the three web pages the method is taken from):

* "Grouped expert GEMM: schedule irregular rows without changing the experts"
  (study.greatitself.com, expert-parallel training notes) -- FLOP convention,
  edge cases, the roofline lab.
* "Section 09: Grouped GEMM" of the OLMo-core MoE report (taotianhua.com) --
  Eq 13 (SwiGLU expert), Eq 14 (padding fraction), Figs 35-37 (the four-expert
  toy), Eq 16 (capacity), Eq 17 (column partition), Eq 18 (entropy deficit).
* "Grouped GEMM" engineering notes of the halo training toolkit (github) --
  drop of out-of-range expert ids before the sort, contiguous per-expert
  blocks, int32 cumulative offsets, the inverse map used by the atomic-free
  unpermute, the gate-then-up weight layout.

Numerics: the forward's per-expert loop runs in float32 on bf16-valued
operands by default, the precision in which the method states its
accumulation, and results are rounded to bf16 with round-to-nearest-even
exactly where the method stores a bf16 tensor. ``precision="f64"`` runs the
same loop in float64 (products of two bf16 values are exact there and sums of
a few thousand keep ~40 bits of headroom); the test suite pins the two against
each other within the float32 error bound. The backward's functions keep
float64 as their default.
"""

from .backward import (expert_backward, grouped_dgrad, grouped_wgrad, permute_backward, swiglu_backward,
                       unpermute_backward)
from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits, round_to_bf16
from .moe import (
    MoeOracleResult,
    capacity_ceil,
    capacity_eq16,
    entropy_deficit,
    exclusive_offsets,
    expert_forward,
    grouped_projection,
    moe_expert_forward,
    padding_fraction,
    permute_rows,
    route_histogram,
    stable_route_order,
    swiglu_rows,
    tile_count,
    token_forward,
    unpermute,
    useful_flops,
)

__all__ = [
    "MoeOracleResult",
    "bf16_bits_to_f64",
    "capacity_ceil",
    "capacity_eq16",
    "entropy_deficit",
    "exclusive_offsets",
    "expert_backward",
    "expert_forward",
    "f64_to_bf16_bits",
    "grouped_dgrad",
    "grouped_projection",
    "grouped_wgrad",
    "permute_backward",
    "unpermute_backward",
    "moe_expert_forward",
    "padding_fraction",
    "permute_rows",
    "round_to_bf16",
    "route_histogram",
    "stable_route_order",
    "swiglu_backward",
    "swiglu_rows",
    "tile_count",
    "token_forward",
    "unpermute",
    "useful_flops",
]
