"""Seeded synthetic inputs for the routed MoE expert step.

Both the oracle-side tests and the HIP-side tests and benchmark draw their
inputs from here, so this module holds input generation only: random expert
ids, routing weights, activations and weights. It contains none of the step's
own arithmetic (no histogram, scan, sort, GEMM, activation or reduction).

Every workload draws from ``numpy.random.default_rng(seed)`` (PCG64) in a
fixed order: expert ids, routing logits, the drop mask, X, W_ug, W_down.
Normals are drawn in float32 and rounded to bf16 by torch's float32->bfloat16
conversion (round-to-nearest-even); routing weights are a float32 softmax of
N(0, 1) logits. bf16 tensors are returned as uint16 bit patterns.

The five named workloads follow the shapes of the pages' kernel benchmarks:
a four-expert toy with rows (1, 4, 3, 2) (OLMo report, Figs 35-37), an edge
case with an empty expert and a one-row expert, a layer shaped like
Qwen3-30B-A3B (hidden 2048, expert intermediate 768, 128 experts, top-8 over
4K tokens; halo notes, isolated-kernel measurement), one GPU's 64-expert
share of an expert-parallel layer with a Zipf-skewed load (OLMo report,
Sec 9.6 on concentrated histograms), and square experts with d = h = 2880 (so
K % 128 = 64 on both projections; halo notes, the K-tail case) with 5% of
dispatch slots set to -1.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_workload", "make_random", "to_bf16_bits"]


def to_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16) through torch's RNE conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _normal_bf16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return to_bf16_bits(x)


def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    return (p / p.sum(axis=1, keepdims=True)).astype(np.float32)


def _distinct_choice(rng: np.random.Generator, T: int, k: int, choices: np.ndarray) -> np.ndarray:
    """k distinct entries of ``choices`` per token, uniformly (first k of a random permutation)."""
    keys = rng.random((T, choices.shape[0]))
    idx = np.argsort(keys, axis=1, kind="stable")[:, :k]
    return choices[idx].astype(np.int32)


@dataclass
class Workload:
    name: str
    T: int
    k: int
    E: int
    d: int
    h: int
    expert_ids: np.ndarray  # int32 [T, k]; values outside [0, E) are dropped slots
    routing_w: np.ndarray  # float32 [T, k]
    x: np.ndarray  # uint16 (bf16 bits) [T, d]
    w_ug: np.ndarray  # uint16 [E, 2h, d]; gate rows [0, h), up rows [h, 2h)
    w_down: np.ndarray  # uint16 [E, h, d]
    description: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def S(self) -> int:
        return self.T * self.k


def _finish(rng, name, T, k, E, d, h, ids, w, x_sigma, w_sigma, description, meta=None):
    x = _normal_bf16(rng, (T, d), x_sigma)
    w_ug = _normal_bf16(rng, (E, 2 * h, d), w_sigma)
    w_down = _normal_bf16(rng, (E, h, d), w_sigma)
    return Workload(name, T, k, E, d, h, np.ascontiguousarray(ids, dtype=np.int32),
                    np.ascontiguousarray(w, dtype=np.float32), x, w_ug, w_down, description, meta or {})


def _toy(seed):
    rng = np.random.default_rng(seed)
    T, k, E, d, h = 10, 1, 4, 64, 128
    ids = rng.permutation(np.array([0, 1, 1, 1, 1, 2, 2, 2, 3, 3], dtype=np.int32)).reshape(T, k)
    w = np.ones((T, k), dtype=np.float32)
    return _finish(rng, "toy", T, k, E, d, h, ids, w, 1.0, 0.02,
                   "4 experts with rows (1,4,3,2), M=10, d=64, h=128, routing weight 1")


def _edge(seed):
    rng = np.random.default_rng(seed)
    T, k, E, d, h = 2048, 2, 8, 512, 384
    allowed = np.array([0, 1, 2, 4, 6, 7], dtype=np.int32)
    ids = _distinct_choice(rng, T, k, allowed)
    t_star = int(rng.integers(T))
    ids[t_star, 0] = 5
    w = _softmax_rows(rng.standard_normal((T, k), dtype=np.float32))
    return _finish(rng, "edge", T, k, E, d, h, ids, w, 1.0, 0.02,
                   "8 experts, top-2 of 2048 tokens, expert 3 empty, expert 5 one row",
                   {"one_row_token": t_star})


def _qwen3_30b(seed):
    rng = np.random.default_rng(seed)
    T, k, E, d, h = 4096, 8, 128, 2048, 768
    ids = _distinct_choice(rng, T, k, np.arange(E, dtype=np.int32))
    w = _softmax_rows(rng.standard_normal((T, k), dtype=np.float32))
    return _finish(rng, "qwen3_30b", T, k, E, d, h, ids, w, 0.02, 0.02,
                   "Qwen3-30B-A3B-shaped layer: 128 experts, top-8 of 4096 tokens, d=2048, h=768")


ZIPF_S = 1.2
ZIPF_RANKS = 60


def _zipf64(seed):
    rng = np.random.default_rng(seed)
    T, k, E, d, h = 8192, 8, 64, 2048, 768
    r = np.arange(1, ZIPF_RANKS + 1, dtype=np.float64)
    p = r ** (-ZIPF_S)
    p /= p.sum()
    rank = rng.choice(ZIPF_RANKS, size=T * k, p=p)
    relabel = rng.permutation(E).astype(np.int32)
    ids = relabel[rank].reshape(T, k)
    w = _softmax_rows(rng.standard_normal((T, k), dtype=np.float32))
    return _finish(rng, "zipf64", T, k, E, d, h, ids, w, 1.0, 0.02,
                   "64-expert share of an EP layer, 8192 tokens x top-8, slots iid Zipf(1.2) over 60 ranks",
                   {"empty_experts": sorted(relabel[ZIPF_RANKS:].tolist())})


def _square(seed):
    rng = np.random.default_rng(seed)
    T, k, E, d, h = 8192, 4, 16, 2880, 2880
    ids = _distinct_choice(rng, T, k, np.arange(E, dtype=np.int32))
    w = _softmax_rows(rng.standard_normal((T, k), dtype=np.float32))
    n_drop = (T * k * 5) // 100
    drop = rng.choice(T * k, size=n_drop, replace=False)
    ids.reshape(-1)[drop] = -1
    return _finish(rng, "square", T, k, E, d, h, ids, w, 1.0, 0.02,
                   "16 square experts d=h=2880 (K%128=64), 8192 tokens x top-4, 5% of slots -1",
                   {"dropped": int(n_drop)})


WORKLOADS = {
    "toy": (1, _toy),
    "edge": (2, _edge),
    "qwen3_30b": (3, _qwen3_30b),
    "zipf64": (4, _zipf64),
    "square": (5, _square),
}


def make_workload(name: str, seed: int | None = None) -> Workload:
    """One of the five named workloads; the default seed is its index 1..5."""
    idx, fn = WORKLOADS[name]
    return fn(idx if seed is None else seed)


def make_random(T: int, k: int, E: int, d: int, h: int, seed: int, drop_frac: float = 0.1,
                distinct: bool = False, x_sigma: float = 1.0, w_sigma: float = 0.05,
                empty_experts=(), name: str = "random") -> Workload:
    """A small random case for fuzzing: ids uniform over [0, E) (distinct per token if asked),
    a ``drop_frac`` share of slots replaced by invalid ids (-1 and other out-of-range values),
    optional experts forced empty (their slots re-drawn among the others)."""
    rng = np.random.default_rng(seed)
    allowed = np.array([e for e in range(E) if e not in set(empty_experts)], dtype=np.int32)
    if T * k == 0:
        ids = np.zeros((T, k), dtype=np.int32)
    elif allowed.size == 0:
        ids = np.full((T, k), -1, dtype=np.int32)
    elif distinct and k <= allowed.size:
        ids = _distinct_choice(rng, T, k, allowed)
    else:
        ids = allowed[rng.integers(0, allowed.size, size=(T, k))].astype(np.int32)
    w = _softmax_rows(rng.standard_normal((T, k), dtype=np.float32)) if T * k else np.zeros((T, k), np.float32)
    if drop_frac > 0 and T * k > 0:
        mask = rng.random(T * k) < drop_frac
        bad = rng.choice(np.array([-1, -1, -1, E, E + 3, -5, 2**30], dtype=np.int64), size=T * k)
        flat = ids.reshape(-1)
        flat[mask] = bad[mask].astype(np.int32)
    return _finish(rng, name, T, k, E, d, h, ids, w, x_sigma, w_sigma, f"random T={T} k={k} E={E} d={d} h={h}")
