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
dispatch slots set to -1. The 64-expert share draws each slot independently,
so a token may send two slots to one expert and one expert may receive more
than T rows; ``zipf64_top8`` is the same layer with eight distinct experts per
token, the way a top-k router picks them.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_workload", "make_random", "to_bf16_bits", "dirichlet_histograms",
           "balanced_counts", "expert_orders", "imbalance_index", "projection_inputs", "SWEEP"]


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


def _zipf64_top8(seed):
    rng = np.random.default_rng(seed)
    T, k, E, d, h = 8192, 8, 64, 2048, 768
    r = np.arange(1, ZIPF_RANKS + 1, dtype=np.float64)
    logp = -ZIPF_S * np.log(r)
    # k distinct ranks per token, drawn without replacement with probabilities proportional to
    # r^-1.2 (Gumbel-top-k: the k largest of log p_r + Gumbel noise), as a top-k router picks them
    keys = logp[None, :] + rng.gumbel(size=(T, ZIPF_RANKS))
    rank = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    relabel = rng.permutation(E).astype(np.int32)
    ids = relabel[rank]
    w = _softmax_rows(rng.standard_normal((T, k), dtype=np.float32))
    return _finish(rng, "zipf64_top8", T, k, E, d, h, ids, w, 1.0, 0.02,
                   "64-expert share of an EP layer, 8192 tokens x top-8 distinct experts, Zipf(1.2) over 60 ranks",
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
    # the zipf64 layer with a top-8 router's distinct experts per token (no expert above T rows)
    "zipf64_top8": (6, _zipf64_top8),
}


def make_workload(name: str, seed: int | None = None) -> Workload:
    """One of the named workloads; the default seed is its index (1..5 for the five, 6 for zipf64_top8)."""
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


def make_counts(T: int, k: int, E: int, d: int, h: int, counts, seed: int, w_sigma: float = 0.05,
                name: str = "counts") -> Workload:
    """Exact rows per expert: expert e gets counts[e] of the T*k slots (placed in random slots, duplicates
    within a token allowed), every other slot an invalid id (-1)."""
    counts = np.asarray(counts, dtype=np.int64)
    if counts.shape != (E,) or counts.min(initial=0) < 0 or counts.sum() > T * k:
        raise ValueError("counts must be E non-negative numbers summing to at most T*k")
    rng = np.random.default_rng(seed)
    flat = np.full(T * k, -1, dtype=np.int32)
    flat[: counts.sum()] = np.repeat(np.arange(E, dtype=np.int32), counts)
    ids = rng.permutation(flat).reshape(T, k)
    w = _softmax_rows(rng.standard_normal((T, k), dtype=np.float32)) if T * k else np.zeros((T, k), np.float32)
    return _finish(rng, name, T, k, E, d, h, ids, w, 1.0, w_sigma,
                   f"exact counts T={T} k={k} E={E} d={d} h={h} rows {counts.tolist()}")


# --------------------------------------------------------------------------
# Inputs of the single-projection sweeps (OLMo report, Sec 9.6, Figs 38-40)
# --------------------------------------------------------------------------

# Fig 40's fixed-work histogram sweep: 16 local experts, M = 65,536 rows, one
# square projection with d = h = 4096; counts are multiples of 8 rows and every
# expert keeps at least one 128-row tile.
SWEEP = {"E": 16, "M": 65536, "dim": 4096, "align": 8, "min_rows": 128, "n_bins": 10, "per_bin": 10}


def balanced_counts(E: int, M: int) -> np.ndarray:
    """M rows split as evenly as possible over E experts (the first M % E experts get one more)."""
    base, extra = divmod(int(M), int(E))
    return np.array([base + (1 if e < extra else 0) for e in range(E)], dtype=np.int64)


def imbalance_index(counts) -> float:
    """Normalised entropy deficit of a histogram, used here only to bin proposals.

    The same statistic as the OLMo report's Eq 18; the test suite checks this
    copy against the oracle's.
    """
    c = np.asarray(counts, dtype=np.float64)
    n, tot = c.shape[0], c.sum()
    if n <= 1 or tot == 0:
        return 0.0
    q = c[c > 0] / tot
    return float(1.0 + np.sum(q * np.log(q)) / np.log(n))


def _counts_from_proposal(p: np.ndarray, M: int, align: int, min_rows: int) -> np.ndarray:
    """Exact counts from a probability vector: every expert keeps ``min_rows``; the remaining
    M - E*min_rows rows are dealt in ``align``-row units by largest remainder."""
    E = p.shape[0]
    units = (M - E * min_rows) // align
    raw = p * units
    base = np.floor(raw).astype(np.int64)
    short = units - int(base.sum())
    if short > 0:
        order = np.argsort(-(raw - base), kind="stable")
        base[order[:short]] += 1
    return min_rows + align * base


def dirichlet_histograms(E: int = SWEEP["E"], M: int = SWEEP["M"], align: int = SWEEP["align"],
                         min_rows: int = SWEEP["min_rows"], n_bins: int = SWEEP["n_bins"],
                         per_bin: int = SWEEP["per_bin"], seed: int = 40, log10_alpha=(-3.0, 2.0),
                         max_draws: int = 500_000) -> list[dict]:
    """Fixed-work load histograms spanning the imbalance range (Fig 40's construction).

    Symmetric-Dirichlet proposals, concentration alpha drawn log-uniformly
    from ``10**log10_alpha``, are turned into exact counts (multiples of
    ``align``, at least ``min_rows`` each, summing to M). The imbalance range
    [0, I_max], where I_max belongs to the most concentrated feasible
    histogram (one expert holding every spare row), is cut into ``n_bins``
    equal-width bins, and the first ``per_bin`` distinct histograms (distinct
    as sorted count lists) landing in each bin are kept. Returns dicts with
    ``counts`` (int64 [E], in proposal order), ``imbalance``, ``alpha``, ``bin``.
    """
    if M % align or min_rows % align or E * min_rows > M:
        raise ValueError("M and min_rows must be multiples of align, and E*min_rows <= M")
    rng = np.random.default_rng(seed)
    peak = np.full(E, min_rows, dtype=np.int64)
    peak[0] = M - (E - 1) * min_rows
    i_max = imbalance_index(peak)
    width = i_max / n_bins
    bins: list[list[dict]] = [[] for _ in range(n_bins)]
    seen = set()
    for _ in range(max_draws):
        alpha = 10.0 ** rng.uniform(*log10_alpha)
        p = rng.dirichlet(np.full(E, alpha))
        counts = _counts_from_proposal(p, M, align, min_rows)
        key = tuple(sorted(counts.tolist()))
        if key in seen:
            continue
        ih = imbalance_index(counts)
        b = min(int(ih / width), n_bins - 1) if width > 0 else 0
        if len(bins[b]) >= per_bin:
            continue
        seen.add(key)
        bins[b].append({"counts": counts, "imbalance": ih, "alpha": alpha, "bin": b})
        if all(len(x) >= per_bin for x in bins):
            break
    else:
        raise RuntimeError(f"only {[len(x) for x in bins]} histograms per bin after {max_draws} proposals")
    return [h for x in bins for h in x]


def expert_orders(E: int, n: int = 4, seed: int = 41) -> list[np.ndarray]:
    """``n`` fixed permutations of the expert index: which expert id gets which count."""
    rng = np.random.default_rng(seed)
    return [rng.permutation(E) for _ in range(n)]


def projection_inputs(M: int, K: int, N: int, E: int, seed: int, device="cpu", x_sigma: float = 1.0,
                      w_sigma: float = 0.02):
    """Activations A [M, K] and per-expert weights W [E, K, N] as bf16 torch tensors on ``device``.

    Drawn with torch's generator for that device seeded with ``seed`` (normals
    in float32, rounded to bf16), so multi-gigabyte operands never pass
    through host memory. The same seed on another device type gives other values.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    a = torch.empty((M, K), dtype=torch.bfloat16, device=device)
    w = torch.empty((E, K, N), dtype=torch.bfloat16, device=device)
    # fill in row blocks so the float32 staging stays small
    step = max(1, (1 << 26) // max(K, 1))
    for lo in range(0, M, step):
        hi = min(M, lo + step)
        a[lo:hi] = (torch.randn((hi - lo, K), generator=g, device=device) * x_sigma).to(torch.bfloat16)
    step = max(1, (1 << 26) // max(N, 1))
    for e in range(E):
        for lo in range(0, K, step):
            hi = min(K, lo + step)
            w[e, lo:hi] = (torch.randn((hi - lo, N), generator=g, device=device) * w_sigma).to(torch.bfloat16)
    return a, w
