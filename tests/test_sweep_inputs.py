"""Inputs of the single-projection sweeps (OLMo report Sec 9.6, Figs 38-40), checked on the CPU."""

import numpy as np
import torch

import oracle
from workloads import (SWEEP, balanced_counts, dirichlet_histograms, expert_orders, imbalance_index,
                       projection_inputs)


def test_imbalance_index_is_eq18():
    """The generator's binning statistic agrees with the oracle's Eq 18 (itself pinned to the
    page's end points) on the sweep's histograms and on edge cases."""
    cases = [h["counts"] for h in dirichlet_histograms()]
    cases += [np.ones(16), np.array([5, 0, 0, 0]), np.array([3]), np.array([0, 0]), np.array([1, 2, 3, 0, 7])]
    for c in cases:
        assert abs(imbalance_index(c) - oracle.entropy_deficit(c)) < 1e-12, c


def test_histograms_fixed_work_and_binned():
    E, M, align, lo = SWEEP["E"], SWEEP["M"], SWEEP["align"], SWEEP["min_rows"]
    hists = dirichlet_histograms()
    assert len(hists) == SWEEP["n_bins"] * SWEEP["per_bin"]
    peak = np.full(E, lo)
    peak[0] = M - (E - 1) * lo
    width = oracle.entropy_deficit(peak) / SWEEP["n_bins"]
    keys = set()
    for h in hists:
        c = h["counts"]
        assert c.shape == (E,) and c.dtype == np.int64
        assert int(c.sum()) == M, "every histogram carries the same rows (and FLOPs)"
        assert (c % align == 0).all() and (c >= lo).all()
        b = h["bin"]
        assert b * width - 1e-12 <= h["imbalance"] <= (b + 1) * width + 1e-12
        keys.add(tuple(sorted(c.tolist())))
    assert len(keys) == len(hists), "histograms are distinct"
    per_bin = np.bincount([h["bin"] for h in hists], minlength=SWEEP["n_bins"])
    assert (per_bin == SWEEP["per_bin"]).all()


def test_histograms_deterministic():
    a, b = dirichlet_histograms(), dirichlet_histograms()
    assert all((x["counts"] == y["counts"]).all() for x, y in zip(a, b))
    c = dirichlet_histograms(seed=7)
    assert any((x["counts"] != y["counts"]).any() for x, y in zip(a, c))


def test_balanced_and_orders():
    assert balanced_counts(16, 65536).tolist() == [4096] * 16
    assert balanced_counts(4, 10).tolist() == [3, 3, 2, 2]
    assert oracle.entropy_deficit(balanced_counts(16, 65536)) == 0.0
    orders = expert_orders(16, 4)
    assert len(orders) == 4 and all(sorted(o.tolist()) == list(range(16)) for o in orders)
    assert len({tuple(o.tolist()) for o in orders}) == 4


def test_projection_inputs_cpu():
    a, w = projection_inputs(64, 48, 40, 3, seed=5)
    assert a.shape == (64, 48) and w.shape == (3, 48, 40)
    assert a.dtype == torch.bfloat16 and w.dtype == torch.bfloat16
    a2, w2 = projection_inputs(64, 48, 40, 3, seed=5)
    assert torch.equal(a.view(torch.int16), a2.view(torch.int16)) and torch.equal(w.view(torch.int16), w2.view(torch.int16))
    assert 0.8 < float(a.float().std()) < 1.2 and 0.015 < float(w.float().std()) < 0.025


def test_exact_count_workload():
    from workloads import make_counts

    counts = [3, 0, 5, 1]
    wl = make_counts(T=5, k=2, E=4, d=8, h=8, counts=counts, seed=7)
    ids = wl.expert_ids.reshape(-1)
    assert ids.shape == (10,)
    np.testing.assert_array_equal(np.bincount(ids[ids >= 0], minlength=4), counts)
    assert int((ids < 0).sum()) == 10 - sum(counts)
    assert wl.routing_w.shape == (5, 2) and np.allclose(wl.routing_w.sum(axis=1), 1.0, atol=1e-6)
    try:
        make_counts(T=2, k=2, E=2, d=8, h=8, counts=[3, 2], seed=1)
    except ValueError:
        pass
    else:
        raise AssertionError("more rows than slots must be refused")
