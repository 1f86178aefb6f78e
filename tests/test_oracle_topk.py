"""Pins of the oracle's per-row top-k (no GPU)."""
import numpy as np
import pytest

from oracle import topk_row


def _full_sort(vals, k):
    """Brute force: sort every position by (value descending, position ascending)."""
    ranked = sorted(range(len(vals)), key=lambda p: (-float(vals[p]), p))
    return sorted(ranked[:k])


@pytest.mark.parametrize("seed", range(30))
def test_equals_full_sort_on_tiny_inputs(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 40))
    k = int(rng.integers(1, n))
    vals = rng.integers(-4, 5, size=n).astype(np.float64)   # many ties on purpose
    got = topk_row(vals, n, k)
    assert list(got) == _full_sort(vals, k)


@pytest.mark.parametrize("visible,k", [(0, 4), (1, 4), (3, 4), (4, 4), (2048, 2048), (5, 2048)])
def test_short_rows_select_every_visible_position_in_order(visible, k):
    vals = np.random.default_rng(visible).standard_normal(visible + 10)
    got = topk_row(vals, visible, k)
    assert list(got[:visible]) == list(range(visible))
    assert (got[visible:] == -1).all() and len(got) == k


def test_order_statistic_property():
    rng = np.random.default_rng(9)
    vals = rng.standard_normal(5000)
    k = 700
    sel = topk_row(vals, 5000, k)
    assert len(set(sel.tolist())) == k and (sel >= 0).all()
    mask = np.zeros(5000, bool)
    mask[sel] = True
    assert vals[mask].min() >= vals[~mask].max()


def test_only_visible_positions_compete():
    vals = np.arange(100, dtype=np.float64)    # the largest values sit past the visible length
    got = topk_row(vals, 60, 10)
    assert list(got) == list(range(50, 60))


def test_invariant_to_positive_affine_maps():
    rng = np.random.default_rng(10)
    vals = rng.standard_normal(3000)
    a = topk_row(vals, 3000, 512)
    b = topk_row(3.5 * vals - 7.0, 3000, 512)
    assert np.array_equal(a, b)


def test_ties_go_to_lower_positions():
    vals = np.zeros(10)
    vals[7] = 1.0
    assert list(topk_row(vals, 10, 3)) == [0, 1, 7]
