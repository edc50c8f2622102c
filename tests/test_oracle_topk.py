"""Pins for the oracle's top-k: the pages' toy example, brute force on tiny
inputs with heavy ties and signed zeros, and the n <= k degenerate case."""

import json
import os

import numpy as np

from oracle import dsa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "toy_topk.json")


def brute(v, k):
    order = sorted(range(len(v)), key=lambda i: (-float(v[i]), i))
    return sorted(order[: min(k, len(v))])


def test_toy_example_from_the_pages():
    g = json.load(open(GOLDEN))
    idx, count = dsa.topk(np.array(g["scores"]), g["k"])
    assert count == g["k"]
    assert [int(i) + 1 for i in idx] == g["selected_one_based"]


def test_brute_force_with_ties_and_signed_zero():
    rng = np.random.default_rng(3)
    for trial in range(3000):
        n = int(rng.integers(1, 13))
        k = int(rng.integers(1, 14))
        pool = np.array([0.0, -0.0, 1.0, -1.0, 0.5, 2.0, -3.0, 1e-30, -1e-30])
        v = rng.choice(pool, n) if trial % 2 else rng.standard_normal(n).round(1)
        idx, count = dsa.topk(v, k)
        want = brute(v, k)
        assert count == len(want)
        assert list(idx[:count]) == want
        assert (idx[count:] == -1).all() and len(idx) == k


def test_history_not_longer_than_k_selects_everything():
    for n in (0, 1, 5, 2048):
        v = np.random.default_rng(n).standard_normal(n)
        idx, count = dsa.topk(v, 2048)
        assert count == n
        assert list(idx[:n]) == list(range(n))


def test_all_equal_scores_take_lowest_positions():
    idx, count = dsa.topk(np.full(5000, 0.25, np.float32), 2048)
    assert count == 2048 and list(idx) == list(range(2048))


def test_selected_scores_dominate_the_rest():
    v = np.random.default_rng(7).standard_normal(20000).astype(np.float32)
    idx, count = dsa.topk(v, 2048)
    chosen = np.zeros(v.size, bool)
    chosen[idx[:count]] = True
    assert v[chosen].min() >= v[~chosen].max()
    assert (np.diff(idx) > 0).all()
