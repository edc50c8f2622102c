"""Pins for the oracle's lightning-indexer scores: a textbook single-head case
checked with pure-Python loops over torch-decoded FP8 values, exact rational
arithmetic on small inputs, the identity ReLU(x) - ReLU(-x) = x, linearity in
the head weights, and the pages' toy ranking built through the indexer."""

import json
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import dsa, fp8


def torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # no NaN codes
    return c


def test_single_head_unit_weight_is_textbook_relu_dot():
    rng = np.random.default_rng(5)
    q8 = rand_codes(rng, (1, 128))
    k8 = rand_codes(rng, (9, 128))
    qs = np.array([0.75], np.float32)
    ks = rng.uniform(0.01, 2, 9).astype(np.float32)
    got, mag = dsa.indexer_scores_query(q8, qs, np.ones(1, np.float32), k8, ks)
    qd, kd = torch_decode(q8), torch_decode(k8)
    for s in range(9):
        dot = 0.0
        for d in range(128):
            dot += (float(qs[0]) * qd[0, d]) * (float(ks[s]) * kd[s, d])
        want = max(dot, 0.0)
        assert abs(got[s] - want) <= 1e-12 * max(1.0, abs(want))
        assert abs(mag[s] - want) <= 1e-12 * max(1.0, abs(want))


def test_exact_rational_on_small_inputs():
    rng = np.random.default_rng(6)
    h, d, n = 4, 128, 7
    q8, k8 = rand_codes(rng, (h, d)), rand_codes(rng, (n, d))
    qs = np.array([0.5, 1.0, 2.0, 0.25], np.float32)
    ks = np.array([1, 0.5, 2, 4, 0.125, 1, 8], np.float32)
    w = np.array([0.5, -1.25, 2.0, -0.75], np.float32)
    got, _ = dsa.indexer_scores_query(q8, qs, w, k8, ks)
    qd, kd = torch_decode(q8), torch_decode(k8)
    for s in range(n):
        total = Fraction(0)
        for j in range(h):
            dot = sum(Fraction(float(qd[j, e])) * Fraction(float(kd[s, e])) for e in range(d))
            dot *= Fraction(float(qs[j])) * Fraction(float(ks[s]))
            total += Fraction(float(w[j])) * max(dot, Fraction(0))
        assert abs(Fraction(got[s]) - total) <= abs(total) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 60)


def test_relu_difference_identity_and_zero_weights():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    kx = rng.standard_normal((300, 128)).astype(np.float32)
    q8, qs = fp8.quantize_rows(x)
    k8, ks = fp8.quantize_rows(kx)
    w = (rng.standard_normal(64) / 8).astype(np.float32)
    pos, _ = dsa.indexer_scores_query(q8, qs, w, k8, ks)
    neg, _ = dsa.indexer_scores_query(q8, qs, w, k8 ^ np.uint8(0x80), ks)  # k -> -k
    qd = torch_decode(q8) * qs[:, None].astype(np.float64)
    kd = torch_decode(k8) * ks[:, None].astype(np.float64)
    linear = w.astype(np.float64) @ (qd @ kd.T)
    assert np.allclose(pos - neg, linear, rtol=1e-10, atol=1e-9)
    zero, m0 = dsa.indexer_scores_query(q8, qs, np.zeros(64, np.float32), k8, ks)
    assert (zero == 0).all() and (m0 == 0).all()


def test_linearity_in_head_weights_and_magnitude_bound():
    rng = np.random.default_rng(9)
    q8, qs = fp8.quantize_rows(rng.standard_normal((64, 128)).astype(np.float32))
    k8, ks = fp8.quantize_rows(rng.standard_normal((200, 128)).astype(np.float32))
    w1 = rng.standard_normal(64).astype(np.float32)
    w2 = rng.standard_normal(64).astype(np.float32)
    a, ma = dsa.indexer_scores_query(q8, qs, w1, k8, ks)
    b, _ = dsa.indexer_scores_query(q8, qs, w2, k8, ks)
    c, _ = dsa.indexer_scores_query(q8, qs, (w1.astype(np.float64) + w2).astype(np.float32), k8, ks)
    w12 = w1.astype(np.float64) + w2.astype(np.float64)
    if (w12.astype(np.float32) == w12).all():
        assert np.allclose(a + b, c, rtol=1e-12, atol=1e-9)
    assert (np.abs(a) <= ma + 1e-12).all()


def test_toy_ranking_through_the_indexer():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "toy_topk.json")))
    scores = np.array(g["scores"], np.float32)
    keys = np.zeros((8, 128), np.float32)
    keys[:, 0] = scores  # one nonzero dim per key: the dequantised key equals the toy score
    q = np.zeros((1, 128), np.float32)
    q[0, 0] = 1.0
    q8, qs = fp8.quantize_rows(q)
    k8, ks = fp8.quantize_rows(keys)
    got, _ = dsa.indexer_scores_query(q8, qs, np.ones(1, np.float32), k8, ks)
    assert np.allclose(got, scores, rtol=1e-6)
    idx, count = dsa.topk(got, g["k"])
    assert [int(i) + 1 for i in idx[:count]] == g["selected_one_based"]
