"""Pins for the oracle's indexer alignment loss: the KL divergence against
scipy's rel_entr and softmax, a two-point closed form, Gibbs' inequality and its
equality case, finite differences of the loss through the indexer score, the
linear (all-ReLU-active) case in closed form, and the attention target against
textbook softmaxes on inputs whose logits are known exactly."""

import math

import numpy as np
import pytest
import scipy.special as sp
import torch

from oracle import dsa, fp8, kl

SCALE = 1.0 / math.sqrt(192.0)


def bf16_bits(x):
    t = torch.from_numpy(np.asarray(x, np.float32).copy()).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------- #
# KL(p || Softmax(x)) and its gradient
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("seed", range(5))
def test_kl_matches_scipy(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 300))
    p = rng.dirichlet(np.full(n, 0.3))
    p[rng.random(n) < 0.2] = 0.0  # exact zeros: 0 log 0 = 0
    p /= p.sum()
    x = rng.standard_normal(n) * 4.0
    got, grad, mag = kl.kl_to_softmax(p, x)
    want = sp.rel_entr(p, sp.softmax(x)).sum()
    assert got == pytest.approx(want, rel=1e-12, abs=1e-15)
    assert np.allclose(grad, sp.softmax(x) - p, rtol=0, atol=1e-15)
    assert mag >= abs(got)


def test_kl_two_point_closed_form():
    for a, x, y in [(0.3, 0.2, -1.1), (0.9, 5.0, 5.0), (0.5, -2.0, 3.0)]:
        s = 1.0 / (1.0 + math.exp(y - x))  # Softmax((x, y))[0]
        want = a * math.log(a / s) + (1 - a) * math.log((1 - a) / (1 - s))
        got, grad, _ = kl.kl_to_softmax(np.array([a, 1 - a]), np.array([x, y]))
        assert got == pytest.approx(want, rel=1e-13, abs=1e-15)
        assert grad[0] == pytest.approx(s - a, abs=1e-15)


def test_kl_is_zero_when_softmax_equals_target():
    rng = np.random.default_rng(7)
    p = rng.dirichlet(np.ones(50))
    got, grad, _ = kl.kl_to_softmax(p, np.log(p) + 3.7)  # shift: same softmax
    assert abs(got) < 1e-14
    assert np.abs(grad).max() < 1e-15


def test_gibbs_inequality_and_shift_invariance():
    rng = np.random.default_rng(8)
    for _ in range(50):
        n = int(rng.integers(1, 40))
        p = rng.dirichlet(np.full(n, 0.5))
        x = rng.standard_normal(n) * 3
        a, ga, _ = kl.kl_to_softmax(p, x)
        b, gb, _ = kl.kl_to_softmax(p, x - 11.0)
        assert a >= -1e-15
        assert a == pytest.approx(b, rel=1e-12, abs=1e-15)
        assert abs(ga.sum()) < 1e-14  # Softmax and p both sum to one


def test_kl_gradient_by_finite_differences():
    rng = np.random.default_rng(9)
    n = 9
    p = rng.dirichlet(np.ones(n))
    p[3] = 0.0
    p /= p.sum()
    x = rng.standard_normal(n)
    _, grad, _ = kl.kl_to_softmax(p, x)
    eps = 1e-6
    for i in range(n):
        e = np.zeros(n)
        e[i] = eps
        fd = (kl.kl_to_softmax(p, x + e)[0] - kl.kl_to_softmax(p, x - e)[0]) / (2 * eps)
        assert fd == pytest.approx(grad[i], abs=1e-8)


def test_empty_set():
    got, grad, mag = kl.kl_to_softmax(np.zeros(0), np.zeros(0))
    assert got == 0.0 and grad.shape == (0,) and mag == 0.0
    assert kl.attention_target(bf16_bits(np.ones((4, 576))), np.zeros((0, 576), np.uint16), SCALE).shape == (0,)


# --------------------------------------------------------------------------- #
# the attention target
# --------------------------------------------------------------------------- #
def one_hot_case(coeffs, values):
    """Heads q_h = c_h * e_0 and rows with v_s in dim 0 (zeros elsewhere), all
    exact in bf16, so that z[h, s] = SCALE * c_h * v_s exactly."""
    q = np.zeros((len(coeffs), 576), np.float32)
    q[:, 0] = coeffs
    kv = np.zeros((len(values), 576), np.float32)
    kv[:, 0] = values
    return bf16_bits(q), bf16_bits(kv)


def test_target_of_one_head_is_its_softmax():
    v = np.array([0.5, -1.0, 2.0, 0.25, 3.0, -2.5])
    q, kv = one_hot_case([3.0], v)
    p = kl.attention_target(q, kv, SCALE)
    assert np.allclose(p, sp.softmax(SCALE * 3.0 * v), rtol=1e-14, atol=0)


def test_target_two_rows_is_mean_of_sigmoids():
    c = np.array([1.0, -2.0, 4.0, 0.5, 8.0])
    u, v = 1.5, -0.75
    q, kv = one_hot_case(c, [u, v])
    p = kl.attention_target(q, kv, SCALE)
    # Each head's weight on the second row is sigmoid(z_h1 - z_h0); the heads'
    # sum is divided by its L1 norm, the head count.
    want1 = np.mean(sp.expit(SCALE * c * (v - u)))
    assert p[1] == pytest.approx(want1, rel=1e-14)
    assert p[0] == pytest.approx(1 - want1, rel=1e-14)


def test_target_invariances():
    rng = np.random.default_rng(10)
    q = bf16_bits(rng.standard_normal((16, 576)))
    kv = bf16_bits(rng.standard_normal((40, 576)))
    p = kl.attention_target(q, kv, SCALE)
    assert p.min() > 0 and p.sum() == pytest.approx(1.0, abs=1e-14)
    hp = rng.permutation(16)
    assert np.allclose(kl.attention_target(q[hp], kv, SCALE), p, rtol=1e-13, atol=0)
    rp = rng.permutation(40)
    assert np.allclose(kl.attention_target(q, kv[rp], SCALE), p[rp], rtol=1e-13, atol=0)
    # identical rows share the mass evenly; one row takes all of it
    same = np.repeat(kv[:1], 7, axis=0)
    assert np.allclose(kl.attention_target(q, same, SCALE), 1 / 7, rtol=1e-14, atol=0)
    assert kl.attention_target(q, kv[:1], SCALE)[0] == 1.0


def test_target_is_mean_of_head_weights_from_attention_lse():
    # Each head's weights exp(z - lse) come from the attention's own log-sum-exp
    # (a separate, pinned oracle function); their mean over the heads is p.
    c = np.array([1.0, -3.0, 0.5, 6.0])
    v = np.array([0.5, -1.0, 2.0, 1.25, -0.375])
    q, kv = one_hot_case(c, v)
    _, lse = dsa.sparse_mla(q, kv, SCALE)
    z = SCALE * c[:, None] * v[None, :]
    want = np.exp(z - lse[:, None]).mean(axis=0)
    assert np.allclose(kl.attention_target(q, kv, SCALE), want, rtol=1e-13, atol=0)


# --------------------------------------------------------------------------- #
# backward through the indexer score
# --------------------------------------------------------------------------- #
def small_indexer(seed, h=8, d=16, n=12):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((h, d)), rng.standard_normal(h), rng.standard_normal((n, d))


def test_indexer_logits_equal_the_fp8_indexer():
    rng = np.random.default_rng(11)
    q8, qs = fp8.quantize_rows(rng.standard_normal((64, 128)).astype(np.float32))
    k8, ks = fp8.quantize_rows(rng.standard_normal((300, 128)).astype(np.float32))
    w = (rng.standard_normal(64) / 8).astype(np.float32)
    want, _ = dsa.indexer_scores_query(q8, qs, w, k8, ks)
    got = kl.indexer_logits(kl.dequantise(q8, qs), w, kl.dequantise(k8, ks))
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_loss_gradients_by_finite_differences(seed):
    qh, w, kh = small_indexer(20 + seed)
    assert np.abs(qh @ kh.T).min() > 1e-3  # no ReLU kink within the step
    p = np.random.default_rng(30 + seed).dirichlet(np.ones(kh.shape[0]))

    def loss(qh_, w_, kh_):
        return kl.kl_to_softmax(p, kl.indexer_logits(qh_, w_, kh_))[0]

    _, g, _ = kl.kl_to_softmax(p, kl.indexer_logits(qh, w, kh))
    dw, dq, dk = kl.indexer_backward_query(qh, w, kh, g)
    eps = 1e-6
    for j in range(w.shape[0]):
        e = np.zeros_like(w)
        e[j] = eps
        fd = (loss(qh, w + e, kh) - loss(qh, w - e, kh)) / (2 * eps)
        assert fd == pytest.approx(dw[j], rel=1e-5, abs=1e-9)
    rng = np.random.default_rng(40 + seed)
    for _ in range(4):
        vq = rng.standard_normal(qh.shape)
        fd = (loss(qh + eps * vq, w, kh) - loss(qh - eps * vq, w, kh)) / (2 * eps)
        assert fd == pytest.approx((dq * vq).sum(), rel=1e-5, abs=1e-9)
        vk = rng.standard_normal(kh.shape)
        fd = (loss(qh, w, kh + eps * vk) - loss(qh, w, kh - eps * vk)) / (2 * eps)
        assert fd == pytest.approx((dk * vk).sum(), rel=1e-5, abs=1e-9)


def test_backward_linear_case_closed_form():
    # All dots positive: I = (w^T qh) kh^T is linear, so the gradients are
    # outer products.
    rng = np.random.default_rng(12)
    qh = np.abs(rng.standard_normal((6, 10)))
    kh = np.abs(rng.standard_normal((9, 10)))
    w = rng.standard_normal(6)
    g = rng.standard_normal(9)
    dw, dq, dk = kl.indexer_backward_query(qh, w, kh, g)
    u = w @ qh  # [d]
    assert np.allclose(dk, np.outer(g, u), rtol=1e-13, atol=1e-14)
    assert np.allclose(dq, np.outer(w, g @ kh), rtol=1e-13, atol=1e-14)
    assert np.allclose(dw, qh @ (kh.T @ g), rtol=1e-13, atol=1e-14)


def test_backward_inactive_relu_gives_zero():
    rng = np.random.default_rng(13)
    qh = np.abs(rng.standard_normal((5, 8)))
    kh = -np.abs(rng.standard_normal((7, 8)))  # every dot negative
    dw, dq, dk = kl.indexer_backward_query(qh, rng.standard_normal(5), kh, rng.standard_normal(7))
    assert not dw.any() and not dq.any() and not dk.any()


def test_kl_with_minus_inf_logits():
    """A logit of -inf has softmax weight 0.  Where p is 0 too the entry drops
    out: KL and the other gradients equal scipy's over the finite entries, and
    its own gradient is 0.  Where p > 0 the KL is +inf and the gradient -p."""
    rng = np.random.default_rng(21)
    n = 40
    x = rng.standard_normal(n) * 2.0
    dead = np.zeros(n, bool)
    dead[[0, 7, 19, 39]] = True
    x[dead] = -np.inf
    p = rng.dirichlet(np.ones(n))
    p[dead] = 0.0
    p /= p.sum()
    got, grad, _ = kl.kl_to_softmax(p, x)
    live = ~dead
    assert got == pytest.approx(sp.rel_entr(p[live], sp.softmax(x[live])).sum(), rel=1e-12)
    assert np.allclose(grad[live], sp.softmax(x[live]) - p[live], rtol=0, atol=1e-15)
    assert (grad[dead] == 0.0).all()
    p2 = rng.dirichlet(np.ones(n))  # mass on the -inf entries
    got2, grad2, _ = kl.kl_to_softmax(p2, x)
    assert got2 == np.inf
    assert np.isfinite(grad2).all() and np.allclose(grad2[dead], -p2[dead], rtol=0, atol=0)
