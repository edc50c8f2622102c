"""The indexer KL loss and the indexer backward at the full prefill size
(16384 causal tokens, k = 2048), in the launch configuration the benchmark
times.

As in the forward's full-size parity, the loss takes the library's own top-k
sets, attention log-sum-exps and indexer scores as its inputs (the same
isolation as the attention checks: the oracle gets the same sets and scores),
and the backward takes the loss's gradient as its upstream gradient.

* Sampled queries are checked element by element against the oracle
  (tolerances as in the small parity tests).
* Every query is checked for what holds at any size: p sums to one over a
  non-empty set, the gradient sums to zero, KL >= 0, everything finite.
* dk is pinned as a whole by homogeneity: the score is degree-1 homogeneous in
  each key (and in each query head vector and each weight), so
  sum_rows dk . kh = sum_t sum_s g_ts I_ts = sum_(t,j) dw_tj w_tj.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_long_context_dsa_amd as dsa
from gpu_util import GpuInputs, OracleView, banner, bf16_bits
from workloads import make_config

pytestmark = pytest.mark.gpu

P_RTOL = 1e-4
KL_RTOL = 1e-4


def check_kl_query(wl, ov, i, positions, scores_row, g_gpu, p_gpu, kl_gpu, where):
    r = ov.rows(i, positions)
    kv = bf16_bits(wl.kv[torch.from_numpy(r).cuda()])
    x = scores_row[positions].astype(np.float64)
    kl_ref, g_ref, p_ref, mag = oracle.indexer_kl_query(bf16_bits(wl.q_mla[i]), kv, x, wl.softmax_scale)
    n = len(positions)
    assert (np.abs(p_gpu[:n] - p_ref) <= P_RTOL * p_ref + 1e-12).all(), f"{where}: target"
    assert (np.abs(g_gpu[:n] - g_ref) <= P_RTOL * (2 * p_ref + g_ref) + 1e-12).all(), f"{where}: grad"
    assert abs(kl_gpu - kl_ref) <= KL_RTOL * (1.0 + mag), f"{where}: kl {kl_gpu} vs {kl_ref}"


@pytest.fixture(scope="module")
def prefill():
    wl = make_config(3, device="cuda")
    banner(f"kl full size: {wl.name}, {wl.nq} queries")
    g = GpuInputs(wl)
    nq, k = wl.nq, wl.k
    out = torch.empty((nq, 128, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((nq, 128), dtype=torch.float32, device="cuda")
    idx = torch.empty((nq, k), dtype=torch.int32, device="cuda")
    dsa.dsa_forward(g.queries, g.layout, g.q8, g.qs, wl.w, g.k8, g.ks, wl.q_mla, wl.kv, k, wl.softmax_scale, out, lse,
                    idx)
    del out
    scores = g.scores()
    torch.cuda.synchronize()
    yield wl, g, idx, lse, scores
    del g, idx, lse, scores
    torch.cuda.empty_cache()


def test_sparse_stage_full_size(prefill):
    wl, g, idx, lse, scores = prefill
    nq, k = wl.nq, wl.k
    grad = torch.empty((nq, k), dtype=torch.float32, device="cuda")
    target = torch.empty((nq, k), dtype=torch.float32, device="cuda")
    kl = torch.empty((nq,), dtype=torch.float32, device="cuda")
    loss = torch.empty((1,), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_kl_sparse(g.queries, g.layout, wl.q_mla, wl.kv, idx, None, k, lse, wl.softmax_scale, scores, grad,
                              kl, target=target, loss=loss)
    torch.cuda.synchronize()
    # every query
    nv = wl.q_nvis.to(torch.int64)
    cnt = torch.clamp(nv, max=k)
    live = torch.arange(k, device="cuda")[None, :] < cnt[:, None]
    psum = (target.double() * live).sum(1)
    has = cnt > 0
    assert torch.isfinite(grad).all() and torch.isfinite(kl).all() and torch.isfinite(target).all()
    assert (psum[has] - 1).abs().max().item() <= 1e-5
    assert (grad.double() * live).sum(1).abs().max().item() <= 1e-5
    assert kl.min().item() >= -1e-5 and (kl[~has] == 0).all()
    assert abs(loss.item() - kl.double().sum().item()) <= 1e-6 * abs(loss.item())
    # sampled queries against the oracle
    ov = OracleView(wl)
    idx_h = idx.cpu().numpy()
    rng = np.random.default_rng(3)
    pick = sorted({1, 2, 2047, 2048, 2049, nq - 1} | set(int(x) for x in rng.choice(nq, 8, replace=False)))
    banner(f"kl sparse oracle on queries {pick}")
    for i in pick:
        c = int(cnt[i])
        s_row = scores[i].cpu().numpy()
        check_kl_query(wl, ov, i, idx_h[i, :c], s_row, grad[i].cpu().numpy(), target[i].cpu().numpy(),
                       float(kl[i]), f"q{i}")

    # backward from this gradient: sampled dq / dw, dk as a whole
    dq = torch.empty((nq, 64, 128), dtype=torch.float32, device="cuda")
    dw = torch.empty((nq, 64), dtype=torch.float32, device="cuda")
    dk = torch.zeros((wl.rows, 128), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_backward(g.queries, g.layout, g.q8, g.qs, wl.w, g.k8, g.ks, idx, None, k, grad, dq, dw, dk)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all() and torch.isfinite(dw).all() and torch.isfinite(dk).all()
    # sum_t sum_s g I (I from the scores the loss used) = sum dw . w = sum_rows dk . kh
    ii = torch.clamp(idx.to(torch.int64), min=0)
    zero = torch.zeros((), dtype=torch.float64, device="cuda")
    gI = torch.where(live, grad.double() * torch.gather(scores, 1, ii).double(), zero)  # padding reads NaN scores
    gi = gI.sum().item()
    dww = (dw.double() * wl.w.double()).sum().item()
    kh = oracle.dequantise(g.k8.cpu().numpy(), g.ks.cpu().numpy())
    dkk = float((dk.cpu().numpy().astype(np.float64) * kh).sum())
    mag = gI.abs().sum().item()
    assert abs(dww - gi) <= 1e-3 * mag, (dww, gi, mag)
    assert abs(dkk - gi) <= 1e-3 * mag, (dkk, gi, mag)
    k8h, ksh = oracle.quantize_rows(wl.k_idx.cpu().numpy())
    for i in pick[:6]:
        c = int(cnt[i])
        q8, qs = oracle.quantize_rows(wl.q_idx[i].cpu().numpy())
        rows = ov.rows(i, idx_h[i, :c])
        qh = oracle.dequantise(q8, qs)
        khs = oracle.dequantise(k8h[rows], ksh[rows])
        gq = grad[i, :c].cpu().numpy().astype(np.float64)
        w = wl.w[i].cpu().numpy().astype(np.float64)
        rw, rq, _ = oracle.indexer_backward_query(qh, w, khs, gq)
        dots = qh @ khs.T
        magd = np.abs(qh) @ np.abs(khs).T
        amb = np.abs(dots) <= 2.0 ** -16 * magd
        gate = ((dots > 0) | amb) * (np.abs(w)[:, None] * np.abs(gq)[None, :])
        tq = 1e-4 * (gate @ np.abs(khs)) + (amb * (np.abs(w)[:, None] * np.abs(gq)[None, :])) @ np.abs(khs)
        assert (np.abs(dq[i].cpu().numpy() - rq) <= tq + 1e-30).all(), f"q{i} dq"
        assert (np.abs(dw[i].cpu().numpy() - rw) <= 1e-4 * (magd @ np.abs(gq)) + 1e-30).all(), f"q{i} dw"


def test_dense_warmup_full_size(prefill):
    wl, g, idx, lse, scores = prefill
    nq = wl.nq
    out = torch.empty((nq, 128, 512), dtype=torch.float32, device="cuda")
    lse_d = torch.empty((nq, 128), dtype=torch.float32, device="cuda")
    dsa.dsa_dense_mla(g.queries, g.layout, wl.q_mla, wl.kv, wl.softmax_scale, out, lse_d)
    del out
    ld = scores.shape[1]
    grad = torch.full((nq, ld), float("nan"), dtype=torch.float32, device="cuda")
    kl = torch.empty((nq,), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_kl_dense(g.queries, g.layout, wl.q_mla, wl.kv, lse_d, wl.softmax_scale, scores, grad, kl)
    torch.cuda.synchronize()
    nv = wl.q_nvis.to(torch.int64)
    live = torch.arange(ld, device="cuda")[None, :] < nv[:, None]
    assert torch.isfinite(grad[live]).all() and torch.isfinite(kl).all()
    assert torch.where(live, grad.double(), torch.zeros_like(grad, dtype=torch.float64)).sum(1).abs().max() <= 1e-5
    assert kl.min().item() >= -1e-5
    ov = OracleView(wl)
    pick = [1, 2, 5000, nq - 1]
    banner(f"kl dense oracle on queries {pick}")
    for i in pick:
        n = int(nv[i])
        # (the target is not requested here: KL and gradient only)
        r = ov.rows(i, np.arange(n))
        kv = bf16_bits(wl.kv[torch.from_numpy(r).cuda()])
        x = scores[i, :n].cpu().numpy().astype(np.float64)
        kl_ref, g_ref, p_ref, mag = oracle.indexer_kl_query(bf16_bits(wl.q_mla[i]), kv, x, wl.softmax_scale)
        gg = grad[i, :n].cpu().numpy()
        assert (np.abs(gg - g_ref) <= P_RTOL * (2 * p_ref + g_ref) + 1e-12).all(), f"dense q{i}: grad"
        assert abs(float(kl[i]) - kl_ref) <= KL_RTOL * (1.0 + mag), f"dense q{i}: kl"
