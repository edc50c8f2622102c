"""GPU parity of dsa_indexer_backward (gradients of the indexer score with
respect to w, the dequantised q and the dequantised k) against the oracle's
indexer_backward_query on the same seeded inputs.

The upstream gradient dL/dI is a seeded synthetic array and the sets are seeded
random selections, so the oracle reads nothing the HIP path produced; the FP8
codes on both sides come from their own quantisers (bit-identical, see the
quantiser tests).

Tolerances.  The GPU takes the FP8 products exactly, sums them in fp32, and
runs the two contractions on bf16 MFMA with the fp32 operand split into
hi + lo bf16 (within 2^-17 relative), accumulating in fp32:
  dw : |dw_gpu - dw_ref| <= 1e-4 * sum_s |g_s| sum_d |qh_jd kh_sd|
  dq : |dq_gpu - dq_ref| <= 1e-4 * |w_j| sum_s [dot > 0] |g_s| |kh_s| + A
  dk : |dk_gpu - dk_ref| <= 1e-4 * sum_(t,j) [dot > 0] |g| |w_j| |qh_j| + A
where A adds the full size of the terms whose gate [dot > 0] fp32 rounding can
flip: pairs with |dot| <= 2^-16 sum_d |qh_d kh_d| (the sum of 128 exact
products in fp32 is within 2^-17 of that bound).  The gate is an integer
decision taken from floating point, so such pairs may go either way.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_long_context_dsa_amd as dsa
from gpu_util import GpuInputs, OracleView, banner
from workloads import make_custom

pytestmark = pytest.mark.gpu

RTOL = 1e-4
AMBIGUOUS = 2.0 ** -16


def random_selection(wl, k, seed):
    rng = np.random.default_rng(seed)
    nv = wl.q_nvis.cpu().numpy()
    idx = np.full((wl.nq, k), -1, np.int32)
    cnt = np.zeros(wl.nq, np.int32)
    for i in range(wl.nq):
        c = min(k, int(nv[i]))
        idx[i, :c] = np.sort(rng.choice(int(nv[i]), c, replace=False)) if c else []
        cnt[i] = c
    return idx, cnt


def run_bwd(g, idx, cnt, k, grad_h):
    wl = g.wl
    dq = torch.full((wl.nq, 64, 128), float("nan"), dtype=torch.float32, device="cuda")
    dw = torch.full((wl.nq, 64), float("nan"), dtype=torch.float32, device="cuda")
    dk = torch.zeros((wl.rows, 128), dtype=torch.float32, device="cuda")
    gi = torch.from_numpy(idx).cuda() if idx is not None else None
    gc = torch.from_numpy(cnt).cuda() if cnt is not None else None
    dsa.dsa_indexer_backward(g.queries, g.layout, g.q8, g.qs, wl.w, g.k8, g.ks, gi, gc, k,
                             torch.from_numpy(grad_h).cuda(), dq, dw, dk)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dw.cpu().numpy(), dk.cpu().numpy()


class Reference:
    """Oracle gradients and their tolerance bounds, accumulated over queries."""

    def __init__(self, wl):
        self.wl = wl
        self.ov = OracleView(wl)
        self.dk = np.zeros((wl.rows, 128))
        self.dk_tol = np.zeros((wl.rows, 128))
        k_all = wl.k_idx.cpu().numpy()
        self.k8, self.ks = oracle.quantize_rows(k_all)

    def query(self, i, positions, g):
        """Oracle dq, dw for query i over `positions` with upstream g, and the
        query's terms added into dk.  Returns (dq, dw, dq_tol, dw_tol)."""
        wl = self.wl
        q8, qs = oracle.quantize_rows(wl.q_idx[i].cpu().numpy())
        qh = oracle.dequantise(q8, qs)
        rows = self.ov.rows(i, positions)
        kh = oracle.dequantise(self.k8[rows], self.ks[rows])
        w = wl.w[i].cpu().numpy().astype(np.float64)
        g = np.asarray(g, np.float64)
        dw, dq, dk = oracle.indexer_backward_query(qh, w, kh, g)
        np.add.at(self.dk, rows, dk)
        # tolerance bounds
        dots = qh @ kh.T
        mag = np.abs(qh) @ np.abs(kh).T
        amb = np.abs(dots) <= AMBIGUOUS * mag
        on = (dots > 0) | amb
        gate = on * (np.abs(w)[:, None] * np.abs(g)[None, :])
        amb_gate = amb * (np.abs(w)[:, None] * np.abs(g)[None, :])
        dq_tol = RTOL * (gate @ np.abs(kh)) + amb_gate @ np.abs(kh)
        dk_tol = RTOL * (gate.T @ np.abs(qh)) + amb_gate.T @ np.abs(qh)
        np.add.at(self.dk_tol, rows, dk_tol)
        dw_tol = RTOL * (mag @ np.abs(g))
        return dq, dw, dq_tol, dw_tol


def check(name, got, want, tol):
    err = np.abs(got.astype(np.float64) - want)
    bad = err > tol + 1e-30
    assert not bad.any(), f"{name}: {bad.sum()} entries off; worst err {err.max():.3e} (tol there {tol.flat[np.argmax(err)]:.3e})"


def compare_sparse(wl, g, idx, cnt, k, grad_h, queries=None):
    dq, dw, dk = run_bwd(g, idx, cnt, k, grad_h)
    ref = Reference(wl)
    nv = wl.q_nvis.cpu().numpy()
    for i in range(wl.nq):
        c = int(cnt[i])
        keep = [j for j in range(c) if 0 <= idx[i, j] < nv[i]]
        rq, rw, tq, tw = ref.query(i, idx[i, keep], grad_h[i, keep])
        if queries is None or i in queries:
            check(f"q{i} dq", dq[i], rq, tq)
            check(f"q{i} dw", dw[i], rw, tw)
    check("dk", dk, ref.dk, ref.dk_tol)
    return dq, dw, dk


@pytest.mark.parametrize("paged", [False, True])
def test_sparse_backward_ragged_sets(paged):
    banner(f"indexer backward sparse ragged paged={paged}")
    wl = make_custom(seq_lens=[1, 33, 100, 2047, 2049, 7000], device="cuda", seed=71, paged=paged)
    g = GpuInputs(wl)
    k = 2048
    idx, cnt = random_selection(wl, k, 1)
    grad_h = (np.random.default_rng(2).standard_normal((wl.nq, k)) * 1e-2).astype(np.float32)
    dq, dw, _ = compare_sparse(wl, g, idx, cnt, k, grad_h)
    assert np.isfinite(dq).all() and np.isfinite(dw).all()


def test_sparse_backward_skips_entries_outside_history():
    banner("indexer backward invalid entries")
    wl = make_custom(seq_lens=[500, 3000], device="cuda", seed=72)
    g = GpuInputs(wl)
    k = 256
    idx, cnt = random_selection(wl, k, 3)
    idx[0, 5] = -1
    idx[0, 9] = 500
    idx[1, 0] = 12345
    grad_h = (np.random.default_rng(4).standard_normal((wl.nq, k)) * 1e-2).astype(np.float32)
    compare_sparse(wl, g, idx, cnt, k, grad_h)


def test_sparse_backward_shared_keys_prefill():
    """300 causal queries of one sequence: their sets share key rows, so dk
    sums the terms of many queries."""
    banner("indexer backward prefill shared keys")
    wl = make_custom(seq_lens=[3000], device="cuda", seed=73, prefill=True, queries_per_seq=300)
    g = GpuInputs(wl)
    k = 512
    idx, cnt = random_selection(wl, k, 5)
    grad_h = (np.random.default_rng(6).standard_normal((wl.nq, k)) * 1e-2).astype(np.float32)
    compare_sparse(wl, g, idx, cnt, k, grad_h, queries=[0, 1, 150, 299])


@pytest.mark.parametrize("paged", [False, True])
def test_dense_backward(paged):
    """Every visible position (dense warm-up), grad by position; the long
    history splits one query over many workgroups."""
    banner(f"indexer backward dense paged={paged}")
    wl = make_custom(seq_lens=[0, 1, 77, 9000], device="cuda", seed=74, paged=paged)
    g = GpuInputs(wl)
    ld = (wl.max_nvis + 63) // 64 * 64
    grad_h = (np.random.default_rng(7).standard_normal((wl.nq, ld)) * 1e-3).astype(np.float32)
    dq, dw, dk = run_bwd(g, None, None, 0, grad_h)
    ref = Reference(wl)
    nv = wl.q_nvis.cpu().numpy()
    assert (dq[0] == 0).all() and (dw[0] == 0).all()
    for i in range(1, wl.nq):
        n = int(nv[i])
        rq, rw, tq, tw = ref.query(i, np.arange(n), grad_h[i, :n])
        check(f"q{i} dq", dq[i], rq, tq)
        check(f"q{i} dw", dw[i], rw, tw)
    check("dk", dk, ref.dk, ref.dk_tol)


def test_backward_dk_accumulates_and_dq_is_deterministic():
    """dk is added to (two calls give twice one call, within rounding); with
    one workgroup per query dq and dw are bit-identical between runs."""
    banner("indexer backward accumulate / determinism")
    wl = make_custom(seq_lens=[1500] * 4, device="cuda", seed=75, prefill=True, queries_per_seq=300)
    g = GpuInputs(wl)
    k = 64
    idx, cnt = random_selection(wl, k, 8)
    grad = torch.from_numpy((np.random.default_rng(9).standard_normal((wl.nq, k)) * 1e-2).astype(np.float32)).cuda()
    gi, gc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    outs = []
    dk = torch.zeros((wl.rows, 128), dtype=torch.float32, device="cuda")
    for _ in range(2):
        dq = torch.empty((wl.nq, 64, 128), dtype=torch.float32, device="cuda")
        dw = torch.empty((wl.nq, 64), dtype=torch.float32, device="cuda")
        dsa.dsa_indexer_backward(g.queries, g.layout, g.q8, g.qs, wl.w, g.k8, g.ks, gi, gc, k, grad, dq, dw, dk)
        torch.cuda.synchronize()
        outs.append((dq.cpu().numpy(), dw.cpu().numpy(), dk.cpu().numpy().copy()))
    assert (outs[0][0].view(np.uint32) == outs[1][0].view(np.uint32)).all()
    assert (outs[0][1].view(np.uint32) == outs[1][1].view(np.uint32)).all()
    # Atomic sums of a few hundred fp32 terms in varying order: within 1e-5 of
    # the largest entry (the rounding of such sums), not relative per entry.
    one, two = outs[0][2].astype(np.float64), outs[1][2].astype(np.float64)
    assert np.abs(two - 2 * one).max() <= 1e-5 * np.abs(one).max()


def test_backward_zero_upstream_and_count_null():
    """grad = 0 gives dq = dw = 0 exactly and leaves dk unchanged; count = NULL
    means min(k, n_vis) members."""
    banner("indexer backward zero grad / count NULL")
    wl = make_custom(seq_lens=[300, 2500], device="cuda", seed=76)
    g = GpuInputs(wl)
    k = 512
    idx, cnt = random_selection(wl, k, 10)
    gi = torch.from_numpy(idx).cuda()
    dq = torch.full((wl.nq, 64, 128), float("nan"), dtype=torch.float32, device="cuda")
    dw = torch.full((wl.nq, 64), float("nan"), dtype=torch.float32, device="cuda")
    dk = torch.full((wl.rows, 128), 0.25, dtype=torch.float32, device="cuda")
    zero = torch.zeros((wl.nq, k), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_backward(g.queries, g.layout, g.q8, g.qs, wl.w, g.k8, g.ks, gi, None, k, zero, dq, dw, dk)
    torch.cuda.synchronize()
    assert (dq == 0).all() and (dw == 0).all() and (dk == 0.25).all()
    # count NULL against the explicit count
    grad_h = (np.random.default_rng(11).standard_normal((wl.nq, k)) * 1e-2).astype(np.float32)
    a = run_bwd(g, idx, None, k, grad_h)
    b = run_bwd(g, idx, cnt, k, grad_h)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=1e-6, atol=1e-7 * max(1.0, np.abs(y).max()))
