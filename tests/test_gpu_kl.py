"""GPU parity of the indexer KL loss (dsa_indexer_kl_sparse / _dense) against
the oracle's target, KL and gradient on the same seeded inputs.

The indexer scores fed to both sides are seeded synthetic logits (the loss's
own input, independent of the HIP indexer), and the sparse sets are seeded
random selections.  The HIP call also takes the attention's log-sum-exp, which
comes from the library's own attention over the same set (dsa_sparse_mla_* or
dsa_dense_mla); the oracle recomputes the attention itself.

Tolerances (the target and the logits of the softmax are fp32 on the GPU; the
attention logits come from exact bf16 products summed in fp32, so p is within
about 1e-5 relative):
  target : |p_gpu - p_ref| <= 1e-4 * p_ref + 1e-12
  grad   : |g_gpu - g_ref| <= 1e-4 * (p_ref + softmax_ref) + 1e-12
  kl     : |kl_gpu - kl_ref| <= 1e-4 * (1 + sum_s p |ln p - ln softmax|)
(a relative error d in p moves each term p (ln p - ln q) by at most
d * p * (1 + |ln p - ln q|)).
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_long_context_dsa_amd as dsa
from gpu_util import OracleView, banner, bf16_bits
from workloads import make_custom

pytestmark = pytest.mark.gpu

P_RTOL = 1e-4
KL_RTOL = 1e-4


def layout_of(wl):
    q = dsa.Queries(wl.q_seq, wl.q_nvis, wl.max_nvis)
    if wl.block_size:
        lay = dsa.KvLayout(wl.num_seqs, wl.rows, block_table=wl.block_table, block_size=wl.block_size)
    else:
        lay = dsa.KvLayout(wl.num_seqs, wl.rows, seq_row0=wl.row0)
    return q, lay


def synthetic_scores(wl, seed, std=3.0):
    """Seeded N(0, std^2) indexer logits [nq, ld] (host copy and device copy)."""
    ld = max(64, (wl.max_nvis + 63) // 64 * 64)
    s = (np.random.default_rng(seed).standard_normal((wl.nq, ld)) * std).astype(np.float32)
    return s, torch.from_numpy(s).cuda()


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


def run_sparse(wl, idx, cnt, k, scores_d, lse=None):
    q, lay = layout_of(wl)
    g_idx, g_cnt = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    if lse is None:
        out = torch.empty((wl.nq, 128, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((wl.nq, 128), dtype=torch.float32, device="cuda")
        dsa.dsa_sparse_mla_decode(q, lay, wl.q_mla, wl.kv, g_idx, g_cnt, k, wl.softmax_scale, out, lse)
    grad = torch.full((wl.nq, k), float("nan"), dtype=torch.float32, device="cuda")
    target = torch.full((wl.nq, k), float("nan"), dtype=torch.float32, device="cuda")
    kl = torch.full((wl.nq,), float("nan"), dtype=torch.float32, device="cuda")
    loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_kl_sparse(q, lay, wl.q_mla, wl.kv, g_idx, g_cnt, k, lse, wl.softmax_scale, scores_d, grad, kl,
                              target=target, loss=loss)
    torch.cuda.synchronize()
    return grad.cpu().numpy(), target.cpu().numpy(), kl.cpu().numpy(), float(loss.item()), lse


def run_dense(wl, scores_d, lse=None):
    q, lay = layout_of(wl)
    if lse is None:
        out = torch.empty((wl.nq, 128, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((wl.nq, 128), dtype=torch.float32, device="cuda")
        dsa.dsa_dense_mla(q, lay, wl.q_mla, wl.kv, wl.softmax_scale, out, lse)
    ld = scores_d.shape[1]
    grad = torch.full((wl.nq, ld), float("nan"), dtype=torch.float32, device="cuda")
    target = torch.full((wl.nq, ld), float("nan"), dtype=torch.float32, device="cuda")
    kl = torch.full((wl.nq,), float("nan"), dtype=torch.float32, device="cuda")
    loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_kl_dense(q, lay, wl.q_mla, wl.kv, lse, wl.softmax_scale, scores_d, grad, kl, target=target,
                             loss=loss)
    torch.cuda.synchronize()
    return grad.cpu().numpy(), target.cpu().numpy(), kl.cpu().numpy(), float(loss.item()), lse


def check_query(wl, ov, i, positions, scores_row, g_gpu, p_gpu, kl_gpu, where):
    """positions: the members of the set in output order; g_gpu and p_gpu hold
    the GPU's values in the same order."""
    r = ov.rows(i, positions)
    kv = bf16_bits(wl.kv[torch.from_numpy(r).cuda()]) if r.size else np.zeros((0, 576), np.uint16)
    x = scores_row[positions].astype(np.float64)
    kl_ref, g_ref, p_ref, mag = oracle.indexer_kl_query(bf16_bits(wl.q_mla[i]), kv, x, wl.softmax_scale)
    n = len(positions)
    dp = np.abs(p_gpu[:n] - p_ref)
    assert (dp <= P_RTOL * p_ref + 1e-12).all(), f"{where}: target err {dp.max():.3e}"
    soft = g_ref + p_ref  # Softmax(I) over the set
    dg = np.abs(g_gpu[:n] - g_ref)
    assert (dg <= P_RTOL * (p_ref + soft) + 1e-12).all(), f"{where}: grad err {dg.max():.3e}"
    assert abs(kl_gpu - kl_ref) <= KL_RTOL * (1.0 + mag), f"{where}: kl {kl_gpu} vs {kl_ref} (mag {mag:.3e})"
    return kl_ref


@pytest.mark.parametrize("paged", [False, True])
def test_sparse_kl_ragged_sets(paged):
    banner(f"kl sparse ragged paged={paged}")
    wl = make_custom(seq_lens=[1, 2, 31, 33, 100, 2047, 2048, 2049, 7000], device="cuda", seed=61, paged=paged)
    k = 2048
    idx, cnt = random_selection(wl, k, 5)
    s_h, s_d = synthetic_scores(wl, 6)
    grad, target, kl, loss, _ = run_sparse(wl, idx, cnt, k, s_d)
    ov = OracleView(wl)
    for i in range(wl.nq):
        c = int(cnt[i])
        check_query(wl, ov, i, idx[i, :c], s_h[i], grad[i], target[i], kl[i], f"q{i}")
        assert (grad[i, c:] == 0).all() and (target[i, c:] == 0).all()
    assert kl[0] == 0.0 and grad[0, 0] == 0.0 and target[0, 0] == 1.0  # one member: p = q = 1
    assert abs(loss - kl.astype(np.float64).sum()) <= 1e-6 * max(1.0, abs(loss))  # the sum of the terms


def test_sparse_kl_skips_entries_outside_history():
    """-1 and out-of-range entries inside count are not members: grad and
    target 0 there, and the loss over the remaining members."""
    banner("kl sparse invalid entries")
    wl = make_custom(seq_lens=[500, 3000], device="cuda", seed=62)
    k = 256
    idx, cnt = random_selection(wl, k, 7)
    idx[0, 3] = -1
    idx[0, 10] = 500
    idx[1, 0] = 99999
    s_h, s_d = synthetic_scores(wl, 8)
    # The attention's lse over the same members (the MLA call skips such entries too).
    grad, target, kl, _, _ = run_sparse(wl, idx, cnt, k, s_d)
    ov = OracleView(wl)
    for i in range(wl.nq):
        c = int(cnt[i])
        nv = int(wl.q_nvis[i])
        keep = [j for j in range(c) if 0 <= idx[i, j] < nv]
        drop = [j for j in range(c) if not 0 <= idx[i, j] < nv]
        assert drop
        check_query(wl, ov, i, idx[i, keep], s_h[i], grad[i, keep], target[i, keep], kl[i], f"q{i}")
        assert (grad[i, drop] == 0).all() and (target[i, drop] == 0).all()


def test_sparse_kl_many_queries():
    """Prefill-shaped: 300 causal queries of one sequence, sets up to k = 1024
    (several tiles and a ragged last tile per target block)."""
    banner("kl sparse 300 prefill queries")
    wl = make_custom(seq_lens=[3000], device="cuda", seed=63, prefill=True, queries_per_seq=300)
    k = 1024
    idx, cnt = random_selection(wl, k, 9)
    s_h, s_d = synthetic_scores(wl, 10)
    grad, target, kl, _, _ = run_sparse(wl, idx, cnt, k, s_d)
    ov = OracleView(wl)
    for i in [0, 1, 77, 298, 299]:
        c = int(cnt[i])
        check_query(wl, ov, i, idx[i, :c], s_h[i], grad[i], target[i], kl[i], f"q{i}")


@pytest.mark.parametrize("paged,block", [(False, 64), (True, 64), (True, 256)])
def test_dense_kl_decode(paged, block):
    banner(f"kl dense decode paged={paged} block={block}")
    wl = make_custom(seq_lens=[0, 1, 33, 2048, 5000], device="cuda", seed=64, paged=paged, block_size=block)
    s_h, s_d = synthetic_scores(wl, 11)
    grad, target, kl, _, _ = run_dense(wl, s_d)
    ov = OracleView(wl)
    nv = wl.q_nvis.cpu().numpy()
    assert kl[0] == 0.0
    for i in range(1, wl.nq):
        n = int(nv[i])
        check_query(wl, ov, i, np.arange(n), s_h[i], grad[i], target[i], kl[i], f"q{i}")
        assert np.isnan(grad[i, n:]).all()  # past the history: untouched


def test_dense_kl_long_history():
    """40000 positions: the target runs over many workgroups of one query and
    the loss kernel streams the whole history."""
    banner("kl dense 40000 positions")
    wl = make_custom(seq_lens=[40000, 1500], device="cuda", seed=65)
    s_h, s_d = synthetic_scores(wl, 12, std=1.0)
    grad, target, kl, _, _ = run_dense(wl, s_d)
    ov = OracleView(wl)
    for i in range(wl.nq):
        n = int(wl.q_nvis[i])
        check_query(wl, ov, i, np.arange(n), s_h[i], grad[i], target[i], kl[i], f"q{i}")


def test_dense_equals_sparse_over_all_positions_bit_exact():
    """Given the same lse, the dense call and the sparse call with idx = 0..n-1
    read the same rows in the same order: identical bits."""
    banner("kl dense vs sparse")
    wl = make_custom(seq_lens=[2048, 700], device="cuda", seed=66, prefill=True, queries_per_seq=40)
    k = 2048
    nv = wl.q_nvis.cpu().numpy()
    idx = np.full((wl.nq, k), -1, np.int32)
    for i in range(wl.nq):
        idx[i, :nv[i]] = np.arange(nv[i])
    cnt = np.minimum(nv, k).astype(np.int32)
    s_h, s_d = synthetic_scores(wl, 13)
    _, _, _, _, lse = run_dense(wl, s_d)
    g_d, p_d, kl_d, loss_d, _ = run_dense(wl, s_d, lse=lse)
    g_s, p_s, kl_s, loss_s, _ = run_sparse(wl, idx, cnt, k, s_d, lse=lse)
    for i in range(wl.nq):
        n = int(nv[i])
        assert (g_d[i, :n].view(np.uint32) == g_s[i, :n].view(np.uint32)).all()
        assert (p_d[i, :n].view(np.uint32) == p_s[i, :n].view(np.uint32)).all()
    assert (kl_d.view(np.uint32) == kl_s.view(np.uint32)).all() and loss_d == loss_s


def test_deterministic():
    banner("kl determinism")
    wl = make_custom(seq_lens=[6000, 3000], device="cuda", seed=67)
    k = 2048
    idx, cnt = random_selection(wl, k, 14)
    _, s_d = synthetic_scores(wl, 15)
    a = run_sparse(wl, idx, cnt, k, s_d)
    b = run_sparse(wl, idx, cnt, k, s_d, lse=a[4])
    for x, y in zip(a[:3], b[:3]):
        assert (x.view(np.uint32) == y.view(np.uint32)).all()


def test_kl_degenerate_cases():
    """k = 1 (every set one member: p = Softmax = 1, KL = 0, gradient 0), and an
    empty batch, which still writes the loss (0)."""
    banner("kl degenerate")
    wl = make_custom(seq_lens=[5, 3000], device="cuda", seed=68)
    idx, cnt = random_selection(wl, 1, 16)
    _, s_d = synthetic_scores(wl, 17)
    grad, target, kl, loss, _ = run_sparse(wl, idx, cnt, 1, s_d)
    assert (kl == 0).all() and (grad == 0).all() and (target == 1).all() and loss == 0.0
    q = dsa.Queries(wl.q_seq[:0], wl.q_nvis[:0], 0)
    _, lay = layout_of(wl)
    loss_t = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    e = torch.empty((0,), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_kl_dense(q, lay, wl.q_mla[:0], wl.kv, e.view(0, 128), wl.softmax_scale, e.view(0, 64),
                             e.view(0, 64), e, loss=loss_t)
    torch.cuda.synchronize()
    assert loss_t.item() == 0.0


def test_kl_minus_inf_scores():
    """Indexer scores of -inf (softmax weight 0), including each query's first
    set member: no NaN; the gradient is -p there and Softmax - p elsewhere, and
    the KL term is +inf (the target puts mass on every member)."""
    banner("kl -inf scores")
    wl = make_custom(seq_lens=[300, 2500], device="cuda", seed=69)
    k = 2048
    idx, cnt = random_selection(wl, k, 18)
    s_h, _ = synthetic_scores(wl, 19)
    for i in range(wl.nq):
        s_h[i, idx[i, :cnt[i]:7]] = -np.inf  # every 7th member, member 0 included
    grad, target, kl, loss, _ = run_sparse(wl, idx, cnt, k, torch.from_numpy(s_h).cuda())
    ov = OracleView(wl)
    for i in range(wl.nq):
        c = int(cnt[i])
        pos = idx[i, :c]
        r = ov.rows(i, pos)
        kv = bf16_bits(wl.kv[torch.from_numpy(r).cuda()])
        kl_ref, g_ref, p_ref, _ = oracle.indexer_kl_query(bf16_bits(wl.q_mla[i]), kv, s_h[i, pos].astype(np.float64),
                                                          wl.softmax_scale)
        assert kl_ref == np.inf and kl[i] == np.inf, f"q{i}: kl {kl[i]}"
        assert np.isfinite(grad[i, :c]).all() and np.isfinite(target[i, :c]).all()
        assert (np.abs(target[i, :c] - p_ref) <= P_RTOL * p_ref + 1e-12).all()
        soft = g_ref + p_ref
        assert (np.abs(grad[i, :c] - g_ref) <= P_RTOL * (p_ref + soft) + 1e-12).all(), f"q{i}: grad"
    assert loss == np.inf
