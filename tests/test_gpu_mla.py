"""GPU parity of dsa_sparse_mla_decode / _prefill against the oracle's sparse
attention on the same selected positions (max-abs <= 2e-2 * max|O| and
mean-abs <= 5e-3 * mean|O| per query, lse within 2e-3), plus exact and
degenerate cases."""

import numpy as np
import pytest
import torch

import oracle
import sparse_long_context_dsa_amd as dsa
from gpu_util import OracleView, banner, bf16_bits, check_out
from workloads import make_custom

pytestmark = pytest.mark.gpu


def random_selection(wl, k, seed, counts=None):
    rng = np.random.default_rng(seed)
    nv = wl.q_nvis.cpu().numpy()
    idx = np.full((wl.nq, k), -1, np.int32)
    cnt = np.zeros(wl.nq, np.int32)
    for i in range(wl.nq):
        c = min(k, int(nv[i])) if counts is None else counts[i]
        sel = np.sort(rng.choice(int(nv[i]), c, replace=False)) if c else np.zeros(0, np.int64)
        idx[i, :c] = sel
        cnt[i] = c
    return idx, cnt


def run_mla(wl, idx, cnt, k, decode, with_count=True):
    g_idx = torch.from_numpy(idx).cuda()
    g_cnt = torch.from_numpy(cnt).cuda() if with_count else None
    q = dsa.Queries(wl.q_seq, wl.q_nvis, wl.max_nvis)
    if wl.block_size:
        lay = dsa.KvLayout(wl.num_seqs, wl.rows, block_table=wl.block_table, block_size=wl.block_size)
    else:
        lay = dsa.KvLayout(wl.num_seqs, wl.rows, seq_row0=wl.row0)
    out = torch.full((wl.nq, 128, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((wl.nq, 128), float("nan"), dtype=torch.float32, device="cuda")
    fn = dsa.dsa_sparse_mla_decode if decode else dsa.dsa_sparse_mla_prefill
    fn(q, lay, wl.q_mla, wl.kv, g_idx, g_cnt, k, wl.softmax_scale, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def compare(wl, idx, cnt, k, decode, queries=None, with_count=True):
    out, lse = run_mla(wl, idx, cnt, k, decode, with_count)
    ov = OracleView(wl)
    for i in (range(wl.nq) if queries is None else queries):
        o_ref, l_ref = ov.mla(i, idx[i, :cnt[i]])
        check_out(out[i], o_ref, lse[i], l_ref, f"{wl.name} q{i} decode={decode}")
    return out, lse


@pytest.mark.parametrize("decode", [True, False])
def test_single_query_2048_of_4096(decode):
    banner(f"mla single query decode={decode}")
    wl = make_custom(seq_lens=[4096], device="cuda", seed=41)
    idx, cnt = random_selection(wl, 2048, 1)
    compare(wl, idx, cnt, 2048, decode)


@pytest.mark.parametrize("decode", [True, False])
def test_ragged_counts_and_paging(decode):
    banner(f"mla ragged paged decode={decode}")
    wl = make_custom(seq_lens=[1, 31, 33, 100, 2047, 2048, 2049, 7000], device="cuda", seed=42, paged=True)
    idx, cnt = random_selection(wl, 2048, 2)
    compare(wl, idx, cnt, 2048, decode)


def test_count_null_means_min_k_nvis():
    banner("mla count NULL")
    wl = make_custom(seq_lens=[700, 3000], device="cuda", seed=43)
    idx, cnt = random_selection(wl, 1024, 3)
    compare(wl, idx, cnt, 1024, True, with_count=False)


def test_many_queries_split_counts():
    banner("mla 70 queries")
    wl = make_custom(seq_lens=[2500] * 70, device="cuda", seed=44)
    idx, cnt = random_selection(wl, 2048, 4)
    compare(wl, idx, cnt, 2048, True, queries=[0, 33, 69])
    compare(wl, idx, cnt, 2048, False, queries=[1, 68])


def test_empty_selection_and_single_row_exact():
    banner("mla empty and k=1")
    wl = make_custom(seq_lens=[50, 50], device="cuda", seed=45)
    idx = np.array([[-1], [17]], np.int32)
    cnt = np.array([0, 1], np.int32)
    for decode in (True, False):
        out, lse = run_mla(wl, idx, cnt, 1, decode)
        assert (out[0] == 0).all() and np.isneginf(lse[0]).all()
        row = int(wl.row0[1].item()) + 17  # position 17 of sequence 1
        v = bf16_bits(wl.kv[row]).astype(np.uint32) << 16
        vrow = v.view(np.float32)[:512]
        assert (out[1] == vrow[None, :]).all(), "one selected row must be returned exactly"


def test_index_order_does_not_matter():
    banner("mla permuted indices")
    wl = make_custom(seq_lens=[3000], device="cuda", seed=46)
    idx, cnt = random_selection(wl, 2048, 5)
    a, la = run_mla(wl, idx, cnt, 2048, False)
    perm = idx.copy()
    perm[0, :2048] = np.random.default_rng(0).permutation(idx[0, :2048])
    b, lb = run_mla(wl, perm, cnt, 2048, False)
    # Only the rounding of P to bf16 depends on the order (through the running
    # maximum each tile is scaled by): each weight moves by at most 2^-9 relative.
    vmax = np.abs((bf16_bits(wl.kv).astype(np.uint32) << 16).view(np.float32)[:, :512]).max()
    assert np.abs(a - b).max() <= 2.0 ** -8 * vmax
    assert np.abs(la - lb).max() <= 1e-5 * np.abs(la).max()
    ov = OracleView(wl)
    o_ref, l_ref = ov.mla(0, idx[0])
    check_out(b[0], o_ref, lb[0], l_ref, "permuted")


@pytest.mark.parametrize("decode", [True, False])
def test_positions_outside_history_are_skipped(decode):
    """Entries outside [0, q_nvis) break the contract; the kernels must then
    neither read past the cache nor let them into the softmax: the result is
    the attention over the valid entries alone (paged cache, tiles of which
    some are partial and some hold several such entries)."""
    banner(f"mla out-of-range positions decode={decode}")
    wl = make_custom(seq_lens=[3000, 900, 64], device="cuda", seed=47, paged=True)
    idx, cnt = random_selection(wl, 2048, 6)
    nv = wl.q_nvis.cpu().numpy()
    rng = np.random.default_rng(7)
    bad = idx.copy()
    valid = []
    for i in range(wl.nq):
        c = int(cnt[i])
        hit = rng.choice(c, size=min(c, 40), replace=False)
        vals = np.where(rng.random(hit.size) < 0.5, -1 - rng.integers(0, 1000, hit.size),
                        nv[i] + rng.integers(0, 1000, hit.size))
        bad[i, hit] = vals
        keep = np.ones(c, bool)
        keep[hit] = False
        valid.append(idx[i, :c][keep])
    out, lse = run_mla(wl, bad, cnt, 2048, decode)
    ov = OracleView(wl)
    for i in range(wl.nq):
        o_ref, l_ref = ov.mla(i, valid[i])
        check_out(out[i], o_ref, lse[i], l_ref, f"out-of-range q{i} decode={decode}")


@pytest.mark.parametrize("decode", [True, False])
def test_paged_pool_beyond_4gib(decode):
    """A paged latent pool of 4.4 GB (more than 4 GiB of rows) whose block
    table alternates blocks at the start and at the end of the pool, so that
    row offsets no longer fit in 32 bits."""
    from types import SimpleNamespace
    banner(f"mla paged pool > 4 GiB decode={decode}")
    bs, nblocks = 64, 59392                     # 3,801,088 rows x 1152 bytes = 4.38 GB
    rows = bs * nblocks
    seq_len, nseq = 4096, 2
    per_seq = seq_len // bs
    low = np.arange(nseq * per_seq // 2)
    high = nblocks - 1 - np.arange(nseq * per_seq // 2)
    order = np.empty(nseq * per_seq, np.int64)
    order[0::2], order[1::2] = low, high        # neighbours in a sequence lie ~4.3 GB apart
    table = order.reshape(nseq, per_seq).astype(np.int32)
    kv = torch.empty((rows, 576), dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    for b in order:
        kv[b * bs:(b + 1) * bs] = torch.randn((bs, 576), generator=g, device="cuda").to(torch.bfloat16)
    q_mla = torch.randn((nseq, 128, 576), generator=g, device="cuda").to(torch.bfloat16)
    wl = SimpleNamespace(
        name="paged pool 4.4 GB", nq=nseq, num_seqs=nseq, rows=rows, kv=kv, q_mla=q_mla,
        q_seq=torch.arange(nseq, dtype=torch.int32, device="cuda"),
        q_nvis=torch.full((nseq,), seq_len, dtype=torch.int32, device="cuda"), max_nvis=seq_len,
        block_size=bs, block_table=torch.from_numpy(table).cuda(), row0=None, softmax_scale=192 ** -0.5)
    idx, cnt = random_selection(wl, 2048, 9)
    compare(wl, idx, cnt, 2048, decode)
    del kv
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ dense mode


def run_dense(wl):
    q = dsa.Queries(wl.q_seq, wl.q_nvis, wl.max_nvis)
    if wl.block_size:
        lay = dsa.KvLayout(wl.num_seqs, wl.rows, block_table=wl.block_table, block_size=wl.block_size)
    else:
        lay = dsa.KvLayout(wl.num_seqs, wl.rows, seq_row0=wl.row0)
    out = torch.full((wl.nq, 128, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((wl.nq, 128), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_dense_mla(q, lay, wl.q_mla, wl.kv, wl.softmax_scale, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check_dense(wl, queries):
    out, lse = run_dense(wl)
    ov = OracleView(wl)
    for i in queries:
        r = ov.rows(i)
        kv = bf16_bits(wl.kv[torch.from_numpy(r).cuda()]) if r.size else np.zeros((0, 576), np.uint16)
        o_ref, l_ref = oracle.dense_mla(bf16_bits(wl.q_mla[i]), kv, wl.softmax_scale)
        check_out(out[i], o_ref, lse[i], l_ref, f"dense {wl.name} q{i}")
    return out, lse


@pytest.mark.parametrize("paged,block", [(False, 64), (True, 64), (True, 256)])
def test_dense_decode_against_oracle(paged, block):
    """Every visible position, one query per sequence: histories around tile
    and split boundaries, contiguous and paged caches (oracle: the separately
    written dense attention)."""
    banner(f"dense mla decode paged={paged} block={block}")
    wl = make_custom(seq_lens=[0, 1, 31, 33, 2048, 5000, 20000], device="cuda", seed=51, paged=paged,
                     block_size=block)
    out, lse = check_dense(wl, range(1, wl.nq))
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()


def test_dense_prefill_causal():
    banner("dense mla prefill")
    wl = make_custom(seq_lens=[3000], device="cuda", seed=52, prefill=True, queries_per_seq=300)
    check_dense(wl, [0, 1, 150, 298, 299])


def test_dense_history_longer_than_one_workgroup_holds():
    """70000 positions: more tiles than one workgroup's row table, so the
    launch must split the rows even for a single query."""
    banner("dense mla 70000 positions")
    wl = make_custom(seq_lens=[70000], device="cuda", seed=53)
    check_dense(wl, [0])


def test_dense_equals_sparse_over_all_positions_bit_exact():
    """With one workgroup per query (many queries), the dense mode and the
    sparse prefill given idx = 0 .. n-1 gather the same tiles in the same order:
    the outputs must agree bit for bit."""
    banner("dense vs sparse over every position")
    wl = make_custom(seq_lens=[2048] * 4, device="cuda", seed=54, prefill=True, queries_per_seq=150)
    out_d, lse_d = run_dense(wl)
    nv = wl.q_nvis.cpu().numpy()
    idx = np.full((wl.nq, 2048), -1, np.int32)
    for i in range(wl.nq):
        idx[i, :nv[i]] = np.arange(nv[i])
    out_s, lse_s = run_mla(wl, idx, np.minimum(nv, 2048).astype(np.int32), 2048, False)
    assert (out_d.view(np.uint32) == out_s.view(np.uint32)).all()
    assert (lse_d.view(np.uint32) == lse_s.view(np.uint32)).all()
