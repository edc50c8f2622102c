"""GPU parity of the decode attention's head-group path against the oracle's
sparse attention.  Decode batches of up to 64 queries split each query's 128
heads over four workgroups of 32.  From 48 to 64 queries each attends over the
whole selection and writes final outputs (no partials, no combine); up to 32
queries split the selection's rows as well (S splits, (O / l, lse) partials
merged by the combine kernel); 33 to 47 and more than 64 queries take the
row-split kernel.  These tests drive both forms with partial and empty tiles
and splits, paged caches, positions outside the history, a NULL count array
and a paged pool beyond 4 GiB, at the same tolerances as the other attention
tests (max-abs <= 2e-2 * max|O|, mean-abs <= 5e-3 * mean|O| per query, lse
within 2e-3)."""

import numpy as np
import pytest
import torch

import sparse_long_context_dsa_amd as dsa
from gpu_util import OracleView, banner, bf16_bits, check_out
from test_gpu_mla import compare, random_selection, run_mla
from workloads import make_custom

pytestmark = pytest.mark.gpu


def widen(seq_lens, n=48):
    """The lengths repeated, or cut, to n queries."""
    reps = (n + len(seq_lens) - 1) // len(seq_lens)
    return (list(seq_lens) * reps)[:n]


def test_hg_ragged_lengths_paged():
    banner("mla head groups: ragged lengths, paged")
    lens = [1, 31, 33, 100, 2047, 2048, 2049, 7000]
    wl = make_custom(seq_lens=widen(lens), device="cuda", seed=61, paged=True)
    idx, cnt = random_selection(wl, 2048, 11)
    compare(wl, idx, cnt, 2048, True, queries=list(range(0, 48, 5)) + [47])


def test_hg_counts_around_tile_edges():
    """Selections of 0 .. 2048 rows: empty, one row (returned exactly), and
    counts on both sides of the 16-row tile, the 8-row line group and the
    four-wavefront round of tiles."""
    banner("mla head groups: counts around tile edges")
    counts = [0, 1, 2, 7, 8, 9, 15, 16, 17, 63, 64, 65, 79, 80, 100, 1000, 1023, 1024, 2047, 2048]
    wl = make_custom(seq_lens=[3000] * 64, device="cuda", seed=62)
    cnt_all = np.array(widen(counts, 64), np.int32)
    idx, cnt = random_selection(wl, 2048, 12, counts=cnt_all)
    out, lse = run_mla(wl, idx, cnt, 2048, True)
    ov = OracleView(wl)
    for i in range(len(counts)):
        c = int(cnt[i])
        if c == 0:
            assert (out[i] == 0).all() and np.isneginf(lse[i]).all(), f"q{i}: empty selection"
            continue
        if c == 1:
            row = int(wl.row0[i].item()) + int(idx[i, 0])
            v = (bf16_bits(wl.kv[row]).astype(np.uint32) << 16).view(np.float32)[:512]
            assert (out[i] == v[None, :]).all(), f"q{i}: one selected row must be returned exactly"
        o_ref, l_ref = ov.mla(i, idx[i, :c])
        check_out(out[i], o_ref, lse[i], l_ref, f"head groups q{i} count {c}")


def test_hg_count_null_means_min_k_nvis():
    banner("mla head groups: count NULL, k = 1024")
    wl = make_custom(seq_lens=widen([700, 3000], 64), device="cuda", seed=63)
    idx, cnt = random_selection(wl, 1024, 13)
    compare(wl, idx, cnt, 1024, True, queries=[0, 1, 62, 63], with_count=False)


def test_hg_positions_outside_history_are_skipped():
    banner("mla head groups: out-of-range positions")
    wl = make_custom(seq_lens=widen([3000, 900, 64]), device="cuda", seed=64, paged=True)
    idx, cnt = random_selection(wl, 2048, 14)
    nv = wl.q_nvis.cpu().numpy()
    rng = np.random.default_rng(15)
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
    out, lse = run_mla(wl, bad, cnt, 2048, True)
    ov = OracleView(wl)
    for i in [0, 1, 2, 46, 47]:
        o_ref, l_ref = ov.mla(i, valid[i])
        check_out(out[i], o_ref, lse[i], l_ref, f"head groups out-of-range q{i}")


def _same_first_eight(n_other, n_hg, seed):
    """Two batches whose first eight queries hold identical inputs and
    selections, of n_other and n_hg queries; returns both runs' outputs."""
    lens = [2100, 3000, 4096, 2500, 5000, 2048, 3333, 2222]
    wa = make_custom(seq_lens=lens + [2600] * (n_other - 8), device="cuda", seed=seed)
    wb = make_custom(seq_lens=lens + [2600] * (n_hg - 8), device="cuda", seed=seed)
    wb.q_mla[:8] = wa.q_mla[:8]
    for i, n in enumerate(lens):
        ra, rb = int(wa.row0[i].item()), int(wb.row0[i].item())
        wb.kv[rb:rb + n] = wa.kv[ra:ra + n]
    ia, ca = random_selection(wa, 2048, seed + 1)
    ib, cb = random_selection(wb, 2048, seed + 2)
    ib[:8], cb[:8] = ia[:8], ca[:8]
    a, la = run_mla(wa, ia, ca, 2048, True)
    b, lb = run_mla(wb, ib, cb, 2048, True)
    vmax = np.abs((bf16_bits(wa.kv).astype(np.uint32) << 16).view(np.float32)[:, :512]).max()
    return a[:8], la[:8], b[:8], lb[:8], vmax


@pytest.mark.parametrize("n_hg", [64, 8])
def test_hg_same_queries_as_split_path(n_hg):
    """Forty queries take the row-split path; the same first eight at the
    head of a 64-query batch (head groups, one split) or alone (head groups,
    eight row splits) take the head-group kernel.  All attend over the same
    rows, so only the rounding of P to bf16 (relative to different running
    maxima) may differ: at most 2^-9 of each weight."""
    banner(f"mla head groups ({n_hg} queries) vs row splits (40 queries)")
    a, la, b, lb, vmax = _same_first_eight(40, n_hg, 65)
    assert np.abs(a - b).max() <= 2.0 ** -8 * vmax
    assert np.abs(la - lb).max() <= 1e-5 * np.abs(la).max()


@pytest.mark.parametrize("nq", [1, 5, 16, 20, 32])
def test_hg_row_splits_small_batches(nq):
    """Up to 32 queries: S = min(64 / nq, k / 128) row splits per head group
    (16, 12, 4, 3 and 2 here; 12 takes the combine's general form)."""
    banner(f"mla head groups with row splits: {nq} queries")
    lens = [4096, 2049, 30000, 2500, 7000, 2048, 100000, 3001]
    wl = make_custom(seq_lens=widen(lens, nq), device="cuda", seed=70 + nq, paged=nq % 2 == 0)
    idx, cnt = random_selection(wl, 2048, 19 + nq)
    compare(wl, idx, cnt, 2048, True, queries=sorted({0, nq // 2, nq - 1}))


def test_hg_split_counts_around_split_edges():
    """16 queries at k = 2048: four splits of 512 rows.  Counts on both sides
    of each split boundary leave later splits empty or with one row; one row
    in all is still returned exactly through the combine."""
    banner("mla head groups: counts around split edges")
    counts = [0, 1, 127, 128, 129, 511, 512, 513, 1024, 1025, 1535, 1536, 1537, 2000, 2047, 2048]
    wl = make_custom(seq_lens=[3000] * 16, device="cuda", seed=66)
    idx, cnt = random_selection(wl, 2048, 20, counts=np.array(counts, np.int32))
    out, lse = run_mla(wl, idx, cnt, 2048, True)
    ov = OracleView(wl)
    for i, c in enumerate(counts):
        if c == 0:
            assert (out[i] == 0).all() and np.isneginf(lse[i]).all(), f"q{i}: empty selection"
            continue
        if c == 1:
            row = int(wl.row0[i].item()) + int(idx[i, 0])
            v = (bf16_bits(wl.kv[row]).astype(np.uint32) << 16).view(np.float32)[:512]
            assert (out[i] == v[None, :]).all(), f"q{i}: one selected row must be returned exactly"
        o_ref, l_ref = ov.mla(i, idx[i, :c])
        check_out(out[i], o_ref, lse[i], l_ref, f"head-group splits q{i} count {c}")


def test_hg_row_splits_count_null_k_1024():
    banner("mla head groups with row splits: count NULL, k = 1024")
    wl = make_custom(seq_lens=[700, 3000, 1024, 1500], device="cuda", seed=67)
    idx, cnt = random_selection(wl, 1024, 21)
    compare(wl, idx, cnt, 1024, True, with_count=False)


@pytest.mark.parametrize("nq", [48, 40, 6])
def test_hg_paged_pool_beyond_4gib(nq):
    """A batch over a 4.4 GB paged pool whose block table alternates blocks
    at its start and end (row offsets beyond 32 bits: the 64-bit gather form),
    for each decode form: head groups (48), row splits (40), head groups with
    row splits (6)."""
    from types import SimpleNamespace
    banner(f"mla decode {nq} queries: paged pool > 4 GiB")
    bs, nblocks = 64, 59392                     # 3,801,088 rows x 1152 bytes = 4.38 GB
    rows = bs * nblocks
    seq_len, nseq = 4096, 2
    per_seq = seq_len // bs
    low = np.arange(nseq * per_seq // 2)
    high = nblocks - 1 - np.arange(nseq * per_seq // 2)
    order = np.empty(nseq * per_seq, np.int64)
    order[0::2], order[1::2] = low, high
    table = order.reshape(nseq, per_seq).astype(np.int32)
    kv = torch.empty((rows, 576), dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(78)
    for b in order:
        kv[b * bs:(b + 1) * bs] = torch.randn((bs, 576), generator=g, device="cuda").to(torch.bfloat16)
    q_mla = torch.randn((nq, 128, 576), generator=g, device="cuda").to(torch.bfloat16)
    wl = SimpleNamespace(
        name="paged pool 4.4 GB", nq=nq, num_seqs=nseq, rows=rows, kv=kv, q_mla=q_mla,
        q_seq=(torch.arange(nq, dtype=torch.int32, device="cuda") % nseq),
        q_nvis=torch.full((nq,), seq_len, dtype=torch.int32, device="cuda"), max_nvis=seq_len,
        block_size=bs, block_table=torch.from_numpy(table).cuda(), row0=None, softmax_scale=192 ** -0.5)
    idx, cnt = random_selection(wl, 2048, 18)
    compare(wl, idx, cnt, 2048, True, queries=[0, 1, nq - 1])
    del kv
    torch.cuda.empty_cache()
