"""End-to-end parity of dsa_forward (indexer -> top-k -> sparse MLA):
* the selected positions equal the oracle's top-k of the GPU's own scores
  (dsa_indexer_scores runs the same kernel, so the scores are the ones
  dsa_forward selected from), bit for bit;
* against the oracle's own scores, differences are near-ties only;
* the output equals the oracle's attention over the GPU's positions;
* short histories (n_vis <= k) attend to everything;
* two runs are bit-identical."""

import pytest
import torch

from gpu_util import GpuInputs, banner, check_queries, run_forward
from workloads import make_config, make_custom

pytestmark = pytest.mark.gpu


def test_config0():
    banner("forward config 0")
    wl = make_config(0, device="cuda")
    g = GpuInputs(wl)
    out, lse, idx = run_forward(g)
    check_queries(wl, g, out, lse, idx, [0])
    # the pages' full-attention reading for histories that fit in k
    o2, l2, i2 = run_forward(g, k=2048)
    assert torch.equal(o2, out) and torch.equal(i2, idx), "forward is not deterministic"


def test_short_and_boundary_histories():
    banner("forward short histories")
    wl = make_custom(seq_lens=[1, 5, 2047, 2048, 2049, 3000, 0], device="cuda", seed=51)
    g = GpuInputs(wl)
    out, lse, idx = run_forward(g)
    check_queries(wl, g, out, lse, idx, range(wl.nq))


def test_prefill_small():
    banner("forward prefill small")
    wl = make_custom(seq_lens=[2600], device="cuda", seed=52, prefill=True)
    g = GpuInputs(wl)
    out, lse, idx = run_forward(g)
    check_queries(wl, g, out, lse, idx, [0, 1, 2, 100, 2047, 2048, 2049, 2050, 2599])


def test_small_k():
    banner("forward k=64")
    wl = make_custom(seq_lens=[500, 64, 65, 9000], device="cuda", seed=53, paged=True, plant=True)
    g = GpuInputs(wl)
    out, lse, idx = run_forward(g, k=64)
    check_queries(wl, g, out, lse, idx, range(wl.nq), k=64)


def _fwd_ws_bytes(g, k):
    import sparse_long_context_dsa_amd as dsa
    return dsa.dsa_workspace_bytes(dsa.DSA_OP_FORWARD, g.queries, k)


@pytest.mark.parametrize("paged", [False, True])
def test_prefill_where_the_indexer_selects(paged):
    """Two 6000-token causal prefills (12000 queries): one indexer block covers
    each query's whole history, so the indexer selects each row itself and no
    score leaves the chip (the forward's workspace then holds no score rows).
    Every query's positions equal the standalone top-k of the same scores
    (dsa_topk on dsa_indexer_scores), and sampled queries match the oracle."""
    import sparse_long_context_dsa_amd as dsa
    banner(f"forward prefill, indexer selects, paged={paged}")
    wl = make_custom(seq_lens=[6000, 6000], device="cuda", seed=54, prefill=True, paged=paged)
    g = GpuInputs(wl)
    assert _fwd_ws_bytes(g, wl.k) < wl.nq * 6000 * 4, "expected the selecting indexer (no score rows)"
    out, lse, idx = run_forward(g)
    ref = torch.full_like(idx, -7)
    dsa.dsa_topk(g.queries, g.scores(), wl.k, ref)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref), "indexer selection differs from the standalone top-k of the same scores"
    check_queries(wl, g, out, lse, idx, [0, 1, 2, 2047, 2048, 2049, 5999, 6000, 6001, 8048, 8049, 11999])


@pytest.mark.parametrize("k", [2048, 64])
def test_prefill_where_the_indexer_selects_heavy_ties(k):
    """The same path with five distinct key rows repeated along the cache, so
    every query's scores take five values and the selection is decided by
    the lower-position rule among exact ties."""
    import sparse_long_context_dsa_amd as dsa
    banner(f"forward prefill, indexer selects, heavy ties, k={k}")
    wl = make_custom(seq_lens=[9000], device="cuda", seed=55, prefill=True)
    wl.k_idx.copy_(wl.k_idx[torch.arange(wl.rows, device="cuda") % 5])
    g = GpuInputs(wl)
    assert _fwd_ws_bytes(g, k) < wl.nq * 9000 * 4, "expected the selecting indexer (no score rows)"
    out, lse, idx = run_forward(g, k=k)
    ref = torch.full_like(idx, -7)
    dsa.dsa_topk(g.queries, g.scores(), k, ref)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref)
    check_queries(wl, g, out, lse, idx, [0, 63, 64, 65, 2048, 2049, 4000, 8999], k=k, near_ties=False)


# ------------------------------------------------------------------ long rows
# Batches whose longest history lies in (16384, 131072]: the forward's top-k
# (streaming or two-kernel, from the indexer's fused histogram) must equal the
# standalone top-k of the same scores (which builds its own histogram).

def _standalone_topk(g, k):
    import sparse_long_context_dsa_amd as dsa
    ref = torch.full((g.wl.nq, k), -7, dtype=torch.int32, device="cuda")
    dsa.dsa_topk(g.queries, g.scores(), k, ref)
    torch.cuda.synchronize()
    return ref


@pytest.mark.parametrize("paged", [False, True])
def test_long_rows_mixed_lengths(paged):
    """Long rows, rows of at most 16384 (one block each) and rows of at most k
    (everything) in one batch."""
    banner(f"forward long rows, mixed lengths, paged={paged}")
    lens = [40000, 16384, 16385, 3000, 2048, 100000, 0, 131072, 2049, 65536]
    wl = make_custom(seq_lens=lens, device="cuda", seed=56, paged=paged, plant=True)
    g = GpuInputs(wl)
    out, lse, idx = run_forward(g)
    assert torch.equal(idx, _standalone_topk(g, wl.k)), "forward selection differs from the standalone top-k"
    check_queries(wl, g, out, lse, idx, [0, 2, 3, 4, 6, 8, 9])


@pytest.mark.parametrize("lens", [[9000, 12000, 5000], [40000] * 16, [131072] * 8 + [20000] * 56],
                         ids=["row-blocks", "streaming", "two-kernel"])
def test_rows_of_mostly_negative_scores(lens):
    """Rows whose head weights are all negative score below zero almost
    everywhere (the k-th key among negative keys, the threshold bins in the
    lower half of the first digit), beside rows with weights of either sign:
    on every top-k path the forward must select what the standalone top-k
    selects."""
    banner(f"forward, negative scores, {len(lens)} rows up to {max(lens)}")
    wl = make_custom(seq_lens=lens, device="cuda", seed=61)
    wl.w[::2] = -wl.w[::2].abs()   # every other query: all weights negative
    g = GpuInputs(wl)
    out, lse, idx = run_forward(g)
    assert torch.equal(idx, _standalone_topk(g, wl.k)), "forward selection differs from the standalone top-k"
    check_queries(wl, g, out, lse, idx, [0, 1])


@pytest.mark.parametrize("k", [2048, 100])
def test_long_rows_heavy_ties(k):
    """Five distinct key rows repeated along the cache: each score takes one of
    five values, a fifth of the row ties in the threshold bin (more than the
    candidate buffers hold), and ties keep the lowest positions."""
    banner(f"forward long rows, heavy ties, k={k}")
    wl = make_custom(seq_lens=[70000, 30000], device="cuda", seed=58)
    wl.k_idx.copy_(wl.k_idx[torch.arange(wl.rows, device="cuda") % 5])
    g = GpuInputs(wl)
    out, lse, idx = run_forward(g, k=k)
    assert torch.equal(idx, _standalone_topk(g, k))
    check_queries(wl, g, out, lse, idx, [0, 1], k=k, near_ties=False)


# ------------------------------------------------------------------ workspace state
@pytest.mark.parametrize("lens", [[9000, 12000, 5000], [40000] * 16, [131072] * 8 + [20000] * 56],
                         ids=["row-blocks", "streaming", "two-kernel"])
def test_forward_workspace_contents_do_not_matter(lens):
    """The forward leaves its top-k histograms zero in the workspace and does not
    clear them at the start of a call.  A workspace that holds other data (here
    0xA5 bytes) must give the same result, the histograms being checked against
    their rows' lengths and rebuilt, and must be left clean for the next call."""
    import sparse_long_context_dsa_amd as dsa
    banner(f"forward workspace contents, {len(lens)} rows up to {max(lens)}")
    wl = make_custom(seq_lens=lens, device="cuda", seed=59)
    g = GpuInputs(wl)
    k = wl.k

    def fwd(ws):
        out = torch.full((wl.nq, 128, 512), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((wl.nq, 128), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((wl.nq, k), -7, dtype=torch.int32, device="cuda")
        dsa.dsa_forward(g.queries, g.layout, g.q8, g.qs, wl.w, g.k8, g.ks, wl.q_mla, wl.kv, k, wl.softmax_scale,
                        out, lse, idx, ws=ws)
        torch.cuda.synchronize()
        return out, lse, idx

    ws = dsa.workspace(dsa.DSA_OP_FORWARD, g.queries, k)
    runs = [fwd(ws), fwd(ws)]
    ws.fill_(0xA5)
    runs += [fwd(ws), fwd(ws)]
    ref = _standalone_topk(g, k)
    for i, (out, lse, idx) in enumerate(runs):
        assert torch.equal(idx, ref), f"run {i}: selection differs from the standalone top-k"
        assert torch.equal(out, runs[0][0]) and torch.equal(lse, runs[0][1]), f"run {i}: output differs"
