"""GPU parity of dsa_indexer_scores against the oracle (tolerance 1e-3 of the
magnitude M = sum_j |w_j| ReLU(dot_j)), plus a bit-exact case where every fp32
partial sum is exact."""

import numpy as np
import pytest
import torch

import oracle
import sparse_long_context_dsa_amd as dsa
from gpu_util import GpuInputs, OracleView, banner, check_scores
from workloads import make_config, make_custom

pytestmark = pytest.mark.gpu


def compare(wl, queries=None, ld=None):
    g = GpuInputs(wl)
    s = g.scores(ld)
    torch.cuda.synchronize()
    ov = OracleView(wl)
    worst = 0.0
    nv = wl.q_nvis.cpu().numpy()
    host = s.cpu().numpy()
    for i in (range(wl.nq) if queries is None else queries):
        ref, mag = ov.indexer(i)
        n = int(nv[i])
        worst = max(worst, check_scores(host[i, :n], ref, mag, f"{wl.name} query {i}"))
        if n < host.shape[1]:
            assert np.isnan(host[i, n:]).all(), "scores written past n_vis"
    return worst


def test_config0_decode_4096():
    banner("indexer config 0")
    compare(make_config(0, device="cuda"))


def test_ragged_contiguous_tails():
    banner("indexer ragged contiguous")
    wl = make_custom(seq_lens=[1, 63, 64, 65, 1000, 4097, 9000, 0], device="cuda", seed=11)
    compare(wl)


def test_paged_with_planted_keys():
    banner("indexer paged planted")
    wl = make_custom(seq_lens=[300, 5000, 64, 12345], device="cuda", seed=12, paged=True, plant=True)
    compare(wl)


def test_paged_block_256():
    banner("indexer paged block 256")
    wl = make_custom(seq_lens=[700, 2500], device="cuda", seed=14, paged=True, block_size=256)
    compare(wl)


def test_prefill_queries_share_a_sequence():
    banner("indexer prefill")
    wl = make_custom(seq_lens=[5000], device="cuda", seed=13, prefill=True, queries_per_seq=40)
    compare(wl, ld=5056)


def test_exact_grid_values_bit_exact():
    """q, k on {0, +-0.5, +-1, +-2}, unit scales, power-of-two weights: every
    product and partial sum is exact in fp32, so the GPU must match bit for bit."""
    banner("indexer exact grid")
    rng = np.random.default_rng(21)
    vals = np.array([0x00, 0x30, 0x38, 0x40, 0xB0, 0xB8, 0xC0], np.uint8)  # 0, .5, 1, 2, -.5, -1, -2
    nq, L = 3, 1500
    q8 = rng.choice(vals, (nq, 64, 128))
    k8 = rng.choice(vals, (nq * L, 128))
    qs = np.ones((nq, 64), np.float32)
    ks = (2.0 ** rng.integers(-3, 4, nq * L)).astype(np.float32)
    w = ((2.0 ** rng.integers(-4, 2, (nq, 64))) * rng.choice([-1, 1], (nq, 64))).astype(np.float32)
    dev = "cuda"
    queries = dsa.Queries(torch.arange(nq, dtype=torch.int32, device=dev),
                          torch.full((nq,), L, dtype=torch.int32, device=dev), L)
    layout = dsa.KvLayout(nq, nq * L, seq_row0=torch.arange(nq, dtype=torch.int64, device=dev) * L)
    scores = torch.empty((nq, 1504), dtype=torch.float32, device=dev)
    dsa.dsa_indexer_scores(queries, layout, torch.from_numpy(q8).to(dev), torch.from_numpy(qs).to(dev),
                           torch.from_numpy(w).to(dev), torch.from_numpy(k8).to(dev), torch.from_numpy(ks).to(dev),
                           scores)
    host = scores.cpu().numpy()
    for i in range(nq):
        ref, _ = oracle.indexer_scores_query(q8[i], qs[i], w[i], k8[i * L:(i + 1) * L], ks[i * L:(i + 1) * L])
        assert (host[i, :L].astype(np.float64) == ref).all()
