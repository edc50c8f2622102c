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


def e8m0_inputs(wl):
    """Device inputs with the keys quantised by the E8M0 variant: codes, bytes
    and the equal fp32 scales 2^(b - 127)."""
    g = GpuInputs(wl)
    k8 = torch.empty_like(g.k8)
    kb = torch.empty((wl.rows,), dtype=torch.uint8, device=k8.device)
    ks = torch.empty((wl.rows,), dtype=torch.float32, device=k8.device)
    dsa.dsa_quantize_fp8_e8m0(wl.k_idx, k8, kb, ks)
    return g, k8, kb, ks


def test_e8m0_key_scales_against_oracle():
    """dsa_indexer_scores_e8m0 on keys quantised with power-of-two scales,
    against the oracle fed the same E8M0 quantisation (ragged paged decode)."""
    banner("indexer e8m0 key scales")
    wl = make_custom(seq_lens=[1, 63, 65, 3000, 9000], device="cuda", seed=15, paged=True, plant=True)
    g, k8, kb, _ = e8m0_inputs(wl)
    ld = (wl.max_nvis + 63) // 64 * 64
    s = torch.full((wl.nq, ld), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_scores_e8m0(g.queries, g.layout, g.q8, g.qs, wl.w, k8, kb, s)
    torch.cuda.synchronize()
    host = s.cpu().numpy()
    nv = wl.q_nvis.cpu().numpy()
    ov = OracleView(wl)
    for i in range(wl.nq):
        ref, mag = ov.indexer(i, e8m0=True)
        n = int(nv[i])
        check_scores(host[i, :n], ref, mag, f"e8m0 query {i}")
        assert np.isnan(host[i, n:]).all()


def test_e8m0_equals_fp32_power_of_two_scales_bit_exact():
    """The E8M0 entry point and the fp32 one given the same scales 2^(b - 127)
    compute the same thing: the scores must agree bit for bit (decode 4 x 20000
    and a prefill batch)."""
    banner("indexer e8m0 vs fp32 scales")
    for wl in (make_custom(seq_lens=[20000] * 4, device="cuda", seed=16),
               make_custom(seq_lens=[3000], device="cuda", seed=17, prefill=True, queries_per_seq=64)):
        g, k8, kb, ks = e8m0_inputs(wl)
        ld = (wl.max_nvis + 63) // 64 * 64
        a = torch.full((wl.nq, ld), float("nan"), dtype=torch.float32, device="cuda")
        b = torch.full((wl.nq, ld), float("nan"), dtype=torch.float32, device="cuda")
        dsa.dsa_indexer_scores_e8m0(g.queries, g.layout, g.q8, g.qs, wl.w, k8, kb, a)
        dsa.dsa_indexer_scores(g.queries, g.layout, g.q8, g.qs, wl.w, k8, ks, b)
        torch.cuda.synchronize()
        av, bv = a.cpu().numpy(), b.cpu().numpy()
        assert (np.isnan(av) == np.isnan(bv)).all()
        fin = ~np.isnan(av)
        assert (av[fin].view(np.uint32) == bv[fin].view(np.uint32)).all()
