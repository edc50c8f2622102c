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
