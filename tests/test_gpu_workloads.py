"""Reproducibility of the workload generator on the GPU (the device tensors the
HIP path and, through host copies, the oracle read): the same seed gives the
same bytes, and any 65536-row chunk regenerates on its own from its seed."""

import pytest
import torch

from gpu_util import banner
from workloads import gen, make_custom

pytestmark = pytest.mark.gpu


def test_device_generation_is_reproducible():
    banner("generator on the device: twice the same bytes")
    kw = dict(seq_lens=[70000, 3000, 64], device="cuda", seed=21, plant=True)
    a, b = make_custom(**kw), make_custom(**kw)
    for f in ("q_idx", "w", "k_idx", "q_mla", "kv"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    rows, seed = a.rows, 21 * 10 + 5  # the latent cache's seed in make_custom
    c0, c1 = gen.CHUNK, min(rows, 2 * gen.CHUNK)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed * 7919 + 1)
    alone = torch.randn((c1 - c0, gen.D), generator=g, device="cuda").to(torch.bfloat16)
    assert torch.equal(a.kv[c0:c1], alone)
