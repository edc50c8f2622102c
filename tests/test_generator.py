"""Pins of the seeded workload generator (the one module both the HIP path's
tests and the oracle read their inputs from).  It holds none of the method's
arithmetic; what is pinned here is reproducibility: the same seed gives the same
bytes (stored SHA-256 digests, written by tests/golden/make_generator_hashes.py,
which calls only the generator), any 65536-row chunk can be regenerated on its
own from its chunk seed, and the planted-key structure has the stated shape."""

import json
import math
import os

import numpy as np
import torch

from workloads import gen, make_custom

HERE = os.path.dirname(os.path.abspath(__file__))


def _load():
    import importlib.util
    spec = importlib.util.spec_from_file_location("mgh", os.path.join(HERE, "golden", "make_generator_hashes.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_generator_bytes_match_stored_digests():
    stored = json.load(open(os.path.join(HERE, "golden", "generator_hashes.json")))
    got = _load().compute()
    for name, case in stored["cases"].items():
        assert got[name] == case["sha256"], name


def test_any_chunk_regenerates_on_its_own():
    rows, cols, seed = 3 * gen.CHUNK + 77, 8, 5
    full = gen._normal((rows, cols), "cpu", seed)
    for c in (0, 2, 3):
        c0, c1 = c * gen.CHUNK, min(rows, (c + 1) * gen.CHUNK)
        g = torch.Generator(device="cpu")
        g.manual_seed(seed * 7919 + c)
        alone = torch.randn((c1 - c0, cols), generator=g)
        assert torch.equal(full[c0:c1], alone), c


def test_same_seed_same_bytes_different_seed_different_bytes():
    a = make_custom(seq_lens=[900, 50], device="cpu", seed=3, paged=True)
    b = make_custom(seq_lens=[900, 50], device="cpu", seed=3, paged=True)
    c = make_custom(seq_lens=[900, 50], device="cpu", seed=4, paged=True)
    for f in ("q_idx", "w", "k_idx", "q_mla", "kv", "block_table"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
        assert not torch.equal(getattr(a, f), getattr(c, f)), f


def test_planted_rows_and_paged_permutation():
    L = [3000, 150, 12800]
    wl = make_custom(seq_lens=L, device="cpu", seed=9, plant=True)
    for s, n in enumerate(L):
        npl = int(math.floor(0.01 * n))
        pos = wl.planted.get(s, np.zeros(0, np.int64))
        assert len(pos) == npl and len(set(pos.tolist())) == npl and (np.diff(pos) > 0).all()
        if npl:
            rows = int(wl.row0[s]) + pos
            mean = wl.q_idx[s].mean(dim=0)
            dev = wl.k_idx[torch.from_numpy(rows)] - mean  # 0.5 N(0,1) noise around the query's head mean
            assert abs(float(dev.std()) - 0.5) < 0.1 and abs(float(dev.mean())) < 0.1
    p = make_custom(seq_lens=[1000, 64, 129], device="cpu", seed=9, paged=True)
    bt = p.block_table.numpy()
    used = np.concatenate([bt[0, :16], bt[1, :1], bt[2, :3]])
    assert sorted(used.tolist()) == list(range(p.rows // 64))  # one permutation of the physical blocks
