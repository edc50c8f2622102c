"""Pins for the oracle's sparse MQA-mode MLA attention: closed forms (one row,
two rows, zero query), a pure-Python brute force, permutation and paging
invariance, and the n_vis <= k reduction to full attention."""

import math

import numpy as np
import torch

from oracle import dsa, layout

SCALE = 1.0 / math.sqrt(192.0)


def bf16_bits(x):
    t = torch.from_numpy(np.asarray(x, np.float32).copy()).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_vals(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def rand_case(seed, h, n):
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal((h, 576))), bf16_bits(rng.standard_normal((n, 576)))


def test_single_row_returns_its_value_exactly():
    q, kv = rand_case(1, 8, 1)
    o, lse = dsa.sparse_mla(q, kv, SCALE)
    v = bf16_vals(kv)[0, :512]
    assert (o == v[None, :]).all()
    z = SCALE * (bf16_vals(q) @ bf16_vals(kv)[0])
    assert np.allclose(lse, z, rtol=0, atol=1e-12)


def test_two_rows_closed_form():
    q, kv = rand_case(2, 4, 2)
    o, lse = dsa.sparse_mla(q, kv, SCALE)
    qv, kvv = bf16_vals(q), bf16_vals(kv)
    for h in range(4):
        z1 = SCALE * float(qv[h] @ kvv[0])
        z2 = SCALE * float(qv[h] @ kvv[1])
        a = 1.0 / (1.0 + math.exp(z2 - z1))
        want = a * kvv[0, :512] + (1 - a) * kvv[1, :512]
        assert np.allclose(o[h], want, rtol=1e-12, atol=1e-12)
        assert abs(lse[h] - (max(z1, z2) + math.log1p(math.exp(-abs(z1 - z2))))) < 1e-12


def test_zero_query_gives_the_mean_value_row():
    _, kv = rand_case(3, 1, 37)
    q = np.zeros((3, 576), np.uint16)
    o, lse = dsa.sparse_mla(q, kv, SCALE)
    mean = bf16_vals(kv)[:, :512].mean(axis=0)
    assert np.allclose(o, mean[None, :], rtol=1e-13, atol=1e-13)
    assert np.allclose(lse, math.log(37))


def test_pure_python_brute_force():
    q, kv = rand_case(4, 2, 3)
    o, lse = dsa.sparse_mla(q, kv, SCALE)
    qv, kvv = bf16_vals(q).tolist(), bf16_vals(kv).tolist()
    for h in range(2):
        logits = [SCALE * sum(qv[h][d] * kvv[r][d] for d in range(576)) for r in range(3)]
        mx = max(logits)
        ex = [math.exp(z - mx) for z in logits]
        tot = sum(ex)
        for d in (0, 1, 255, 511):
            want = sum(ex[r] * kvv[r][d] for r in range(3)) / tot
            assert abs(o[h, d] - want) < 1e-12
        assert abs(lse[h] - (mx + math.log(tot))) < 1e-12


def test_row_permutation_invariance_and_empty_set():
    q, kv = rand_case(5, 16, 50)
    o, lse = dsa.sparse_mla(q, kv, SCALE)
    perm = np.random.default_rng(0).permutation(50)
    o2, lse2 = dsa.sparse_mla(q, kv[perm], SCALE)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-13) and np.allclose(lse, lse2, rtol=1e-13)
    oe, lsee = dsa.sparse_mla(q, kv[:0], SCALE)
    assert (oe == 0).all() and np.isneginf(lsee).all()


def test_short_history_degrades_to_full_attention():
    rng = np.random.default_rng(6)
    n, k = 300, 2048
    q8 = rng.integers(0, 0x70, (64, 128)).astype(np.uint8)
    k8 = rng.integers(0, 0x70, (n, 128)).astype(np.uint8)
    qs = np.ones(64, np.float32)
    ks = np.ones(n, np.float32)
    w = rng.standard_normal(64).astype(np.float32)
    q, kv = rand_case(7, 128, n)
    o, lse, idx, count, scores = dsa.forward_query(q8, qs, w, k8, ks, q, kv, k, SCALE)
    assert scores is None and count == n and list(idx[:n]) == list(range(n))
    od, lsed = dsa.dense_mla(q, kv, SCALE)
    assert np.allclose(o, od, rtol=1e-10, atol=1e-12) and np.allclose(lse, lsed, rtol=1e-12)


def test_composed_toy_selects_and_attends_rows_2_and_5():
    toy = np.array([0.1, 0.2, 0.8, 0.1, 0.1, 0.7, 0.1, 0.1], np.float32)
    keys = np.zeros((8, 128), np.float32)
    keys[:, 0] = toy
    from oracle import fp8
    k8, ks = fp8.quantize_rows(keys)
    qq = np.zeros((1, 128), np.float32)
    qq[0, 0] = 1.0
    q8, qs = fp8.quantize_rows(qq)
    q, kv = rand_case(8, 4, 8)
    o, lse, idx, count, _ = dsa.forward_query(q8, qs, np.ones(1, np.float32), k8, ks, q, kv, 2, SCALE)
    assert count == 2 and list(idx) == [2, 5]
    o2, lse2 = dsa.sparse_mla(q, kv[[2, 5]], SCALE)
    assert (o == o2).all() and (lse == lse2).all()


def test_paged_layout_maps_like_a_hand_built_table():
    bt = np.array([[3, 0], [1, 2]], np.int32)
    rows = layout.phys_rows(1, [0, 1, 63, 64, 100], block_table=bt, block_size=64)
    assert list(rows) == [64, 65, 127, 128, 164]
    rows0 = layout.phys_rows(0, [0, 65], block_table=bt, block_size=64)
    assert list(rows0) == [192, 1]
    rc = layout.phys_rows(1, [0, 5], row0=np.array([0, 4096]), block_size=0)
    assert list(rc) == [4096, 4101]


def test_paging_invariance():
    rng = np.random.default_rng(9)
    q, kv = rand_case(10, 8, 256)
    idx = np.sort(rng.choice(256, 40, replace=False))
    o, lse = dsa.sparse_mla(q, kv[idx], SCALE)
    perm = rng.permutation(4)  # 4 blocks of 64 placed in a shuffled order
    paged = np.zeros_like(kv)
    for b in range(4):
        paged[perm[b] * 64:(perm[b] + 1) * 64] = kv[b * 64:(b + 1) * 64]
    rows = layout.phys_rows(0, idx, block_table=perm[None, :], block_size=64)
    o2, lse2 = dsa.sparse_mla(q, paged[rows], SCALE)
    assert (o == o2).all() and (lse == lse2).all()
