"""GPU parity of dsa_topk: the oracle's top-k run on the same fp32 scores must
give the same index lists bit for bit (ties to the lower position, ascending
order, -1 padding), on the GPU's own indexer scores and on adversarial
synthetic scores (heavy ties, signed zeros, n around k, long rows)."""

import numpy as np
import pytest
import torch

import oracle
import sparse_long_context_dsa_amd as dsa
from gpu_util import GpuInputs, OracleView, banner, check_topk_near_ties
from workloads import make_config, make_custom

pytestmark = pytest.mark.gpu


def gpu_topk(scores_host, nvis, k):
    nq = len(nvis)
    ld = max(4, (int(max(nvis)) + 3) // 4 * 4) if nq else 4
    s = torch.zeros((nq, ld), dtype=torch.float32)
    for i, n in enumerate(nvis):
        s[i, :n] = torch.from_numpy(np.asarray(scores_host[i][:n], np.float32))
    s = s.cuda()
    q = dsa.Queries(torch.arange(nq, dtype=torch.int32, device="cuda"),
                    torch.tensor(nvis, dtype=torch.int32, device="cuda"), int(max(nvis)))
    idx = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((nq,), -7, dtype=torch.int32, device="cuda")
    dsa.dsa_topk(q, s, k, idx, cnt)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


def assert_same(scores_host, nvis, k, where):
    idx, cnt = gpu_topk(scores_host, nvis, k)
    for i, n in enumerate(nvis):
        ref, rc = oracle.topk(np.asarray(scores_host[i][:n], np.float32), k)
        assert cnt[i] == rc, f"{where} q{i}: count {cnt[i]} vs {rc}"
        assert (idx[i] == ref).all(), f"{where} q{i}: first mismatch at {np.argmax(idx[i] != ref)}"


def test_gpu_scores_config0_bit_exact_and_near_ties():
    banner("topk on config 0 scores")
    wl = make_config(0, device="cuda")
    g = GpuInputs(wl)
    s = g.scores().cpu().numpy()
    n = wl.max_nvis
    assert_same([s[0]], [n], 2048, "config0")
    idx, cnt = gpu_topk([s[0]], [n], 2048)
    ref, mag = OracleView(wl).indexer(0)
    check_topk_near_ties(idx[0], int(cnt[0]), ref, mag, 2048, "config0 vs oracle scores")


def test_gpu_scores_ragged_paged():
    banner("topk on ragged paged scores")
    wl = make_custom(seq_lens=[3000, 2048, 2049, 100, 17000, 8192, 8193], device="cuda", seed=31, paged=True,
                     plant=True)
    g = GpuInputs(wl)
    s = g.scores().cpu().numpy()
    nv = wl.q_nvis.cpu().numpy().tolist()
    assert_same(list(s), nv, 2048, "ragged")


@pytest.mark.parametrize("k", [1, 7, 2048])
def test_heavy_ties_and_signed_zero(k):
    banner(f"topk ties k={k}")
    rng = np.random.default_rng(k)
    nvis = [0, 1, k - 1 if k > 1 else 0, k, k + 1, 5000, 40000]
    rows = []
    for j, n in enumerate(nvis):
        if j % 3 == 0:
            v = rng.integers(0, 6, n).astype(np.float32)          # integer ties
        elif j % 3 == 1:
            v = rng.choice(np.array([0.0, -0.0, 1.0, -1.0, 0.5], np.float32), n)
        else:
            v = rng.standard_normal(n).astype(np.float32)
        rows.append(v)
    assert_same(rows, nvis, k, f"ties k={k}")


def test_all_equal_and_constant_rows():
    banner("topk all equal")
    rows = [np.full(20000, 1.5, np.float32), np.full(9000, -0.0, np.float32), np.zeros(3, np.float32)]
    assert_same(rows, [20000, 9000, 3], 2048, "all-equal")


def test_long_rows_131072():
    banner("topk long rows")
    rng = np.random.default_rng(77)
    rows = [rng.standard_normal(131072).astype(np.float32) for _ in range(3)]
    rows[1] = np.round(rows[1] * 4) / 4  # coarse values: many exact ties at the threshold
    assert_same(rows, [131072, 131072, 100000], 2048, "long")


def test_deterministic_repeat():
    banner("topk determinism")
    rng = np.random.default_rng(5)
    rows = [np.round(rng.standard_normal(50000) * 8).astype(np.float32) for _ in range(4)]
    a, ca = gpu_topk(rows, [50000] * 4, 2048)
    b, cb = gpu_topk(rows, [50000] * 4, 2048)
    assert (a == b).all() and (ca == cb).all()


def test_long_row_boundaries():
    """Just above the one-block row limit, a ragged span, and the longest
    history the library accepts (2^20), once with distinct values and once
    all equal (every position is a candidate; ties go to the lowest)."""
    banner("topk long-row boundaries")
    rng = np.random.default_rng(91)
    nvis = [16385, 24577, 1 << 20, 1 << 20]
    rows = [rng.standard_normal(16385).astype(np.float32),
            np.round(rng.standard_normal(24577) * 2).astype(np.float32),
            rng.standard_normal(1 << 20).astype(np.float32),
            np.full(1 << 20, 0.25, np.float32)]
    assert_same(rows, nvis, 2048, "long boundaries")


def test_short_rows_beside_long_rows():
    """A batch with one long row sends its short rows through the 1024-thread
    row selection of the long-row kernel: the largest short row (16384), one
    just above k, exactly k, a tiny one, with coarse values (many ties at the
    threshold), next to a long row."""
    banner("topk short rows beside a long row")
    rng = np.random.default_rng(23)
    nvis = [16384, 2049, 2048, 5, 40000]
    rows = [np.round(rng.standard_normal(n) * 3).astype(np.float32) for n in nvis]
    rows[0][::7] = 0.0
    rows[0][3::11] = -0.0
    assert_same(rows, nvis, 2048, "short beside long")
    assert_same(rows, nvis, 7, "short beside long, k = 7")


def test_many_rows_take_the_two_kernel_path():
    """Between 33 and 127 rows up to 131072 positions go through the two-kernel
    path (spans of 32768 per block, then one finishing block per row) instead
    of one streaming block per row; the same adversarial rows as above:
    integer ties, signed zeros, all equal (every key a candidate), coarse
    normals, short rows beside long ones."""
    banner("topk two-kernel path, 40 rows")
    rng = np.random.default_rng(41)
    nvis, rows = [], []
    for j in range(40):
        n = int(rng.choice([5, 2048, 2049, 16384, 16385, 40000, 70001, 131072]))
        kind = j % 5
        if kind == 0:
            v = rng.integers(0, 6, n).astype(np.float32)
        elif kind == 1:
            v = rng.choice(np.array([0.0, -0.0, 1.0, -1.0, 0.5], np.float32), n)
        elif kind == 2:
            v = np.full(n, -2.5, np.float32)
        elif kind == 3:
            v = np.round(rng.standard_normal(n) * 3).astype(np.float32)
        else:
            v = rng.standard_normal(n).astype(np.float32)
        nvis.append(n)
        rows.append(v)
    nvis[0], rows[0] = 131072, rng.standard_normal(131072).astype(np.float32)
    assert_same(rows, nvis, 2048, "two-kernel path")
    assert_same(rows, nvis, 3, "two-kernel path, k = 3")


def test_many_rows_streaming_again():
    """From 128 rows the streaming kernel is back (one block per row); 130
    rows of mixed lengths and patterns, some long enough that every key is a
    candidate and LDS overflows into the re-reading path."""
    banner("topk streaming, 130 rows")
    rng = np.random.default_rng(43)
    nvis, rows = [], []
    for j in range(130):
        n = int(rng.choice([7, 2049, 16385, 30000, 99999, 131072]))
        kind = j % 4
        if kind == 0:
            v = np.full(n, 0.75, np.float32)
        elif kind == 1:
            v = rng.choice(np.array([0.0, -0.0, 2.0, -1.0], np.float32), n)
        elif kind == 2:
            v = np.round(rng.standard_normal(n) * 2).astype(np.float32)
        else:
            v = rng.standard_normal(n).astype(np.float32)
        nvis.append(n)
        rows.append(v)
    assert_same(rows, nvis, 2048, "streaming, 130 rows")


@pytest.mark.parametrize("nq", [5, 300])
def test_short_rows_both_row_kernels(nq):
    """Rows of at most 16384 positions: batches of up to 256 rows take the
    1024-thread row kernel, larger ones the 256-thread one (several rows per
    CU).  The same mix for both: integer ties, signed zeros, all equal, n
    around k, the 16384 maximum."""
    banner(f"topk short rows, {nq} rows")
    rng = np.random.default_rng(47 + nq)
    nvis, rows = [], []
    for j in range(nq):
        n = int(rng.choice([0, 1, 2047, 2048, 2049, 4096, 9000, 16384]))
        kind = j % 4
        if kind == 0:
            v = rng.integers(0, 6, n).astype(np.float32)
        elif kind == 1:
            v = rng.choice(np.array([0.0, -0.0, 1.0, -1.0, 0.5], np.float32), n)
        elif kind == 2:
            v = np.full(n, 0.5, np.float32)
        else:
            v = rng.standard_normal(n).astype(np.float32)
        nvis.append(n)
        rows.append(v)
    nvis[0], rows[0] = 16384, rng.standard_normal(16384).astype(np.float32)
    assert_same(rows, nvis, 2048, f"short rows, {nq}")
    assert_same(rows, nvis, 5, f"short rows, {nq}, k = 5")


def _split_tie_row(rng, n, k, m):
    """N(0,1) scores with m more copies of the k-th largest value placed at
    random lower-ranked positions: k - 1 keys are larger and m + 1 equal it,
    so one of the ties is taken (the lowest position) and the boundary holds
    few keys (the one-wavefront ranking, not the third digit)."""
    v = rng.standard_normal(n).astype(np.float32)
    order = np.argsort(-v, kind="stable")
    kth = v[order[k - 1]]
    below = order[k:k + 2000]
    v[rng.choice(below, min(m, len(below)), replace=False)] = kth
    return v


@pytest.mark.parametrize("shape", ["stream", "row_wide", "row", "long"])
def test_few_ties_split_at_the_threshold(shape):
    banner(f"topk split ties, {shape}")
    rng = np.random.default_rng(2024 + len(shape))
    k = 2048
    nvis = {"stream": [4096, 16384, 50000, 131072], "row_wide": [4096, 16384, 2100],
            "row": [3000] * 260, "long": [131072, 70000] * 20}[shape]
    rows = [_split_tie_row(rng, n, k, int(rng.integers(1, 12))) for n in nvis]
    assert_same(rows, nvis, k, f"split ties {shape}")
