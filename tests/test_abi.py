"""Host-only checks of the C ABI: the library loads, exports every function
include/dsa.h declares, sizes workspaces, and rejects bad arguments before it
launches anything (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

import sparse_long_context_dsa_amd as dsa
from sparse_long_context_dsa_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(dsa_\w+)\s*\(", text, flags=re.M)))


def test_library_is_built_and_loads():
    assert os.path.exists(dsa.lib_path()), "run `python -m sparse_long_context_dsa_amd.build` first"
    _lib.lib()


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_decode", "dsa_sparse_mla_prefill",
            "dsa_forward", "dsa_quantize_fp8", "dsa_workspace_bytes"} <= set(names)
    L = _lib.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTED)


def test_status_strings():
    L = _lib.lib()
    assert L.dsa_status_string(0) == b"ok"
    assert b"workspace" in L.dsa_status_string(3)
    assert L.dsa_status_string(99) == b"unknown status"


def _queries(num_q, max_nvis):
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: only host-side checks run
    return _lib.QueriesC(num_q, max_nvis, fake.value, fake.value)


def test_workspace_sizes():
    L = _lib.lib()
    q = _queries(64, 131072)
    topk = L.dsa_workspace_bytes(_lib.DSA_OP_TOPK, ctypes.byref(q), 2048)
    assert topk >= 64 * 131072 * 8  # candidate lists of the two-kernel path
    q16 = _queries(16, 131072)
    t16 = L.dsa_workspace_bytes(_lib.DSA_OP_TOPK, ctypes.byref(q16), 2048)
    assert 16 * 2048 * 4 <= t16 < 16 * 131072  # one streaming block per row: histograms only
    fwd = L.dsa_workspace_bytes(_lib.DSA_OP_FORWARD, ctypes.byref(q), 2048)
    assert fwd >= topk + 64 * 131072 * 4  # plus the score rows
    q128 = _queries(128, 131072)  # from 128 rows: streaming again
    assert L.dsa_workspace_bytes(_lib.DSA_OP_TOPK, ctypes.byref(q128), 2048) < 128 * 131072
    q_long = _queries(64, 262144)
    assert L.dsa_workspace_bytes(_lib.DSA_OP_TOPK, ctypes.byref(q_long), 2048) >= 64 * 262144 * 8  # candidate lists
    assert L.dsa_workspace_bytes(_lib.DSA_OP_MLA_PREFILL, ctypes.byref(q), 2048) == 0
    dec16 = L.dsa_workspace_bytes(_lib.DSA_OP_MLA_DECODE, ctypes.byref(q16), 2048)
    assert dec16 >= 16 * 4 * 128 * 512 * 4  # head groups, four row splits of fp32 partials
    q40 = _queries(40, 131072)  # row splits over all heads
    assert L.dsa_workspace_bytes(_lib.DSA_OP_MLA_DECODE, ctypes.byref(q40), 2048) >= 40 * 2 * 128 * 512 * 4
    # 64 queries split heads, not rows: no partials
    assert L.dsa_workspace_bytes(_lib.DSA_OP_MLA_DECODE, ctypes.byref(q), 2048) == 0
    assert L.dsa_workspace_bytes(_lib.DSA_OP_TOPK, ctypes.byref(q), 0) == ctypes.c_size_t(-1).value
    assert L.dsa_workspace_bytes(77, ctypes.byref(q), 16) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("k", [0, -1, 2049])
def test_topk_rejects_bad_k(k):
    L = _lib.lib()
    q = _queries(4, 100)
    p = ctypes.c_void_p(0x1000)
    st = L.dsa_topk(ctypes.byref(q), p, 128, k, p, None, p, 1 << 30, None)
    assert st == _lib.DSA_ERR_INVALID_ARG
    assert b"k =" in L.dsa_last_error()


def test_topk_rejects_small_workspace_and_bad_ld():
    L = _lib.lib()
    q = _queries(4, 10000)
    p = ctypes.c_void_p(0x1000)
    assert L.dsa_topk(ctypes.byref(q), p, 10000, 2048, p, None, p, 16, None) == _lib.DSA_ERR_WORKSPACE
    assert L.dsa_topk(ctypes.byref(q), p, 9999, 2048, p, None, p, 1 << 34, None) == _lib.DSA_ERR_INVALID_ARG
    assert L.dsa_topk(ctypes.byref(q), p, 10002, 2048, p, None, p, 1 << 34, None) == _lib.DSA_ERR_INVALID_ARG


def test_layout_and_alignment_checks():
    L = _lib.lib()
    q = _queries(2, 5000)
    p = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1004)
    bad_block = _lib.KvLayoutC(2, 48, 10, 0, 1000, p.value, None)
    st = L.dsa_indexer_scores(ctypes.byref(q), ctypes.byref(bad_block), p, None, p, p, p, p, 5000, None)
    assert st == _lib.DSA_ERR_UNSUPPORTED
    no_rows = _lib.KvLayoutC(2, 0, 0, 0, 1000, None, None)
    st = L.dsa_indexer_scores(ctypes.byref(q), ctypes.byref(no_rows), p, None, p, p, p, p, 5000, None)
    assert st == _lib.DSA_ERR_INVALID_ARG
    ok_layout = _lib.KvLayoutC(2, 0, 0, 0, 1000, None, p.value)
    st = L.dsa_indexer_scores(ctypes.byref(q), ctypes.byref(ok_layout), odd, None, p, p, p, p, 5000, None)
    assert st == _lib.DSA_ERR_INVALID_ARG
    st = L.dsa_sparse_mla_decode(ctypes.byref(q), ctypes.byref(ok_layout), p, p, p, None, 2048, 0.07, p,
                                 None, None, 0, None)
    assert st == _lib.DSA_ERR_WORKSPACE
    st = L.dsa_quantize_fp8(p, 10, 100, p, p, None)
    assert st == _lib.DSA_ERR_UNSUPPORTED
    st = L.dsa_forward(ctypes.byref(q), ctypes.byref(ok_layout), p, None, None, p, p, p, p, 2048, 0.07, p,
                       None, None, p, 1 << 40, None)
    assert st == _lib.DSA_ERR_INVALID_ARG


def test_empty_batches_are_accepted_without_launching():
    L = _lib.lib()
    q = _lib.QueriesC(0, 0, None, None)
    lay = _lib.KvLayoutC(0, 0, 0, 0, 0, None, None)
    assert L.dsa_indexer_scores(ctypes.byref(q), ctypes.byref(lay), None, None, None, None, None, None, 0,
                                None) == 0
    assert L.dsa_quantize_fp8(None, 0, 128, None, None, None) == 0


def test_kl_and_backward_argument_checks():
    """The indexer-loss and indexer-backward calls validate on the host."""
    L = _lib.lib()
    q = _queries(3, 5000)
    p = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1002)
    lay = _lib.KvLayoutC(1, 0, 0, 0, 5000, None, p.value)
    # sparse KL: idx required, k in [1, 2048], ld_scores >= max_nvis, 16-byte aligned q / kv
    st = L.dsa_indexer_kl_sparse(ctypes.byref(q), ctypes.byref(lay), p, p, None, None, 2048, p, 0.07, p, 5000, p,
                                 None, p, None, None)
    assert st == _lib.DSA_ERR_INVALID_ARG and b"idx" in L.dsa_last_error()
    st = L.dsa_indexer_kl_sparse(ctypes.byref(q), ctypes.byref(lay), p, p, p, None, 4096, p, 0.07, p, 5000, p,
                                 None, p, None, None)
    assert st == _lib.DSA_ERR_INVALID_ARG and b"k =" in L.dsa_last_error()
    st = L.dsa_indexer_kl_sparse(ctypes.byref(q), ctypes.byref(lay), p, p, p, None, 2048, p, 0.07, p, 4999, p,
                                 None, p, None, None)
    assert st == _lib.DSA_ERR_INVALID_ARG and b"ld_scores" in L.dsa_last_error()
    st = L.dsa_indexer_kl_sparse(ctypes.byref(q), ctypes.byref(lay), odd, p, p, None, 2048, p, 0.07, p, 5000, p,
                                 None, p, None, None)
    assert st == _lib.DSA_ERR_INVALID_ARG
    st = L.dsa_indexer_kl_sparse(ctypes.byref(q), ctypes.byref(lay), p, p, p, None, 2048, None, 0.07, p, 5000,
                                 p, None, p, None, None)
    assert st == _lib.DSA_ERR_INVALID_ARG  # lse missing
    # dense KL: ld_grad >= max_nvis
    st = L.dsa_indexer_kl_dense(ctypes.byref(q), ctypes.byref(lay), p, p, p, 0.07, p, 5000, p, None, 4000, p,
                                None, None)
    assert st == _lib.DSA_ERR_INVALID_ARG and b"ld_grad" in L.dsa_last_error()
    # backward: non-null outputs, k checked when idx is given, ld_grad when it is not
    st = L.dsa_indexer_backward(ctypes.byref(q), ctypes.byref(lay), p, None, p, p, p, p, None, 0, p, 0, p, p, p,
                                None)
    assert st == _lib.DSA_ERR_INVALID_ARG and b"k =" in L.dsa_last_error()
    st = L.dsa_indexer_backward(ctypes.byref(q), ctypes.byref(lay), p, None, p, p, p, None, None, 0, p, 100, p, p,
                                p, None)
    assert st == _lib.DSA_ERR_INVALID_ARG and b"ld_grad" in L.dsa_last_error()
    st = L.dsa_indexer_backward(ctypes.byref(q), ctypes.byref(lay), p, None, p, p, p, p, None, 2048, p, 2048, p,
                                p, None, None)
    assert st == _lib.DSA_ERR_INVALID_ARG  # dk missing
    st = L.dsa_indexer_backward(ctypes.byref(q), ctypes.byref(lay), odd, None, p, p, p, p, None, 2048, p, 2048, p,
                                p, p, None)
    assert st == _lib.DSA_ERR_INVALID_ARG  # misaligned q_fp8


def test_kl_and_backward_accept_empty_batches():
    L = _lib.lib()
    q = _lib.QueriesC(0, 0, None, None)
    lay = _lib.KvLayoutC(0, 0, 0, 0, 0, None, None)
    assert L.dsa_indexer_backward(ctypes.byref(q), ctypes.byref(lay), None, None, None, None, None, None, None, 0,
                                  None, 0, None, None, None, None) == 0
    assert L.dsa_indexer_kl_dense(ctypes.byref(q), ctypes.byref(lay), None, None, None, 0.07, None, 0, None, None, 0,
                                  None, None, None) == 0


# --------------------------------------------------------------------------- #
# The Python binding's own checks: row counts of the [num_q, ld] arrays and of
# the block table.  The C layer only sees ld, so a tensor with fewer rows than
# num_q would be indexed past its end on the device; the binding must refuse it
# before any call.  Host tensors stand in for device tensors here (the device
# test is patched out), and every case fails a check before the library is
# called.
# --------------------------------------------------------------------------- #
@pytest.fixture
def host_as_device(monkeypatch):
    import torch
    monkeypatch.setattr(dsa, "_on_device", lambda t: True)
    return torch


def _host_inputs(torch, nq=3, nvis=100, rows=500):
    q = dsa.Queries(torch.zeros(nq, dtype=torch.int32), torch.full((nq,), nvis, dtype=torch.int32), nvis)
    lay = dsa.KvLayout(1, rows, seq_row0=torch.zeros(1, dtype=torch.int64))
    t = dict(
        q8=torch.zeros((nq, 64, 128), dtype=torch.uint8), qs=torch.ones((nq, 64)), w=torch.ones((nq, 64)),
        k8=torch.zeros((rows, 128), dtype=torch.uint8), ks=torch.ones(rows),
        ke=torch.zeros(rows, dtype=torch.uint8), qm=torch.zeros((nq, 128, 576), dtype=torch.bfloat16),
        kv=torch.zeros((rows, 576), dtype=torch.bfloat16), lse=torch.zeros((nq, 128)), kl=torch.zeros(nq),
        idx=torch.zeros((nq, 2048), dtype=torch.int32), dq=torch.zeros((nq, 64, 128)), dw=torch.zeros((nq, 64)),
        dk=torch.zeros((rows, 128)))
    return q, lay, t


def test_binding_rejects_score_rows_short_of_num_q(host_as_device):
    torch = host_as_device
    q, lay, t = _host_inputs(torch)
    short = torch.zeros((2, 128))  # 3 queries
    narrow = torch.zeros((3, 64))  # max_nvis = 100
    for scores, what in ((short, "scores"), (narrow, "scores"), (torch.zeros(3 * 128), "scores")):
        with pytest.raises(ValueError, match=what):
            dsa.dsa_indexer_scores(q, lay, t["q8"], t["qs"], t["w"], t["k8"], t["ks"], scores)
        with pytest.raises(ValueError, match=what):
            dsa.dsa_indexer_scores_e8m0(q, lay, t["q8"], t["qs"], t["w"], t["k8"], t["ke"], scores)
        with pytest.raises(ValueError, match=what):
            dsa.dsa_topk(q, scores, 2048, t["idx"], ws=torch.zeros(1, dtype=torch.uint8))
        with pytest.raises(ValueError, match=what):
            dsa.dsa_indexer_kl_sparse(q, lay, t["qm"], t["kv"], t["idx"], None, 2048, t["lse"], 0.07, scores,
                                      torch.zeros((3, 2048)), t["kl"])
        with pytest.raises(ValueError, match=what):
            dsa.dsa_indexer_kl_dense(q, lay, t["qm"], t["kv"], t["lse"], 0.07, scores, torch.zeros((3, 128)),
                                     t["kl"])


def test_binding_rejects_grad_rows_short_of_num_q(host_as_device):
    torch = host_as_device
    q, lay, t = _host_inputs(torch)
    scores = torch.zeros((3, 128))
    for grad in (torch.zeros((2, 128)), torch.zeros((3, 99)), torch.zeros(384)):
        with pytest.raises(ValueError, match="grad"):
            dsa.dsa_indexer_kl_dense(q, lay, t["qm"], t["kv"], t["lse"], 0.07, scores, grad, t["kl"])
        with pytest.raises(ValueError, match="grad"):
            dsa.dsa_indexer_backward(q, lay, t["q8"], t["qs"], t["w"], t["k8"], t["ks"], None, None, 0, grad,
                                     t["dq"], t["dw"], t["dk"])
    with pytest.raises(ValueError, match="target"):
        dsa.dsa_indexer_kl_dense(q, lay, t["qm"], t["kv"], t["lse"], 0.07, scores, torch.zeros((3, 128)), t["kl"],
                                 target=torch.zeros((2, 128)))


def test_binding_rejects_block_table_rows_short_of_num_seqs(host_as_device):
    torch = host_as_device
    for bt in (torch.zeros((1, 4), dtype=torch.int32), torch.zeros(8, dtype=torch.int32),
               torch.zeros((2, 0), dtype=torch.int32)):
        lay = dsa.KvLayout(2, 256, block_table=bt, block_size=64)
        with pytest.raises(ValueError, match="block_table"):
            lay.c()
    dsa.KvLayout(2, 256, block_table=torch.zeros((2, 4), dtype=torch.int32), block_size=64).c()


def test_noalloc_decode_refuses_partials_beyond_its_scratch():
    """Host-side: 285 queries at k = 2048 need 2 splits of fp32 partials,
    142.8 MiB, more than the library's scratch; refused before any launch."""
    L = _lib.lib()
    q = _queries(285, 4096)
    p = ctypes.c_void_p(0x1000)
    lay = _lib.KvLayoutC(285, 0, 0, 0, 285 * 4096, None, p.value)
    need = L.dsa_workspace_bytes(_lib.DSA_OP_MLA_DECODE, ctypes.byref(q), 2048)
    assert need > _lib.DSA_NOALLOC_SCRATCH_BYTES
    st = L.dsa_sparse_mla_decode_noalloc(ctypes.byref(q), ctypes.byref(lay), p, p, p, None, 2048, 0.07, p, None,
                                         None)
    assert st == _lib.DSA_ERR_UNSUPPORTED and b"scratch" in L.dsa_last_error()
    assert L.dsa_sparse_mla_decode_noalloc(ctypes.byref(q), ctypes.byref(lay), p, p, p, None, 0, 0.07, p, None,
                                           None) == _lib.DSA_ERR_INVALID_ARG
