"""dsa_sparse_mla_decode_noalloc (the split partials in the library's own
device scratch, no workspace) against dsa_sparse_mla_decode with a workspace:
the same kernels, so the outputs must agree bit for bit.  Two calls in a row on
one GPU, the second smaller (fewer queries, more splits each), so the second
reads none of the first call's leftovers; and one query of each against the
oracle at the usual attention tolerance."""

import numpy as np
import pytest
import torch

import sparse_long_context_dsa_amd as dsa
from gpu_util import OracleView, banner, check_out
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _selection(wl, k, seed):
    rng = np.random.default_rng(seed)
    nv = wl.q_nvis.cpu().numpy()
    idx = np.full((wl.nq, k), -1, np.int32)
    for i in range(wl.nq):
        c = min(k, int(nv[i]))
        idx[i, :c] = np.sort(rng.choice(int(nv[i]), c, replace=False))
    return torch.from_numpy(idx).cuda()


def _both(wl, k, seed):
    q = dsa.Queries(wl.q_seq, wl.q_nvis, wl.max_nvis)
    lay = dsa.KvLayout(wl.num_seqs, wl.rows, seq_row0=wl.row0)
    idx = _selection(wl, k, seed)
    outs = []
    for noalloc in (True, False):
        out = torch.full((wl.nq, 128, 512), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((wl.nq, 128), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            dsa.dsa_sparse_mla_decode_noalloc(q, lay, wl.q_mla, wl.kv, idx, None, k, wl.softmax_scale, out, lse)
        else:
            dsa.dsa_sparse_mla_decode(q, lay, wl.q_mla, wl.kv, idx, None, k, wl.softmax_scale, out, lse)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    return idx.cpu().numpy(), outs


def test_noalloc_matches_workspace_call_twice_second_smaller():
    k = 2048
    ws_need = []
    for nq, seed in ((80, 401), (16, 402)):  # 3 splits (60.1 MiB of partials), then 4 per head group (16.0 MiB)
        banner(f"noalloc decode: {nq} queries x 4096, k={k}")
        wl = make_custom(seq_lens=[4096] * nq, device="cuda", seed=seed)
        q = dsa.Queries(wl.q_seq, wl.q_nvis, wl.max_nvis)
        need = dsa.dsa_workspace_bytes(dsa.DSA_OP_MLA_DECODE, q, k)
        assert 0 < need <= dsa.DSA_NOALLOC_SCRATCH_BYTES
        ws_need.append(need)
        idx, ((o_na, l_na), (o_ws, l_ws)) = _both(wl, k, seed)
        assert (o_na.view(np.uint32) == o_ws.view(np.uint32)).all(), "outputs differ from the workspace call"
        assert (l_na.view(np.uint32) == l_ws.view(np.uint32)).all(), "lse differs from the workspace call"
        ov = OracleView(wl)
        for i in (0, nq - 1):
            o_ref, l_ref = ov.mla(i, idx[i])
            check_out(o_na[i], o_ref, l_na[i], l_ref, f"noalloc q{i}")
    assert ws_need[1] < ws_need[0]


def test_noalloc_head_group_batch_needs_no_scratch():
    """64 queries split their heads instead of their rows: no partials, so the
    entry point uses no scratch, and its outputs equal the workspace call's."""
    k = 2048
    banner("noalloc decode: 64 queries x 4096 (head groups, no partials)")
    wl = make_custom(seq_lens=[4096] * 64, device="cuda", seed=404)
    q = dsa.Queries(wl.q_seq, wl.q_nvis, wl.max_nvis)
    assert dsa.dsa_workspace_bytes(dsa.DSA_OP_MLA_DECODE, q, k) == 0
    idx, ((o_na, l_na), (o_ws, l_ws)) = _both(wl, k, 404)
    assert (o_na.view(np.uint32) == o_ws.view(np.uint32)).all()
    assert (l_na.view(np.uint32) == l_ws.view(np.uint32)).all()
    o_ref, l_ref = OracleView(wl).mla(63, idx[63])
    check_out(o_na[63], o_ref, l_na[63], l_ref, "noalloc head groups q63")


def test_noalloc_rejects_partials_beyond_the_scratch():
    banner("noalloc decode: 285 queries (2 splits, 142.8 MiB) is refused")
    wl = make_custom(seq_lens=[2100] * 285, device="cuda", seed=403)
    q = dsa.Queries(wl.q_seq, wl.q_nvis, wl.max_nvis)
    lay = dsa.KvLayout(wl.num_seqs, wl.rows, seq_row0=wl.row0)
    assert dsa.dsa_workspace_bytes(dsa.DSA_OP_MLA_DECODE, q, 2048) > dsa.DSA_NOALLOC_SCRATCH_BYTES
    idx = torch.zeros((wl.nq, 2048), dtype=torch.int32, device="cuda")
    out = torch.full((wl.nq, 128, 512), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(dsa.DsaError, match="scratch"):
        dsa.dsa_sparse_mla_decode_noalloc(q, lay, wl.q_mla, wl.kv, idx, None, 2048, wl.softmax_scale, out)
    torch.cuda.synchronize()
    assert (out == 7.0).all()  # nothing was launched
