"""Helpers for the GPU parity tests: build the HIP-path inputs from a workload
(FP8 quantisation on the GPU through dsa_quantize_fp8) and the oracle's inputs
from the same workload (host copies of the generator's fp32 / bf16 values,
quantised by the oracle's own codec).  No oracle input comes from the HIP path
except where a test says so (the top-k set check on the GPU's own scores)."""

import numpy as np
import torch

import oracle
import sparse_long_context_dsa_amd as dsa

SCORE_RTOL = 1e-3      # |I_gpu - I_ref| <= 1e-3 * M_ref, M_ref = sum_j |w_j| ReLU(dot_j)
OUT_MAX_RTOL = 2e-2    # max |O_gpu - O_ref| <= 2e-2 * max |O_ref|   (per query)
OUT_MEAN_RTOL = 5e-3   # mean |O_gpu - O_ref| <= 5e-3 * mean |O_ref| (per query)
LSE_ATOL = 2e-3


def banner(msg):
    print(f"[gpu-test] {msg}", flush=True)


class GpuInputs:
    """Device tensors the library consumes for one workload."""

    def __init__(self, wl):
        self.wl = wl
        dev = wl.q_idx.device
        nq, rows = wl.nq, wl.rows
        self.q8 = torch.empty((nq, 64, 128), dtype=torch.uint8, device=dev)
        self.qs = torch.empty((nq, 64), dtype=torch.float32, device=dev)
        self.k8 = torch.empty((rows, 128), dtype=torch.uint8, device=dev)
        self.ks = torch.empty((rows,), dtype=torch.float32, device=dev)
        dsa.dsa_quantize_fp8(wl.q_idx.view(nq * 64, 128), self.q8.view(nq * 64, 128), self.qs.view(nq * 64))
        dsa.dsa_quantize_fp8(wl.k_idx, self.k8, self.ks)
        self.queries = dsa.Queries(wl.q_seq, wl.q_nvis, wl.max_nvis)
        if wl.block_size:
            self.layout = dsa.KvLayout(wl.num_seqs, rows, block_table=wl.block_table, block_size=wl.block_size)
        else:
            self.layout = dsa.KvLayout(wl.num_seqs, rows, seq_row0=wl.row0)

    def scores(self, ld=None):
        ld = ld or ((self.wl.max_nvis + 63) // 64 * 64 or 64)
        s = torch.full((self.wl.nq, ld), float("nan"), dtype=torch.float32, device=self.q8.device)
        dsa.dsa_indexer_scores(self.queries, self.layout, self.q8, self.qs, self.wl.w, self.k8, self.ks, s)
        return s


def bf16_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class OracleView:
    """Host-side oracle inputs for selected queries of a workload."""

    def __init__(self, wl):
        self.wl = wl
        self.q_seq = wl.q_seq.cpu().numpy()
        self.q_nvis = wl.q_nvis.cpu().numpy()
        self.row0 = wl.row0.cpu().numpy() if wl.row0 is not None else None
        self.bt = wl.block_table.cpu().numpy() if wl.block_table is not None else None

    def rows(self, i, positions=None):
        n = int(self.q_nvis[i])
        pos = np.arange(n) if positions is None else np.asarray(positions)
        return oracle.phys_rows(int(self.q_seq[i]), pos, row0=self.row0, block_table=self.bt,
                                block_size=self.wl.block_size)

    def indexer(self, i, e8m0=False):
        """(I, M) of query i over its whole visible history, float64; with
        e8m0, the keys carry the power-of-two scales of the E8M0 quantiser."""
        wl = self.wl
        q8, qs = oracle.quantize_rows(wl.q_idx[i].cpu().numpy())
        r = self.rows(i)
        keys = wl.k_idx[torch.from_numpy(r).to(wl.k_idx.device)].cpu().numpy() if r.size else np.zeros((0, 128), np.float32)
        if e8m0:
            k8, _, ks = oracle.quantize_rows_e8m0(keys)
        else:
            k8, ks = oracle.quantize_rows(keys)
        return oracle.indexer_scores_query(q8, qs, wl.w[i].cpu().numpy(), k8, ks)

    def mla(self, i, positions):
        wl = self.wl
        r = self.rows(i, positions)
        kv = bf16_bits(wl.kv[torch.from_numpy(r).to(wl.kv.device)]) if r.size else np.zeros((0, 576), np.uint16)
        return oracle.sparse_mla(bf16_bits(wl.q_mla[i]), kv, wl.softmax_scale)


def check_scores(gpu_row, ref, mag, where):
    diff = np.abs(gpu_row.astype(np.float64) - ref)
    bad = diff > SCORE_RTOL * mag + 1e-30
    assert not bad.any(), (f"{where}: {bad.sum()} scores outside 1e-3*M; worst diff {diff.max():.3e}, "
                           f"at M={mag[np.argmax(diff)]:.3e}")
    big = np.abs(ref) >= 0.1 * mag
    rel = (diff[big] / np.abs(ref[big])).max() if big.any() else 0.0
    return float(rel)


def check_out(o_gpu, o_ref, lse_gpu, lse_ref, where):
    d = np.abs(o_gpu.astype(np.float64) - o_ref)
    ref_max = np.abs(o_ref).max()
    ref_mean = np.abs(o_ref).mean()
    assert d.max() <= OUT_MAX_RTOL * ref_max + 1e-30, f"{where}: max err {d.max():.3e} vs max|O| {ref_max:.3e}"
    assert d.mean() <= OUT_MEAN_RTOL * ref_mean + 1e-30, f"{where}: mean err {d.mean():.3e} vs mean|O| {ref_mean:.3e}"
    if lse_gpu is not None:
        fin = np.isfinite(lse_ref)
        assert (np.isfinite(lse_gpu) == fin).all(), f"{where}: lse finiteness differs"
        if fin.any():
            e = np.abs(lse_gpu[fin].astype(np.float64) - lse_ref[fin]).max()
            assert e <= LSE_ATOL, f"{where}: lse err {e:.3e}"
    return float(d.max() / max(ref_max, 1e-30)), float(d.mean() / max(ref_mean, 1e-30))


def check_topk_near_ties(idx_gpu, count, scores_ref, mag, k, where):
    """Against the oracle's own scores: positions chosen by only one side must
    lie within the score tolerance of the k-th largest reference score."""
    ref_idx, ref_count = oracle.topk(scores_ref, k)
    assert count == ref_count, f"{where}: count {count} vs {ref_count}"
    a = set(idx_gpu[:count].tolist())
    b = set(ref_idx[:ref_count].tolist())
    diff = sorted(a ^ b)
    if not diff:
        return 0
    vk = np.sort(scores_ref)[::-1][count - 1]
    kth = int(np.nonzero(scores_ref == vk)[0][0])
    for s in diff:
        tol = 2 * SCORE_RTOL * max(mag[s], mag[kth])
        assert abs(scores_ref[s] - vk) <= tol, f"{where}: position {s} differs but is far from the k-th score"
    return len(diff)


def run_forward(g, k=None):
    wl = g.wl
    k = k or wl.k
    out = torch.full((wl.nq, 128, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((wl.nq, 128), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((wl.nq, k), -7, dtype=torch.int32, device="cuda")
    dsa.dsa_forward(g.queries, g.layout, g.q8, g.qs, wl.w, g.k8, g.ks, wl.q_mla, wl.kv, k, wl.softmax_scale,
                    out, lse, idx)
    torch.cuda.synchronize()
    return out, lse, idx


def check_queries(wl, g, out, lse, idx, queries, k=None, near_ties=True):
    k = k or wl.k
    ov = OracleView(wl)
    nv = wl.q_nvis.cpu().numpy()
    need_scores = any(int(nv[i]) > k for i in queries)
    s = g.scores().cpu().numpy() if need_scores else None
    idx_h, out_h, lse_h = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    for i in queries:
        n = int(nv[i])
        if n <= k:
            want = np.full(k, -1)
            want[:n] = np.arange(n)
            assert (idx_h[i] == want).all(), f"q{i}: short history must select everything"
            count = n
        else:
            ref_idx, count = oracle.topk(s[i, :n], k)
            assert (idx_h[i] == ref_idx).all(), f"q{i}: selection differs from the oracle top-k of GPU scores"
            if near_ties:
                ref_scores, mag = ov.indexer(i)
                check_topk_near_ties(idx_h[i], count, ref_scores, mag, k, f"q{i}")
        o_ref, l_ref = ov.mla(i, idx_h[i, :count])
        check_out(out_h[i], o_ref, lse_h[i], l_ref, f"{wl.name} q{i}")
